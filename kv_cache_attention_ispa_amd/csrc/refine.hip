// Refinement residual of the ridge absorption on the int8 matrix cores (gfx950).
//
// The closed form of the technical summary (gist.science, nl/pt), section 2, stage 2 "Layer
// Absorb", dW = (G + lambda I)^-1 C W, is solved in fp32; with an ill-conditioned G (the 14B layer:
// 4680 tokens for 5120 features) one step of iterative refinement brings dW to the accuracy of an
// fp64 solve.  That step needs the residual
//     r = C W - (G + lambda I) dW
// to far more than fp32 accuracy, since its two terms cancel.  It is formed here as one product
//     r = A B - lambda dW,   A = [C | -G]  (d x 2d),   B = [W ; dW]  (2d x d),
// exactly in integer arithmetic up to a truncation of the operands (the splitting scheme of Ozaki
// et al. for accurate matrix products, with fixed-point slices):
//   * row i of A is scaled by 2^-e_i (e_i: the smallest exponent with max_k |A_ik| < 2^e_i) and
//     written as S = 5 signed 7-bit digits: A_ik = 2^e_i sum_a A_a[i][k] 2^-7a + (|rest| < 2^(e_i-35));
//     column j of B likewise with f_j.  The digits are exact in fp64 (each is the truncation of an
//     exactly scaled value);
//   * sum_k A_ik B_kj = 2^(e_i + f_j) sum_{a,b} 2^-7(a+b) sum_k A_a[i][k] B_b[k][j]; the pairs with
//     a + b <= S + 1 (15 of them) are kept.  Each pair is an int8 product with exact int32 sums
//     (|sum| < 2d 127^2 < 2^31 for d < 66,000), added to an fp64 accumulator with its power of two;
//   * so r carries about 35 correct bits relative to max|A_i.| max|B_.j| (fp32: 24), and the
//     15 int8 products cost about a quarter of the two fp64 products they replace.
// Digits are stored k-contiguous for both operands (A_a [d][Kp], B_b transposed [d][Kp], Kp = 2d
// rounded up to 128 with zero padding), so the product is A_a B_b^T with 16-byte row pieces on
// both sides, as in the projection kernel.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int OZ_S = 5;                          // digits per value
constexpr int OZ_PAIRS = OZ_S * (OZ_S + 1) / 2;  // pairs (a, b) with a + b <= S + 1
constexpr int OZ_T = 256;

template <typename P>
__device__ __forceinline__ P* oz_layer(P* p, int64_t step) {
  return (P*)((char*)p + (int64_t)blockIdx.y * step);
}

// exponent e with |x| < 2^e for every |x| <= m (0 for m = 0): frexp's exponent
__device__ __forceinline__ int oz_exp(float m) {
  int e = 0;
  if (m > 0.f) frexpf(m, &e);
  return e;
}

// the S digits of x 2^-e (|x| < 2^e), most significant first
__device__ __forceinline__ void oz_digits(float x, int e, int8_t (&dg)[OZ_S]) {
  double s = ldexp((double)x, -e);   // |s| < 1, exact
#pragma unroll
  for (int a = 0; a < OZ_S; ++a) {
    const double y = s * 128.0;      // exact
    const double t = trunc(y);       // |t| <= 127
    dg[a] = (int8_t)(int)t;
    s = y - t;                       // exact, |s| < 1
  }
}

// ---- A = [C | -G]: one work-group per row; pass 1 the row maximum, pass 2 the digits, four
// consecutive k per thread (one 32-bit store per digit plane).
__global__ __launch_bounds__(OZ_T) void oz_rows_kernel(const float* C, const float* G, int d, int kp, int64_t s_mat,
                                                       int8_t* A, int* ea, int64_t s_ws) {
  C = oz_layer(C, s_mat);
  G = oz_layer(G, s_mat);
  A = oz_layer(A, s_ws);
  ea = oz_layer(ea, s_ws);
  const int i = blockIdx.x, t = threadIdx.x;
  const float* c = C + (int64_t)i * d;
  const float* g = G + (int64_t)i * d;
  float m = 0.f;
  for (int k = 4 * t; k < d; k += 4 * OZ_T) {
    const f32x4 u = *(const f32x4*)(c + k), v = *(const f32x4*)(g + k);
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(u[q]), fabsf(v[q])));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __shared__ float wm[OZ_T / 64];
  if ((t & 63) == 0) wm[t >> 6] = m;
  __syncthreads();
  m = wm[0];
#pragma unroll
  for (int w = 1; w < OZ_T / 64; ++w) m = fmaxf(m, wm[w]);
  const int e = oz_exp(m);
  if (t == 0) ea[i] = e;
  const int64_t plane = (int64_t)d * kp;
  int8_t* row = A + (int64_t)i * kp;
  for (int k = 4 * t; k < kp; k += 4 * OZ_T) {
    uint32_t w[OZ_S] = {};
    if (k < 2 * d) {   // 2d is a multiple of 64: a quad is all C, all G or all padding
      const f32x4 u = k < d ? *(const f32x4*)(c + k) : *(const f32x4*)(g + k - d);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int8_t dg[OZ_S];
        oz_digits(k < d ? u[q] : -u[q], e, dg);
#pragma unroll
        for (int a = 0; a < OZ_S; ++a) w[a] |= (uint32_t)(uint8_t)dg[a] << (8 * q);
      }
    }
#pragma unroll
    for (int a = 0; a < OZ_S; ++a) *(uint32_t*)(row + a * plane + k) = w[a];
  }
}

// ---- B = [W ; dW], column j -> row j of B^T.  Work-group (jb, ks): columns 64 jb .. +63 (those
// below d: d is a multiple of 32), rows k of part ks of [0, 2d) (OZ_KSPLIT parts).
constexpr int OZ_KSPLIT = 8;
template <typename T> __device__ __forceinline__ float oz_w(const void* W, int64_t e) {
  if constexpr (std::is_same<T, F32>::value) return ((const float*)W)[e];
  else return Cvt<T>::to_f(((const uint16_t*)W)[e]);
}

// pass 1: partial column maxima mx[ks][j]
template <typename T>
__global__ __launch_bounds__(OZ_T) void oz_colmax_kernel(const void* W, const float* dW, int d, int64_t s_wmat,
                                                         int64_t s_mat, float* mx, int64_t s_ws) {
  W = oz_layer(W, s_wmat);
  dW = oz_layer(dW, s_mat);
  mx = oz_layer(mx, s_ws);
  const int jb = blockIdx.x, ks = blockIdx.z, t = threadIdx.x, j = 64 * jb + (t & 63);
  const int k0 = (int)((int64_t)2 * d * ks / OZ_KSPLIT), k1 = (int)((int64_t)2 * d * (ks + 1) / OZ_KSPLIT);
  float m = 0.f;
  if (j < d)
    for (int k = k0 + (t >> 6); k < k1; k += OZ_T / 64)
      m = fmaxf(m, fabsf(k < d ? oz_w<T>(W, (int64_t)k * d + j) : dW[(int64_t)(k - d) * d + j]));
  __shared__ float red[OZ_T / 64][64];
  red[t >> 6][t & 63] = m;
  __syncthreads();
  if (t < 64 && j < d) {
#pragma unroll
    for (int w = 1; w < OZ_T / 64; ++w) m = fmaxf(m, red[w][t]);
    mx[(int64_t)ks * d + j] = m;
  }
}

// pass 2: digits of 64 columns x (2d / OZ_KSPLIT) rows, transposed through LDS in 64 x 64 blocks
template <typename T>
__global__ __launch_bounds__(OZ_T) void oz_cols_kernel(const void* W, const float* dW, int d, int kp, int64_t s_wmat,
                                                       int64_t s_mat, const float* mx, int8_t* Bt, int* eb,
                                                       int64_t s_ws) {
  W = oz_layer(W, s_wmat);
  dW = oz_layer(dW, s_mat);
  mx = oz_layer(mx, s_ws);
  Bt = oz_layer(Bt, s_ws);
  eb = oz_layer(eb, s_ws);
  const int jb = blockIdx.x, ks = blockIdx.z, t = threadIdx.x;
  __shared__ int ex[64];
  __shared__ uint32_t tile[OZ_S][64][17];   // [plane][column][4 rows per word], padded
  if (t < 64) {
    float m = 0.f;
    if (64 * jb + t < d)
      for (int q = 0; q < OZ_KSPLIT; ++q) m = fmaxf(m, mx[(int64_t)q * d + 64 * jb + t]);
    ex[t] = oz_exp(m);
    if (ks == 0 && 64 * jb + t < d) eb[64 * jb + t] = ex[t];
  }
  __syncthreads();
  const int64_t plane = (int64_t)d * kp;
  // rows [k0, k1) of part ks; the padding [2d, kp) is written by the last part
  const int k0 = (int)((int64_t)2 * d * ks / OZ_KSPLIT) / 64 * 64;
  const int k1 = ks + 1 == OZ_KSPLIT ? kp : (int)((int64_t)2 * d * (ks + 1) / OZ_KSPLIT) / 64 * 64;
  const int c = t & 63, rq = t >> 6;   // column c, row quad rq + 4 u (u = 0..3) of the 64-row block
  const bool cin = 64 * jb + c < d;
  for (int kb = k0; kb < k1; kb += 64) {
    // thread (rq, c) reads rows kb + 4 (rq + 4 u) .. +3 of column c (coalesced across c)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r4 = rq + 4 * u;
      uint32_t w[OZ_S] = {};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kb + 4 * r4 + q;
        if (cin && k < 2 * d) {
          const float x = k < d ? oz_w<T>(W, (int64_t)k * d + 64 * jb + c) : dW[(int64_t)(k - d) * d + 64 * jb + c];
          int8_t dg[OZ_S];
          oz_digits(x, ex[c], dg);
#pragma unroll
          for (int a = 0; a < OZ_S; ++a) w[a] |= (uint32_t)(uint8_t)dg[a] << (8 * q);
        }
      }
#pragma unroll
      for (int a = 0; a < OZ_S; ++a) tile[a][c][r4] = w[a];
    }
    __syncthreads();
    // row 64 jb + c' of B^T, k = kb .. kb + 63: 16 words per plane; thread t writes 4 words of one
    // (plane, column) pair
    for (int p = t; p < OZ_S * 64 * 4; p += OZ_T) {
      const int a = p / 256, cc = (p >> 2) & 63, part = p & 3;
      if (64 * jb + cc >= d) continue;
      const u32x4 v = {tile[a][cc][4 * part], tile[a][cc][4 * part + 1], tile[a][cc][4 * part + 2],
                       tile[a][cc][4 * part + 3]};
      *(u32x4*)(Bt + a * plane + (int64_t)(64 * jb + cc) * kp + kb + 16 * part) = v;
    }
    __syncthreads();
  }
}

// ---- r = 2^(e_i + f_j) sum_pairs 2^-7(a+b) (A_a B_b^T)_ij - lambda dW_ij.
// 128 x 128 output tiles; work-groups of 6 waves: waves 0-3 multiply (2 x 2 of 64 x 64, 2 x 2 blocks
// of 32 x 32 each, v_mfma_i32_32x32x32_i8), waves 4-5 only issue loads.  The 15 pairs form one
// sequence of 128-byte stages (n_st per pair) through a three-deep LDS ring of direct-to-LDS loads
// issued two stages ahead; one barrier per stage.  After a pair's last stage the int32 sums are
// added to the fp64 accumulators with the pair's power of two and cleared.
// LDS: 16-byte chunk c of row r at r * 128 + 16 (c ^ ((r / 2) % 8)) (as the projection kernel).
constexpr int OZ_BK = 128;                 // bytes (k values) of a row per stage
constexpr int OZ_TILE = 128 * OZ_BK;       // 16 KiB per operand and stage
constexpr uint32_t OZ_OUT = 0xFFFFFFF0u;   // an offset past every buffer below: loads return 0
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef double f64x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int oz_off(int row, int chunk) { return row * OZ_BK + ((chunk ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ void oz_pair(int p, int& a, int& b) {   // pairs ordered by a + b, then a
  int t = 2;
  while (p >= t - 1) { p -= t - 1; ++t; }
  a = 1 + p;
  b = t - a;
}

__global__ __launch_bounds__(384, 1) void oz_gemm_kernel(const int8_t* A, const int* ea, const int8_t* Bt,
                                                         const int* eb, const float* dW, const float* lam, int d,
                                                         int kp, int tiles, int64_t s_ws, int64_t s_mat, int64_t s_lam,
                                                         float* r) {
  A = oz_layer(A, s_ws);
  Bt = oz_layer(Bt, s_ws);
  ea = oz_layer(ea, s_ws);
  eb = oz_layer(eb, s_ws);
  dW = oz_layer(dW, s_mat);
  lam = oz_layer(lam, s_lam);
  r = oz_layer(r, s_ws);
  __shared__ __attribute__((aligned(16))) uint8_t a0[OZ_TILE], a1[OZ_TILE], a2[OZ_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t b0[OZ_TILE], b1[OZ_TILE], b2[OZ_TILE];
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bm = logical / tiles, bn = logical % tiles;
  const int m0 = bm * 128, n0 = bn * 128;
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto aslot = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return a0;
    else if constexpr (j == 1) return a1;
    else return a2;
  };
  auto bslot = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return b0;
    else if constexpr (j == 1) return b1;
    else return b2;
  };
  auto barrier = [&]() { lds_barrier(); };
  const int n_st = kp / OZ_BK;
  const int n_all = OZ_PAIRS * n_st;   // stages of all pairs

  if (wave >= 4) {
    // loader w issues A instructions 8 w .. 8 w + 7 and B instructions 8 w .. 8 w + 7 of a stage;
    // instruction i covers tile rows 8 i .. 8 i + 7: lane l -> row 8 i + l / 8, physical chunk l % 8,
    // logical chunk (l % 8) ^ (4 (i % 2) + l / 16)
    const int w = wave - 4;
    const int64_t plane = (int64_t)d * kp;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)0xFFFFFFF0u, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)Bt, (short)0, (int)0xFFFFFFF0u, 0x00020000);
    uint32_t aoff[8], boff[8];
    bool ain[8], bin[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 8 * w + j, row = 8 * i + (lane >> 3), c = (lane & 7) ^ (4 * (i & 1) + (lane >> 4));
      ain[j] = m0 + row < d;
      bin[j] = n0 + row < d;
      aoff[j] = (uint32_t)((int64_t)(m0 + row) * kp) + 16u * c;
      boff[j] = (uint32_t)((int64_t)(n0 + row) * kp) + 16u * c;
    }
    auto issue = [&](uint8_t* as, uint8_t* bs, int g) {
      const bool ok = g < n_all;
      int pa = 0, pb = 0, s = 0;
      if (ok) {
        const int p = g / n_st;
        s = g - p * n_st;
        oz_pair(p, pa, pb);
      }
      const uint32_t abase = (uint32_t)((pa - 1) * plane) + (uint32_t)s * OZ_BK;
      const uint32_t bbase = (uint32_t)((pb - 1) * plane) + (uint32_t)s * OZ_BK;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(as + 1024 * (8 * w + j)), 16,
                                                 ok && ain[j] ? abase + aoff[j] : OZ_OUT, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(bs + 1024 * (8 * w + j)), 16,
                                                 ok && bin[j] ? bbase + boff[j] : OZ_OUT, 0, 0, 0);
      }
    };
    issue(a0, b0, 0);
    issue(a1, b1, 1);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
    barrier();
    auto lstep = [&](auto J, int g) {   // between barriers g and g + 1 (J = g % 3)
      constexpr int j = decltype(J)::value;
      issue(aslot(std::integral_constant<int, (j + 2) % 3>{}), bslot(std::integral_constant<int, (j + 2) % 3>{}), g + 2);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
      barrier();
    };
    for (int g = 0; g < n_all; g += 3) {
      lstep(std::integral_constant<int, 0>{}, g);
      lstep(std::integral_constant<int, 1>{}, g + 1);
      lstep(std::integral_constant<int, 2>{}, g + 2);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // loads past the last stage (zeros) have landed
    barrier();                                   // the ring is idle
    return;
  }

  const int wm = wave >> 1, wn = wave & 1;
  i32x16 acc[2][2];
  f64x16 sum[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        acc[mi][ni][q] = 0;
        sum[mi][ni][q] = 0.0;
      }
  // fragment rows 64 wm + 32 mi + l % 32 (A) and 64 wn + 32 ni + l % 32 (B^T), chunk 2 kk + l / 32 of
  // k-step kk (k = 32 kk + 16 (l / 32) .. + 15); the swizzle depends on the row only through bits
  // 1-3, the same for r and r + 32, and chunk 2 kk + h = h ^ 2 kk
  const int aoff = oz_off(64 * wm + (lane & 31), hi);
  const int boff = oz_off(64 * wn + (lane & 31), hi);
  barrier();
  auto mstep = [&](auto J, int g) {   // between barriers g and g + 1 (J = g % 3)
    const uint8_t* as = aslot(J);
    const uint8_t* bs = bslot(J);
    i32x4 af[2][2], bf[2][2];
    auto frags = [&](int kk, i32x4* fa, i32x4* fb) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) fa[mi] = *(const i32x4*)(as + ((aoff ^ (kk << 5)) + 32 * mi * OZ_BK));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) fb[ni] = *(const i32x4*)(bs + ((boff ^ (kk << 5)) + 32 * ni * OZ_BK));
    };
    frags(0, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < OZ_BK / 32; ++kk) {
      if (kk + 1 < OZ_BK / 32) frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni], 0, 0, 0);
    }
    // the pair ends with this stage: its exact sums join the fp64 accumulators
    if (g < n_all && (g + 1) % n_st == 0) {
      int pa, pb;
      oz_pair(g / n_st, pa, pb);
      const double sc = ldexp(1.0, -7 * (pa + pb));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            sum[mi][ni][q] = fma((double)acc[mi][ni][q], sc, sum[mi][ni][q]);
            acc[mi][ni][q] = 0;
          }
    }
    barrier();
  };
  // whole ring turns: stages past the last one hold zeros and add nothing
  for (int g = 0; g < n_all; g += 3) {
    mstep(std::integral_constant<int, 0>{}, g);
    mstep(std::integral_constant<int, 1>{}, g + 1);
    mstep(std::integral_constant<int, 2>{}, g + 2);
  }
  barrier();   // the ring is idle
  const double lm = (double)*lam;
  // register q of lane l of block (mi, ni): row 64 wm + 32 mi + 8 (q / 4) + 4 (l / 32) + q % 4,
  // column 64 wn + 32 ni + l % 32
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int col = n0 + 64 * wn + 32 * ni + (lane & 31);
    if (col >= d) continue;
    const int fj = eb[col];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + 64 * wm + 32 * mi + 8 * (q >> 2) + 4 * hi + (q & 3);
        if (row < d) {
          const int64_t e = (int64_t)row * d + col;
          r[e] = (float)(ldexp(sum[mi][ni][q], ea[row] + fj) - lm * (double)dW[e]);
        }
      }
  }
}

}  // namespace

size_t residual_kp(int d) { return (size_t)((2 * d + OZ_BK - 1) / OZ_BK * OZ_BK); }

size_t residual_workspace_bytes(int d) {
  const size_t planes = (size_t)OZ_S * d * residual_kp(d);   // digits of one operand
  return (2 * planes + (size_t)(2 + OZ_KSPLIT) * d * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_residual(const ResidualLaunch& L, hipStream_t s) {
  const int d = L.d;
  const int kp = (int)residual_kp(d);
  const size_t planes = (size_t)OZ_S * d * kp;
  int8_t* A = (int8_t*)L.ws;
  int8_t* Bt = A + planes;
  int* ea = (int*)(Bt + planes);
  int* eb = ea + d;
  float* mx = (float*)(eb + d);
  if (L.rows_too) {
    hipLaunchKernelGGL(oz_rows_kernel, dim3(d, L.batch), dim3(OZ_T), 0, s, L.C, L.G, d, kp, L.s_mat, A, ea, L.s_ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 cg((d + 63) / 64, L.batch, OZ_KSPLIT);
  if (L.w_dtype == DT_BF16) {
    hipLaunchKernelGGL(oz_colmax_kernel<BF16>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, L.s_wmat, L.s_mat, mx, L.s_ws);
    hipLaunchKernelGGL(oz_cols_kernel<BF16>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, kp, L.s_wmat, L.s_mat, mx, Bt, eb,
                       L.s_ws);
  } else if (L.w_dtype == DT_F16) {
    hipLaunchKernelGGL(oz_colmax_kernel<F16>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, L.s_wmat, L.s_mat, mx, L.s_ws);
    hipLaunchKernelGGL(oz_cols_kernel<F16>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, kp, L.s_wmat, L.s_mat, mx, Bt, eb,
                       L.s_ws);
  } else {
    hipLaunchKernelGGL(oz_colmax_kernel<F32>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, L.s_wmat, L.s_mat, mx, L.s_ws);
    hipLaunchKernelGGL(oz_cols_kernel<F32>, cg, dim3(OZ_T), 0, s, L.W, L.dW, d, kp, L.s_wmat, L.s_mat, mx, Bt, eb,
                       L.s_ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = (d + 127) / 128;
  hipLaunchKernelGGL(oz_gemm_kernel, dim3(tiles * tiles, L.batch), dim3(384), 0, s, A, ea, Bt, eb, L.dW, L.lambda, d,
                     kp, tiles, L.s_ws, L.s_mat, L.s_lambda, L.r);
  return hipGetLastError();
}

}  // namespace ispa
