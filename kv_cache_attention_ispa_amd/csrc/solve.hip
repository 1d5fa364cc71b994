// Closed-form ridge absorption for gfx950.
//
// ISPA technical summary (gist.science, nl/pt), section 2, stage 2 "Layer
// Absorb": the weight modulation minimising ||A_loc (W + dW) - A_full W||^2 +
// lambda ||dW||^2 is dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W,
// computed once, without iteration.  With G = A_loc^T A_loc and C = A_loc^T dA:
//
//   R = C W;   G + lambda I = L L^T (blocked right-looking Cholesky, fp32);
//   the sweep also carries the identity, which leaves L^-1 when it ends; then
//   Z = L^-1 R and dW = (L^-1)^T Z are two triangular GEMMs.
//   Optional iterative refinement (a given number of steps): r = C W - (G + lambda I) dW
//   accumulated in fp64 (C W formed once in fp64), then dW += (L^-1)^T (L^-1 r).
//
// "Dynamic layer selection" ranks layers by the reconstruction error epsilon;
// it is evaluated here from the statistics alone (D = dA^T dA, P = W W^T):
//   ||A_loc dW - dA W||^2 = <D, P> - <dW, R> - lambda ||dW||^2   (at the optimum)
//   ||A_full W||^2        = <G, P> + 2 <W, R> + <D, P>.
//
// Every step is a HIP kernel enqueued on the caller's stream; the host never
// waits.  A non-positive pivot sets *info to its 1-based index.
#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int NB = 64;          // Cholesky panel width
constexpr int NT = 256;

// ------------------------------------------------------------------------------------------
// Triangular fp32 GEMM on MFMA (32x32x2): C = alpha * op(A) B + beta * C for d x d row-major
// matrices, op(A) = A lower triangular (TA = false: only k < m0 + 64 contributes to a row block at
// m0) or op(A) = A^T with A lower triangular (TA = true: only k >= m0).  64 x 64 output tiles, 4
// waves of 32 x 32; k streams through a 4-deep LDS ring of 32-wide stages filled by direct-to-LDS
// buffer loads issued three stages ahead; two work-groups per CU.  Tiles are dispatched longest
// k range first.
// A stage holds op(A) rows m0 .. m0+63 x k0 .. k0+31 and B rows k0 .. k0+31 x n0 .. n0+63.
//   TA = false: A[m][k] rows of 128 bytes, 16-byte chunk c of row m at 16 (c ^ (m % 8)); the MFMA
//     k order is permuted so one 16-byte read of A[m][4c .. 4c+3] feeds four MFMAs (the k index of
//     A and B only has to agree within the sum).
//   TA = true: A[k][m] rows of 256 bytes (the stage is a row slice of A itself).
//   B: B[k][n] rows of 256 bytes.
// ------------------------------------------------------------------------------------------
constexpr int TG_TILE = 64, TG_K = 32, TG_RING = 4;
constexpr int TG_STAGE = TG_TILE * TG_K * 4;   // bytes of one operand stage (8 KiB)

struct TrGemm {
  const float* A;
  const float* B;
  float* C;
  int d, tiles;   // tiles per dimension
  float alpha, beta;
  const void* W;  // optional fold: Wn = W + C (final value), in dtype wdt
  void* Wn;
  int wdt;
};

// Wn[e] = W[e] + v, rounded to nearest in W's dtype
__device__ __forceinline__ void fold_store(const TrGemm& g, int64_t e, float v) {
  if (g.wdt == DT_BF16)
    ((uint16_t*)g.Wn)[e] = Cvt<BF16>::from_f(Cvt<BF16>::to_f(((const uint16_t*)g.W)[e]) + v);
  else if (g.wdt == DT_F16)
    ((uint16_t*)g.Wn)[e] = Cvt<F16>::from_f(Cvt<F16>::to_f(((const uint16_t*)g.W)[e]) + v);
  else
    ((float*)g.Wn)[e] = ((const float*)g.W)[e] + v;
}

template <bool TA>
__global__ __launch_bounds__(NT, 2) void trgemm_kernel(TrGemm g) {
  __shared__ __attribute__((aligned(16))) char a0[TG_STAGE], a1[TG_STAGE], a2[TG_STAGE], a3[TG_STAGE];
  __shared__ __attribute__((aligned(16))) char b0[TG_STAGE], b1[TG_STAGE], b2[TG_STAGE], b3[TG_STAGE];
  const int T = g.tiles, d = g.d;
  const int q = blockIdx.x;
  const int bm = TA ? q / T : (T - 1) - q / T, bn = q % T;   // longest k range first
  const int m0 = bm * TG_TILE, n0 = bn * TG_TILE;
  const int k_begin = TA ? m0 : 0, k_end = TA ? d : min(d, m0 + TG_TILE);
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // raw buffers over A and B (reads past the end return zeros)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, (int)((int64_t)d * d * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, (short)0, (int)((int64_t)d * d * 4), 0x00020000);
  // Wave w issues A instructions 2w, 2w + 1 and B instructions 2w, 2w + 1 of a stage (8 each, 1 KiB).
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 2 * wave + j;
    if (TA) {   // A rows k: 4 rows x 256 bytes per instruction, lane -> row i*4 + l/16, chunk l%16
      aoff[j] = (uint32_t)(((4 * i + (lane >> 4)) * d + m0 + 4 * (lane & 15)) * 4);
    } else {    // A rows m: 8 rows x 128 bytes, lane -> row 8i + l/8, physical chunk l%8 = logical ^ (row % 8)
      const int row = 8 * i + (lane >> 3), c = (lane & 7) ^ (row & 7);
      aoff[j] = (uint32_t)(((m0 + row) * d + 4 * c) * 4);
    }
    boff[j] = (uint32_t)(((4 * i + (lane >> 4)) * d + n0 + 4 * (lane & 15)) * 4);
  }
  const int n_st = (k_end - k_begin + TG_K - 1) / TG_K;
  auto issue = [&](char* as, char* bs, int st) {
    const int k0 = k_begin + st * TG_K;
    const bool ok = k0 < k_end;
    // A: TA moves down rows (k0 rows of d floats), else along the row (k0 floats)
    const uint32_t ask = TA ? (uint32_t)k0 * d * 4 : (uint32_t)k0 * 4;
    const uint32_t bsk = (uint32_t)k0 * d * 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(as + 1024 * (2 * wave + j)), 16,
                                               ok ? aoff[j] + ask : 0x80000000u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(bs + 1024 * (2 * wave + j)), 16,
                                               ok ? boff[j] + bsk : 0x80000000u, 0, 0, 0);
    }
  };
  auto aslot = [&](auto J) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return a0;
    else if constexpr (j == 1) return a1;
    else if constexpr (j == 2) return a2;
    else return a3;
  };
  auto bslot = [&](auto J) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return b0;
    else if constexpr (j == 1) return b1;
    else if constexpr (j == 2) return b2;
    else return b3;
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int am = 32 * wm + l32, bnn = 32 * wn + l32;
  issue(a0, b0, 0);
  issue(a1, b1, 1);
  issue(a2, b2, 2);
  // Stage s (slot J = s % 4): wait for its loads, barrier, refill slot (s - 1) % 4 with stage s + 3,
  // then 16 MFMAs.  Sub-stage u (k0 + 8u .. + 7): lane half h takes k = k0 + 8u + 4h + v, v = 0..3.
  auto step = [&](auto J, int s) {
    constexpr int j = decltype(J)::value;
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(8));
    barrier();
    issue(aslot(std::integral_constant<int, (j + 3) % 4>{}), bslot(std::integral_constant<int, (j + 3) % 4>{}), s + 3);
    const char* as = aslot(J);
    const char* bs = bslot(J);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float av[4];
      if (TA) {
#pragma unroll
        for (int v = 0; v < 4; ++v) av[v] = *(const float*)(as + (8 * u + 4 * hi + v) * 256 + 4 * am);
      } else {
        const int c = 2 * u + hi;
        const f32x4 x = *(const f32x4*)(as + am * 128 + 16 * (c ^ (am & 7)));
        av[0] = x[0]; av[1] = x[1]; av[2] = x[2]; av[3] = x[3];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float bv = *(const float*)(bs + (8 * u + 4 * hi + v) * 256 + 4 * bnn);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[v], bv, acc, 0, 0, 0);
      }
    }
  };
  for (int s = 0; s < n_st; s += TG_RING) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    step(std::integral_constant<int, 2>{}, s + 2);
    step(std::integral_constant<int, 3>{}, s + 3);
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // loads past the last stage (zeros) have landed
  const int col = n0 + 32 * wn + l32;
  if (col >= d) return;
  const int64_t e0 = (int64_t)(m0 + 32 * wm + 4 * hi) * d + col;
  float* cb = g.C + e0;
  const int rows = d - (m0 + 32 * wm + 4 * hi);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + (r & 3);
    if (row < rows) {
      const float v = g.beta == 0.f ? g.alpha * acc[r] : fmaf(g.alpha, acc[r], g.beta * cb[(int64_t)row * d]);
      cb[(int64_t)row * d] = v;
      if (g.Wn) fold_store(g, e0 + (int64_t)row * d, v);
    }
  }
}

// C = alpha op(L) B + beta C with L = A lower triangular (op = identity or transpose)
hipError_t run_trgemm(bool transA, const float* A, const float* B, float* C, int d, float alpha, float beta,
                      hipStream_t s, const void* W = nullptr, void* Wn = nullptr, int wdt = 0) {
  TrGemm g;
  g.W = W; g.Wn = Wn; g.wdt = wdt;
  g.A = A; g.B = B; g.C = C;
  g.d = d;
  g.tiles = (d + TG_TILE - 1) / TG_TILE;
  g.alpha = alpha; g.beta = beta;
  const dim3 grid(g.tiles * g.tiles);
  if (transA) hipLaunchKernelGGL(trgemm_kernel<true>, grid, dim3(NT), 0, s, g);
  else hipLaunchKernelGGL(trgemm_kernel<false>, grid, dim3(NT), 0, s, g);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Small kernels
// ------------------------------------------------------------------------------------------
struct Scalars {
  float lambda;
  int pad;
  double dots[8];
};

// Mx = G (lambda joins the diagonal blocks as the sweep factors them); Bx = I (becomes L^-1);
// Wf = W as fp32.
template <typename WT>
__global__ __launch_bounds__(NT) void setup_kernel(const float* G, const typename WT::storage* W, int d, float* Mx,
                                                   float* Bx, float* Wf) {
  const int64_t n = (int64_t)d * d;
  for (int64_t e = blockIdx.x * (int64_t)NT + threadIdx.x; e < n; e += (int64_t)gridDim.x * NT) {
    const int i = (int)(e / d), j = (int)(e % d);
    Mx[e] = G[e];
    Bx[e] = (i == j) ? 1.f : 0.f;
    Wf[e] = Cvt<WT>::to_f(W[e]);
  }
}

// ------------------------------------------------------------------------------------------
// Cholesky sweep, one launch per panel (64-wide block columns, nP of them).  With T_k = L_kk^-1:
//   L_ik = A_ik T_k^T for the blocks below the diagonal, so the trailing update of panel k is
//   A_ij -= X_i X_j^T with X_i = A_ik T_k^T, and the identity part (which becomes L^-1) is
//   B_ic -= X_i (T_k B_kc) for the blocks below, while its block row k ends as T_k B_kc.
// Launch k runs, side by side:
//   * the factorization of diagonal block k (work-group 0): D = A_kk - X_k X_k^T (panel k-1's
//     update of that block), D = L_kk L_kk^T, T_k = L_kk^-1  -> T slot k % 3;
//   * panel k-1's trailing update of every other lower block of A and of the identity part;
//   * the final product T_{k-2} B_{k-2,c} of block row k-2 (no launch reads that row any more).
// The factors L are never needed again: the solve uses L^-1 only.  Launch nP finishes block rows
// nP-2 and nP-1.  Every work-group has 1024 threads (16 waves); the 64 x 64 x 64 products run on
// MFMA 16x16x4 (fp32), one 16 x 16 quadrant per wave.
// ------------------------------------------------------------------------------------------
constexpr int SW_THREADS = 1024;
constexpr int BP = NB + 4;   // LDS pitch of a 64 x 64 block: 16 rows of a wave hit 16 distinct 4-bank groups

struct SweepArgs {
  float* Mx;   // d x d, G + lambda I, lower blocks updated in place
  float* Bx;   // d x d, identity part, becomes L^-1
  float* Tb;   // three 64 x 64 slots: T_k in slot k % 3
  int* info;
  int d, nP, k;
  int n_a, n_i, f_row0, f_rows;   // work items: A blocks, identity blocks, final rows [f_row0, +f_rows)
  // products that do not depend on the sweep ride along in its launches, one K range at a time:
  // R = C W (always) and P = W W^T (for epsilon); this launch computes output blocks
  // [fill0, fill0 + n_fill) of K range [kb0, kb1) (in 64-blocks), added to earlier ranges when kb0 > 0
  const float* C;
  const float* Wf;
  float* R;
  float* P;
  int n_fill, fill0, kb0, kb1;
  // lambda (absolute, or lam * tr(G) / d): set by the first launch's diagonal work-group (which
  // also clears *info) in sc, and added to each diagonal block as it is factored
  Scalars* sc;
  const float* G;
  float lam;
  int relative;
  float* lambda_out;
};

// 64 x 64 block (row block rb, column block cb) of a d x d row-major matrix into LDS, zeros outside.
__device__ __forceinline__ void sw_load(float (*dst)[BP], const float* src, int d, int rb, int cb) {
  const int t = threadIdx.x;
  const int r = t >> 4, c = (t & 15) * 4;
  const int gr = rb * NB + r, gc = cb * NB + c;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (gr < d && gc < d) v = *(const f32x4*)(src + (int64_t)gr * d + gc);
  *(f32x4*)&dst[r][c] = v;
}
__device__ __forceinline__ void sw_load_t(float (*dst)[BP], const float* Tk) {
  const int t = threadIdx.x;
  const int r = t >> 4, c = (t & 15) * 4;
  *(f32x4*)&dst[r][c] = *(const f32x4*)(Tk + r * NB + c);
}

// Quadrant (wave / 4, wave % 4) of X op(Y) over k < 64 (op(Y) = Y^T when ty): 16x16x4 MFMA,
// register r of lane l holds row 4 (l / 16) + r, column l % 16 of the quadrant.
__device__ __forceinline__ f32x4 sw_mm(const float (*X)[BP], const float (*Y)[BP], bool ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (wave >> 2) * 16, n0 = (wave & 3) * 16;
  const int a = lane & 15, kk = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < NB; s4 += 4) {
    const float x = X[m0 + a][s4 + kk];
    const float y = ty ? Y[n0 + a][s4 + kk] : Y[s4 + kk][n0 + a];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc, 0, 0, 0);
  }
  return acc;
}
__device__ __forceinline__ void sw_put(float (*dst)[BP], f32x4 v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (wave >> 2) * 16 + 4 * (lane >> 4), n = (wave & 3) * 16 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[m0 + r][n] = v[r];
}
// global block (rb, cb) of a d x d matrix: C = beta C + v (beta 0 or 1)
__device__ __forceinline__ void sw_store(float* C, int d, int rb, int cb, f32x4 v, bool accumulate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = rb * NB + (wave >> 2) * 16 + 4 * (lane >> 4), n = cb * NB + (wave & 3) * 16 + (lane & 15);
  if (n >= d) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (m0 + r >= d) continue;
    float* c = C + (int64_t)(m0 + r) * d + n;
    *c = accumulate ? *c + v[r] : v[r];
  }
}

// Factorization of the symmetric 64 x 64 block D (in LDS) = L L^T and T = L^-1, two columns per
// barrier.  Thread t owns row i = t/16, columns 4 (t%16) .. +3 of D (symmetric: row j also holds
// column j) and of U, which starts as I.  Step s handles columns j = 2s and j+1: rows j and j+1
// (all earlier steps applied) are published (double-buffered, one barrier per step); every thread
// forms, on its columns, row'_{j+1} = row_{j+1} - (a01 / p0) row_j (row j+1 after elimination with
// row j; p0 = a_jj, a01 = a_{j,j+1}, pivot p1 = a_{j+1,j+1} - a01^2 / p0), and every row i > j+1
// applies both eliminations, a_i -= f0 row_j + f1 row'_{j+1} with f0 = x0 / p0, f1 = (x1 - f0 a01) / p1,
// x0, x1 = row i's entries in columns j, j+1 (by symmetry, rows j and j+1's entries in column i).
// The same combination updates u_i: right-looking Cholesky and forward substitution in one sweep,
// with the divisions by l_jj = sqrt(p_j) deferred: (L^-1)_i = u_i / sqrt(p_i).  Rows past nb (last
// panel) hold the identity.  A non-positive pivot sets *info to its 1-based index (k0 + j + 1) and is
// replaced by 1.
__device__ __forceinline__ void sw_factor(const float (*D)[BP], float (*curb)[2][2][NB], float* pivs, int nb, int k0,
                                          float* Tk, int* info) {
  const int t = threadIdx.x;
  const int i = t >> 4, c0 = (t & 15) * 4;
  float ar[4], ur[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int k = c0 + m;
    ar[m] = (i < nb && k < nb) ? D[i][k] : (i == k ? 1.f : 0.f);
    ur[m] = (i == k) ? 1.f : 0.f;
  }
  auto piv = [](float p) { return p > 0.f ? p : 1.f; };
  for (int j = 0; j < NB; j += 2) {
    float(*cur)[2][NB] = curb[(j >> 1) & 1];
    const int q = i - j;   // 0: row j, 1: row j+1
    if (q == 0 || q == 1) {
      *(f32x4*)&cur[0][q][c0] = f32x4{ar[0], ar[1], ar[2], ar[3]};
      *(f32x4*)&cur[1][q][c0] = f32x4{ur[0], ur[1], ur[2], ur[3]};
    }
    __syncthreads();
    if (i > j) {
      const float p0 = piv(cur[0][0][j]);
      const float a01 = cur[0][0][j + 1];
      const float r0 = __builtin_amdgcn_rcpf(p0);
      const float g = a01 * r0;   // row'_{j+1} = row_{j+1} - g row_j
      const float p1raw = cur[0][1][j + 1] - g * a01;
      const f32x4 a0 = *(const f32x4*)&cur[0][0][c0];
      const f32x4 u0 = *(const f32x4*)&cur[1][0][c0];
      if (q == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ar[e] = fmaf(-g, a0[e], ar[e]);
          ur[e] = fmaf(-g, u0[e], ur[e]);
        }
        if ((t & 15) == 0) {
          pivs[j] = cur[0][0][j];
          pivs[j + 1] = p1raw;
        }
      } else {
        const float f0 = cur[0][0][i] * r0;
        const float f1 = (cur[0][1][i] - f0 * a01) * __builtin_amdgcn_rcpf(piv(p1raw));
        const f32x4 a1 = *(const f32x4*)&cur[0][1][c0];
        const f32x4 u1 = *(const f32x4*)&cur[1][1][c0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ar[e] = fmaf(-f1, fmaf(-g, a0[e], a1[e]), fmaf(-f0, a0[e], ar[e]));
          ur[e] = fmaf(-f1, fmaf(-g, u0[e], u1[e]), fmaf(-f0, u0[e], ur[e]));
        }
      }
    }
  }
  __syncthreads();
  if (t == 0) {
    for (int j = 0; j < nb; ++j)
      if (!(pivs[j] > 0.f)) {
        if (*info == 0) *info = k0 + j + 1;
        break;
      }
  }
  const float inv_i = 1.f / sqrtf(i < nb ? piv(pivs[i]) : 1.f);
  *(f32x4*)(Tk + i * NB + c0) = f32x4{ur[0] * inv_i, ur[1] * inv_i, ur[2] * inv_i, ur[3] * inv_i};
}

__global__ __launch_bounds__(SW_THREADS) void sweep_kernel(SweepArgs a) {
  __shared__ __attribute__((aligned(16))) float L0[NB][BP], L1[NB][BP], L2[NB][BP], L3[NB][BP], L4[NB][BP];
  __shared__ __attribute__((aligned(16))) float curb[2][2][2][NB];
  __shared__ float pivs[NB];
  const int k = a.k, d = a.d;
  int q = blockIdx.x;
  float* Tprev = a.Tb + ((k + 2) % 3) * NB * NB;   // T_{k-1}
  if (k < a.nP) {
    if (q == 0) {
      // diagonal block k: D = A_kk - X_k X_k^T, then factor
      sw_load(L1, a.Mx, d, k, k);
      if (k > 0) {
        sw_load(L0, a.Mx, d, k, k - 1);
        sw_load_t(L2, Tprev);
        __syncthreads();
        sw_put(L3, sw_mm(L0, L2, true));                    // X_k = A_k,k-1 T_{k-1}^T
        __syncthreads();
        const f32x4 xx = sw_mm(L3, L3, true);               // X_k X_k^T
        __syncthreads();
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int m0 = (wave >> 2) * 16 + 4 * (lane >> 4), n = (wave & 3) * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) L1[m0 + r][n] -= xx[r];
      }
      __syncthreads();
      const int nb = min(NB, d - k * NB);
      if (k == 0) {
        // tr(G) in fp64 over the 16 waves, then lambda; info starts at 0
        double t = 0.0;
        for (int i = threadIdx.x; i < d; i += SW_THREADS) t += (double)a.G[(int64_t)i * d + i];
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
        double* red = (double*)&L4[0][0];
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
        __syncthreads();
        if (threadIdx.x == 0) {
          double tr = 0.0;
          for (int w2 = 0; w2 < SW_THREADS / 64; ++w2) tr += red[w2];
          const float l = a.relative ? (float)((double)a.lam * tr / (double)d) : a.lam;
          a.sc->lambda = l;
          if (a.lambda_out) *a.lambda_out = l;
          *a.info = 0;
          red[0] = l;
        }
        __syncthreads();
        if ((int)threadIdx.x < nb) L1[threadIdx.x][threadIdx.x] += (float)red[0];   // G + lambda I
      } else {
        if ((int)threadIdx.x < nb) L1[threadIdx.x][threadIdx.x] += a.sc->lambda;  // G + lambda I
      }
      __syncthreads();
      sw_factor(L1, curb, pivs, nb, k * NB, a.Tb + (k % 3) * NB * NB, a.info);
      return;
    }
    --q;
  }
  if (q < a.n_fill) {
    // block (i, j) of R = C W or P = W W^T over K blocks [kb0, kb1), double-buffered through LDS
    const int nT = a.nP;
    const int g = a.fill0 + q;
    const bool is_p = g >= nT * nT;
    const int tt = g % (nT * nT), i = tt / nT, j = tt % nT;
    const float* X = is_p ? a.Wf : a.C;
    auto bx = [&](int b) { return b ? L3 : L0; };
    auto by = [&](int b) { return b ? L4 : L1; };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    sw_load(bx(0), X, d, i, a.kb0);
    if (is_p) sw_load(by(0), a.Wf, d, j, a.kb0);
    else sw_load(by(0), a.Wf, d, a.kb0, j);
    for (int kb = a.kb0; kb < a.kb1; ++kb) {
      const int b = (kb - a.kb0) & 1;
      __syncthreads();
      if (kb + 1 < a.kb1) {
        sw_load(bx(b ^ 1), X, d, i, kb + 1);
        if (is_p) sw_load(by(b ^ 1), a.Wf, d, j, kb + 1);
        else sw_load(by(b ^ 1), a.Wf, d, kb + 1, j);
      }
      const f32x4 v = sw_mm(bx(b), by(b), is_p);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += v[r];
    }
    sw_store(is_p ? a.P : a.R, d, i, j, acc, a.kb0 > 0);
    return;
  }
  q -= a.n_fill;
  if (q < a.n_a) {
    // trailing block (i, j) of A, k <= j <= i < nP, other than (k, k): A_ij -= X_i X_j^T
    int p = q + 1;
    int ii = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
    while ((ii + 1) * (ii + 2) / 2 <= p) ++ii;
    while (ii * (ii + 1) / 2 > p) --ii;
    const int i = k + ii, j = k + (p - ii * (ii + 1) / 2);
    sw_load(L0, a.Mx, d, i, k - 1);
    sw_load_t(L2, Tprev);
    if (i != j) sw_load(L1, a.Mx, d, j, k - 1);
    __syncthreads();
    sw_put(L3, sw_mm(L0, L2, true));                        // X_i
    if (i != j) sw_put(L4, sw_mm(L1, L2, true));            // X_j
    __syncthreads();
    const f32x4 v = sw_mm(L3, i != j ? L4 : L3, true);
    sw_store(a.Mx, d, i, j, -v, true);
    return;
  }
  q -= a.n_a;
  if (q < a.n_i) {
    // identity part below panel k-1: B_ic -= X_i (T_{k-1} B_{k-1,c}), c < k
    const int i = k + q / k, c = q % k;
    sw_load(L0, a.Mx, d, i, k - 1);
    sw_load(L1, a.Bx, d, k - 1, c);
    sw_load_t(L2, Tprev);
    __syncthreads();
    sw_put(L3, sw_mm(L0, L2, true));                        // X_i
    sw_put(L4, sw_mm(L2, L1, false));                       // T_{k-1} B_{k-1,c}
    __syncthreads();
    const f32x4 v = sw_mm(L3, L4, false);
    sw_store(a.Bx, d, i, c, -v, true);
    return;
  }
  q -= a.n_i;
  // final block rows: B_rc = T_r B_rc, c <= r
  int r = a.f_row0, n = r + 1;
  if (q >= n) {
    q -= n;
    r += 1;
  }
  sw_load(L1, a.Bx, d, r, q);
  sw_load_t(L2, a.Tb + (r % 3) * NB * NB);
  __syncthreads();
  const f32x4 v = sw_mm(L2, L1, false);
  sw_store(a.Bx, d, r, q, v, false);
}

// out = A B accumulated in fp64 (A, B fp32 [d, d] row-major); 64 x 64 tile per work-group,
// 4 x 4 outputs per thread.  MODE 0: R64 = A B (fp64 store).  MODE 1: the refinement residual
// r = R64 - lambda dW - A B with A = G and B = dW (fp32 store).
template <int MODE>
__global__ __launch_bounds__(NT) void gemm64_kernel(const float* A, const float* B, int d, const Scalars* sc,
                                                    double* R64, float* r) {
  __shared__ float as[16][65];
  __shared__ float bs[16][65];
  const int tpd = (d + 63) / 64;
  const int i0 = (blockIdx.x / tpd) * 64, j0 = (blockIdx.x % tpd) * 64;
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 16) {
    __syncthreads();
    for (int e = tid; e < 64 * 16; e += NT) {
      const int a = e / 16, kk = e % 16;
      as[kk][a] = (i0 + a < d && k0 + kk < d) ? A[(int64_t)(i0 + a) * d + k0 + kk] : 0.f;
      const int kk2 = e / 64, b = e % 64;
      bs[kk2][b] = (j0 + b < d && k0 + kk2 < d) ? B[(int64_t)(k0 + kk2) * d + j0 + b] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma((double)as[kk][ti * 4 + u], (double)bs[kk][tj * 4 + w], acc[u][w]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = i0 + ti * 4 + u, j = j0 + tj * 4 + w;
      if (i < d && j < d) {
        const int64_t e = (int64_t)i * d + j;
        if (MODE == 0)
          R64[e] = acc[u][w];
        else
          r[e] = (float)(R64[e] - (double)sc->lambda * (double)B[e] - acc[u][w]);
      }
    }
}

// Partial dot products for epsilon: <D,P>, <G,P>, <W,R>, <dW,R>, <dW,dW> (fp64 per block).
__global__ __launch_bounds__(NT) void dots_kernel(const float* D, const float* G, const float* P, const float* Wf,
                                                  const float* R, const float* dW, int64_t n, double* part) {
  double s[5] = {0, 0, 0, 0, 0};
  for (int64_t e = blockIdx.x * (int64_t)NT + threadIdx.x; e < n; e += (int64_t)gridDim.x * NT) {
    const double p = P[e], r = R[e], dw = dW[e];
    s[0] += (double)D[e] * p;
    s[1] += (double)G[e] * p;
    s[2] += (double)Wf[e] * r;
    s[3] += dw * r;
    s[4] += dw * dw;
  }
  __shared__ double red[5][NT];
  for (int q = 0; q < 5; ++q) red[q][threadIdx.x] = s[q];
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o)
      for (int q = 0; q < 5; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x < 5) part[blockIdx.x * 5 + threadIdx.x] = red[threadIdx.x][0];
}

// eps = sqrt(max(<D,P> - <dW,R> - lambda <dW,dW>, 0) / (<G,P> + 2 <W,R> + <D,P>)), partials added
// in block order
__global__ __launch_bounds__(NT) void eps_kernel(const double* part, int nblk, const Scalars* sc, float* eps) {
  __shared__ double red[5][NT];
  double t[5] = {0, 0, 0, 0, 0};
  for (int b = threadIdx.x; b < nblk; b += NT)
    for (int q = 0; q < 5; ++q) t[q] += part[b * 5 + q];
  for (int q = 0; q < 5; ++q) red[q][threadIdx.x] = t[q];
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o)
      for (int q = 0; q < 5; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double lam = sc->lambda;
    const double num2 = red[0][0] - red[3][0] - lam * red[4][0];
    const double den2 = red[1][0] + 2.0 * red[2][0] + red[0][0];
    *eps = (float)sqrt((num2 > 0.0 ? num2 : 0.0) / den2);
  }
}

constexpr int DOT_BLOCKS = 512;

struct WsLayout {
  float* Mx;   // d x d
  float* Bx;   // d x d: I, then L^-1
  float* Rs;   // d x d: refinement residual
  float* Rc;   // d x d
  float* Wf;   // d x d
  float* P;    // d x d (W W^T)
  float* T;    // three NB x NB slots
  Scalars* sc;
  double* part;
  double* R64; // d x d, C W accumulated in fp64 (refinement only)
};

WsLayout carve(void* ws, int d) {
  char* p = (char*)ws;
  const size_t dd = (size_t)d * d * sizeof(float);
  WsLayout w;
  w.Mx = (float*)p; p += dd;
  w.Bx = (float*)p; p += dd;
  w.Rs = (float*)p; p += dd;
  w.Rc = (float*)p; p += dd;
  w.Wf = (float*)p; p += dd;
  w.P = (float*)p; p += dd;
  w.T = (float*)p; p += 3 * NB * NB * sizeof(float);
  w.sc = (Scalars*)p; p += 256;
  w.part = (double*)p; p += DOT_BLOCKS * 5 * sizeof(double);
  w.R64 = (double*)p;
  return w;
}

#define ISPA_TRY(x)                      \
  do {                                   \
    hipError_t e_ = (x);                 \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

}  // namespace

size_t solve_workspace_bytes(int d) {
  return (size_t)d * d * sizeof(float) * 6 + 3 * NB * NB * sizeof(float) + 256 + DOT_BLOCKS * 5 * sizeof(double) +
         (size_t)d * d * sizeof(double) + 256;
}

hipError_t launch_solve(const SolveLaunch& L, hipStream_t s) {
  const int d = L.d;
  WsLayout w = carve(L.ws, d);
  const int64_t dd = (int64_t)d * d;
  const int eb = (int)((dd + NT - 1) / NT > 2048 ? 2048 : (dd + NT - 1) / NT);

  if (L.w_dtype == DT_BF16)
    hipLaunchKernelGGL(setup_kernel<BF16>, dim3(eb), dim3(NT), 0, s, L.G, (const uint16_t*)L.W, d, w.Mx, w.Bx, w.Wf);
  else if (L.w_dtype == DT_F16)
    hipLaunchKernelGGL(setup_kernel<F16>, dim3(eb), dim3(NT), 0, s, L.G, (const uint16_t*)L.W, d, w.Mx, w.Bx, w.Wf);
  else
    hipLaunchKernelGGL(setup_kernel<F32>, dim3(eb), dim3(NT), 0, s, L.G, (const float*)L.W, d, w.Mx, w.Bx, w.Wf);
  ISPA_TRY(hipGetLastError());

  // Cholesky sweep (one launch per panel, plus one that finishes the last two block rows of L^-1)
  {
    const int nP = (d + NB - 1) / NB;
    // R = C W and (for epsilon) P = W W^T ride along, split into three K ranges spread over the
    // launches in order, so a range is added only after the one before it is complete
    const int n_launch = nP + 1;
    const int n_out = nP * nP * (L.eps ? 2 : 1);
    const int n_range = n_launch < 3 ? n_launch : 3;   // launch k works on range k * n_range / n_launch
    for (int k = 0; k <= nP; ++k) {
      SweepArgs a;
      a.Mx = w.Mx;
      a.Bx = w.Bx;
      a.Tb = w.T;
      a.info = L.info;
      a.d = d;
      a.nP = nP;
      a.k = k;
      const int m = nP - k;   // block rows at or below panel k
      a.n_a = (k >= 1 && m >= 1) ? m * (m + 1) / 2 - 1 : 0;
      a.n_i = (k >= 1 && m >= 1) ? m * k : 0;
      int n_f = 0;
      if (k == nP) {
        a.f_row0 = nP >= 2 ? nP - 2 : nP - 1;
        a.f_rows = nP >= 2 ? 2 : 1;
        n_f = nP >= 2 ? (nP - 1) + nP : nP;
      } else {
        a.f_row0 = k - 2;
        a.f_rows = k >= 2 ? 1 : 0;
        n_f = k >= 2 ? k - 1 : 0;
      }
      const int range = k * n_range / n_launch;
      const int first = (range * n_launch + n_range - 1) / n_range;   // first launch of this range
      const int next = ((range + 1) * n_launch + n_range - 1) / n_range;
      const int slot = k - first, n_slots = next - first;
      a.sc = w.sc;
      a.G = L.G;
      a.lam = L.lambda;
      a.relative = L.lambda_relative;
      a.lambda_out = L.lambda_out;
      a.C = L.C;
      a.Wf = w.Wf;
      a.R = w.Rc;
      a.P = w.P;
      a.kb0 = range * nP / n_range;
      a.kb1 = (range + 1) * nP / n_range;
      a.fill0 = (int)((int64_t)n_out * slot / n_slots);
      a.n_fill = a.kb0 < a.kb1 ? (int)((int64_t)n_out * (slot + 1) / n_slots) - a.fill0 : 0;
      const int grid = (k < nP ? 1 : 0) + a.n_fill + a.n_a + a.n_i + n_f;
      hipLaunchKernelGGL(sweep_kernel, dim3(grid), dim3(SW_THREADS), 0, s, a);
      ISPA_TRY(hipGetLastError());
    }
  }
  // Z = L^-1 R (L^-1 lower triangular: only k < m0 + 64 contributes), into Mx (no longer needed)
  ISPA_TRY(run_trgemm(false, w.Bx, w.Rc, w.Mx, d, 1.f, 0.f, s));
  // dW = (L^-1)^T Z   (op(A) upper triangular: only k >= m0 contributes)
  // (W_new = W + dW is written by the last product that updates dW)
  ISPA_TRY(run_trgemm(true, w.Bx, w.Mx, L.delta_w, d, 1.f, 0.f, s, L.W, L.refine > 0 ? nullptr : L.w_new, L.w_dtype));
  if (L.refine > 0) {
    // iterative refinement: r = C W - (G + lambda I) dW with fp64 accumulation (C W formed once in
    // fp64), then dW += (L^-1)^T (L^-1 r) with the fp32 factor
    const int tpd = (d + 63) / 64;
    hipLaunchKernelGGL(gemm64_kernel<0>, dim3(tpd * tpd), dim3(NT), 0, s, L.C, w.Wf, d, w.sc, w.R64, nullptr);
    ISPA_TRY(hipGetLastError());
    for (int it = 0; it < L.refine; ++it) {
      hipLaunchKernelGGL(gemm64_kernel<1>, dim3(tpd * tpd), dim3(NT), 0, s, L.G, L.delta_w, d, w.sc, w.R64, w.Rs);
      ISPA_TRY(hipGetLastError());
      // t = L^-1 r (into Mx, no longer needed), dW += (L^-1)^T t
      ISPA_TRY(run_trgemm(false, w.Bx, w.Rs, w.Mx, d, 1.f, 0.f, s));
      ISPA_TRY(run_trgemm(true, w.Bx, w.Mx, L.delta_w, d, 1.f, 1.f, s, L.W, it + 1 == L.refine ? L.w_new : nullptr,
                          L.w_dtype));
    }
  }
  if (L.eps) {
    hipLaunchKernelGGL(dots_kernel, dim3(DOT_BLOCKS), dim3(NT), 0, s, L.D, L.G, w.P, w.Wf, w.Rc, L.delta_w, dd, w.part);
    ISPA_TRY(hipGetLastError());
    hipLaunchKernelGGL(eps_kernel, dim3(1), dim3(NT), 0, s, w.part, DOT_BLOCKS, w.sc, L.eps);
    ISPA_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace ispa
