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

// Work-group b -> tile rank (ranks: longest k range first).  Two work-groups share a CU and the
// dispatcher deals them out round-robin, so b and b + 256 tend to meet on one CU; the second 256
// take the ranks in reverse, which pairs each long tile with a short one.
__device__ __forceinline__ int tg_rank(int b, int n) {
  const int hi = n < 512 ? n : 512;
  return (b >= 256 && b < hi) ? 256 + (hi - 1 - b) : b;
}

template <bool TA>
__global__ __launch_bounds__(NT, 2) void trgemm_kernel(TrGemm g) {
  __shared__ __attribute__((aligned(16))) char a0[TG_STAGE], a1[TG_STAGE], a2[TG_STAGE], a3[TG_STAGE];
  __shared__ __attribute__((aligned(16))) char b0[TG_STAGE], b1[TG_STAGE], b2[TG_STAGE], b3[TG_STAGE];
  const int T = g.tiles, d = g.d;
  const int q = tg_rank(blockIdx.x, gridDim.x);
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
  auto barrier = [&]() { lds_barrier(); };

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
constexpr int SW_FILL_RANGES = 6;   // K ranges of the R / P products (4 blocks each at d = 1536)
static_assert(SW_THREADS >= 512, "the diagonal factorization uses 512 threads");
constexpr int BP = NB + 4;   // LDS pitch of a 64 x 64 block: 16 rows of a wave hit 16 distinct 4-bank groups

struct SweepArgs {
  float* Mx;   // d x d, G + lambda I, lower blocks updated in place
  float* Bx;   // d x d, identity part, becomes L^-1
  float* Tb;   // three 64 x 64 slots: T_k in slot k % 3
  int* info;
  int d, nP, k;
  int n_a, n_i, f_row0, f_rows;   // work items: A blocks, identity blocks, final rows [f_row0, +f_rows)
  // products that do not depend on the sweep ride along in its launches, one K range at a time:
  // R = C W (always) and the lower block triangle of P = W W^T (for epsilon); this launch computes output blocks
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
// The same block in two halves: this thread's 16 bytes from global memory, then into LDS.
__device__ __forceinline__ f32x4 sw_gload(const float* src, int d, int rb, int cb) {
  const int t = threadIdx.x;
  const int gr = rb * NB + (t >> 4), gc = cb * NB + (t & 15) * 4;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (gr < d && gc < d) v = *(const f32x4*)(src + (int64_t)gr * d + gc);
  return v;
}
__device__ __forceinline__ void sw_lput(float (*dst)[BP], f32x4 v) {
  const int t = threadIdx.x;
  *(f32x4*)&dst[t >> 4][(t & 15) * 4] = v;
}
__device__ __forceinline__ void sw_load_t(float (*dst)[BP], const float* Tk) {
  const int t = threadIdx.x;
  const int r = t >> 4, c = (t & 15) * 4;
  *(f32x4*)&dst[r][c] = *(const f32x4*)(Tk + r * NB + c);
}

// p-th entry (row-major) of a lower triangle: row ii, column jj <= ii.
__device__ __forceinline__ void tri_decode(int p, int& ii, int& jj) {
  int r = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= p) ++r;
  while (r * (r + 1) / 2 > p) --r;
  ii = r;
  jj = p - r * (r + 1) / 2;
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

// Factorization of the symmetric 64 x 64 block D (in LDS) = L L^T and T = L^-1 with 2 x 2 pivot
// blocks, one barrier per pivot pair.  512 threads work: pair p = t/16 holds rows 2p and 2p+1 at
// columns 4 (t%16) .. +3 of one combined row per matrix row (columns left of the current pivot hold
// u_i, the row of U that accumulates the eliminations and starts as e_i; the others hold the Schur
// complement), and in all 16 lanes its own diagonal block B_p = [[d00, d01], [d01, d11]].  Step s
// publishes rows 2s, 2s+1 as they stand and B_s^-1; every row i of a later pair then takes
// w_i -= [x0 x1] B_s^-1 [w_2s; w_2s+1] with x0, x1 the row's Schur entries in the pivot columns (read,
// by symmetry, from the published rows), which zeroes those entries; they are set to the u values
// -[x0 x1] B_s^-1 instead, and the pair's own block gets the same update.  At the end U D U^T is
// block diagonal with blocks B_p, so T = C^-1 U with C = chol(B_p) per pair: row 2p is u_2p / sqrt(p0),
// row 2p+1 is (u_2p+1 - g u_2p) / sqrt(p1) with p0 = d00, g = d01 / p0, p1 = d11 - g d01.  The
// pivots p0, p1 are the scalar Cholesky pivots; a non-positive one sets *info to its 1-based index
// (k0 + j + 1) and the block is then replaced by I (the results are undefined).  Rows past nb (last
// panel) hold the identity.
__device__ __forceinline__ void sw_factor(const float (*D)[BP], float (*curb)[2][2][NB], float* pivs, int nb, int k0,
                                          float* Tk, int* info) {
  __shared__ __attribute__((aligned(16))) float binv[2][4];
  const int t = threadIdx.x;
  const bool act = t < 512;
  const int p = (t >> 4) & 31, cg = t & 15, c0 = 4 * cg;
  auto dv = [&](int i, int k) { return (i < nb && k < nb) ? D[i][k] : (i == k ? 1.f : 0.f); };
  float w[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) w[h][e] = dv(2 * p + h, c0 + e);
  float d00 = dv(2 * p, 2 * p), d01 = dv(2 * p, 2 * p + 1), d11 = dv(2 * p + 1, 2 * p + 1);
  float b00 = 0.f, b01 = 0.f, b11 = 0.f;
  auto invert = [&]() {
    const float det = fmaf(d00, d11, -d01 * d01);
    const bool ok = d00 > 0.f && det > 0.f;
    const float rd = __builtin_amdgcn_rcpf(ok ? det : 1.f);
    b00 = ok ? d11 * rd : 1.f;
    b01 = ok ? -d01 * rd : 0.f;
    b11 = ok ? d00 * rd : 1.f;
  };
  if (act && p == 0) invert();
  // step s; the pivot columns 2s, 2s+1 sit at positions m, m+1 of column group s/2
  auto step = [&](auto parc, int s) {
    constexpr int par = decltype(parc)::value, m = 2 * par;
    float(*cur)[NB] = curb[par][0];
    if (act && p == s) {
      *(f32x4*)&cur[0][c0] = f32x4{w[0][0], w[0][1], w[0][2], w[0][3]};
      *(f32x4*)&cur[1][c0] = f32x4{w[1][0], w[1][1], w[1][2], w[1][3]};
      if (cg == 0) *(f32x4*)&binv[par][0] = f32x4{b00, b01, b11, 0.f};
    }
    __syncthreads();
    if (act && p > s) {
      const f32x4 bv = *(const f32x4*)&binv[par][0];
      const f32x4 P0 = *(const f32x4*)&cur[0][c0];
      const f32x4 P1 = *(const f32x4*)&cur[1][c0];
      const f32x2 X0 = *(const f32x2*)&cur[0][2 * p];
      const f32x2 X1 = *(const f32x2*)&cur[1][2 * p];
      float f0[2], f1[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f0[h] = fmaf(X1[h], bv[1], X0[h] * bv[0]);
        f1[h] = fmaf(X1[h], bv[2], X0[h] * bv[1]);
      }
      d00 = fmaf(-f1[0], X1[0], fmaf(-f0[0], X0[0], d00));
      d01 = fmaf(-f1[0], X1[1], fmaf(-f0[0], X0[1], d01));
      d11 = fmaf(-f1[1], X1[1], fmaf(-f0[1], X0[1], d11));
      const bool own = cg == (s >> 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[h][e] = fmaf(-f1[h], P1[e], fmaf(-f0[h], P0[e], w[h][e]));
        w[h][m] = own ? -f0[h] : w[h][m];
        w[h][m + 1] = own ? -f1[h] : w[h][m + 1];
      }
      if (p == s + 1) invert();
    }
  };
  for (int s = 0; s < NB / 2; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
  }
  const int j = 2 * p;
  const float p0 = d00 > 0.f ? d00 : 1.f;
  const float g = d01 / p0;
  const float p1raw = fmaf(-g, d01, d11);
  const float p1 = p1raw > 0.f ? p1raw : 1.f;
  if (act && cg == 0) {
    pivs[j] = d00;
    pivs[j + 1] = p1raw;
  }
  __syncthreads();
  if (t < 64) {
    // first non-positive (or NaN) pivot of the block, if any
    const uint64_t bad = __ballot(t < nb && !(pivs[t] > 0.f));
    if (t == 0 && bad != 0 && *info == 0) *info = k0 + __builtin_ctzll(bad) + 1;
  }
  if (act) {
    const float s0 = 1.f / sqrtf(p0), s1 = 1.f / sqrtf(p1);
    float o0[4], o1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = c0 + e;
      const float u0 = k < j ? w[0][e] : (k == j ? 1.f : 0.f);
      const float u1 = k < j ? w[1][e] : (k == j + 1 ? 1.f : 0.f);
      o0[e] = u0 * s0;
      o1[e] = fmaf(-g, u0, u1) * s1;
    }
    *(f32x4*)(Tk + j * NB + c0) = f32x4{o0[0], o0[1], o0[2], o0[3]};
    *(f32x4*)(Tk + (j + 1) * NB + c0) = f32x4{o1[0], o1[1], o1[2], o1[3]};
  }
}

__global__ __launch_bounds__(SW_THREADS) void sweep_kernel(SweepArgs a) {
  // four blocks (plus the factorization's few hundred bytes) keep two work-groups on a CU
  __shared__ __attribute__((aligned(16))) float L0[NB][BP], L1[NB][BP], L2[NB][BP], L3[NB][BP];
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
        const f32x4 x = sw_mm(L0, L2, true);                // X_k = A_k,k-1 T_{k-1}^T
        __syncthreads();
        sw_put(L0, x);
        __syncthreads();
        const f32x4 xx = sw_mm(L0, L0, true);               // X_k X_k^T
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
        double* red = (double*)&L2[0][0];
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
    // block (i, j) of R = C W (all blocks) or P = W W^T (j <= i: P is symmetric) over K blocks
    // [kb0, kb1)
    const int nT = a.nP;
    const int g = a.fill0 + q;
    const bool is_p = g >= nT * nT;
    int i = g / nT, j = g % nT;
    if (is_p) tri_decode(g - nT * nT, i, j);
    const float* X = is_p ? a.Wf : a.C;
    // K block kb0 + t passes through registers (loaded two steps ahead) into LDS slot t % 2
    const int n = a.kb1 - a.kb0;
    auto gx = [&](int t) { return sw_gload(X, d, i, a.kb0 + t); };
    auto gy = [&](int t) { return is_p ? sw_gload(a.Wf, d, j, a.kb0 + t) : sw_gload(a.Wf, d, a.kb0 + t, j); };
    f32x4 rx[2], ry[2];
    sw_lput(L0, gx(0));
    sw_lput(L1, gy(0));
    if (n > 1) {
      rx[1] = gx(1);
      ry[1] = gy(1);
    }
    if (n > 2) {
      rx[0] = gx(2);
      ry[0] = gy(2);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](auto bc, int t) {
      constexpr int b = decltype(bc)::value;
      __syncthreads();
      const f32x4 v = b ? sw_mm(L2, L3, is_p) : sw_mm(L0, L1, is_p);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += v[r];
      if (t + 1 < n) {
        sw_lput(b ? L0 : L2, rx[b ^ 1]);
        sw_lput(b ? L1 : L3, ry[b ^ 1]);
      }
      if (t + 3 < n) {
        rx[b ^ 1] = gx(t + 3);
        ry[b ^ 1] = gy(t + 3);
      }
    };
    for (int t = 0; t < n; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < n) step(std::integral_constant<int, 1>{}, t + 1);
    }
    sw_store(is_p ? a.P : a.R, d, i, j, acc, a.kb0 > 0);
    return;
  }
  q -= a.n_fill;
  if (q < a.n_a) {
    // trailing block (i, j) of A, k <= j <= i < nP, other than (k, k): A_ij -= X_i X_j^T
    int ii, jj;
    tri_decode(q + 1, ii, jj);
    const int i = k + ii, j = k + jj;
    sw_load(L0, a.Mx, d, i, k - 1);
    sw_load_t(L2, Tprev);
    if (i != j) sw_load(L1, a.Mx, d, j, k - 1);
    __syncthreads();
    const f32x4 xi = sw_mm(L0, L2, true);                   // X_i
    const f32x4 xj = i != j ? sw_mm(L1, L2, true) : xi;     // X_j
    __syncthreads();
    sw_put(L0, xi);
    sw_put(L1, xj);
    __syncthreads();
    const f32x4 v = sw_mm(L0, L1, true);
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
    const f32x4 xi = sw_mm(L0, L2, true);                   // X_i
    const f32x4 tb = sw_mm(L2, L1, false);                  // T_{k-1} B_{k-1,c}
    __syncthreads();
    sw_put(L0, xi);
    sw_put(L1, tb);
    __syncthreads();
    const f32x4 v = sw_mm(L0, L1, false);
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

// out = A B accumulated in fp64 (A, B fp32 [d, d] row-major; products of fp32 values are exact in
// fp64) on v_mfma_f64_16x16x4f64.  128 x 128 tiles of 4 waves (2 x 2 of 64 x 64, each 4 x 4 blocks of
// 16 x 16); k in stages of 16 staged through LDS as fp64 (A row-major with an odd pitch, so the 16
// rows a quarter-wave reads at one k fall in distinct banks; B row-major), the next stage's global
// loads held in registers while the current one multiplies; one barrier per stage.
// MFMA operands: lane l holds A[16 i + l%16][4 s + l/16] and B[4 s + l/16][16 j + l%16]; result
// register r of lane l is element (16 i + l/16 + 4 r, 16 j + l%16) (rows interleaved; a probe of the
// instruction on the device fixed this).
// MODE 0: R64 = A B (fp64 store).  MODE 1: the refinement residual r = R64 - lambda dW - A B with
// A = G and B = dW (fp32 store).  d is a multiple of 32.
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
constexpr int G64_AP = 17, G64_BP = 130;   // LDS pitches in doubles

template <int MODE>
__global__ __launch_bounds__(NT, 2) void gemm64_kernel(const float* A, const float* B, int d, const Scalars* sc,
                                                       double* R64, float* r) {
  __shared__ double as[2][128 * G64_AP];
  __shared__ __attribute__((aligned(16))) double bs[2][16 * G64_BP];
  const int tpd = (d + 127) / 128;
  const int i0 = (blockIdx.x / tpd) * 128, j0 = (blockIdx.x % tpd) * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 15, lk = lane >> 4;
  f64x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f64x4{0.0, 0.0, 0.0, 0.0};
  // stage loads: A rows i0 + q/4, columns k0 + 4 (q%4) .. +3; B row k0 + q/32, columns j0 + 4 (q%32) .. +3
  f32x4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + NT * h;
      const int ar = q >> 2, ac = 4 * (q & 3), br = q >> 5, bc = 4 * (q & 31);
      ra[h] = i0 + ar < d ? *(const f32x4*)(A + (int64_t)(i0 + ar) * d + k0 + ac) : f32x4{0.f, 0.f, 0.f, 0.f};
      rb[h] = j0 + bc < d ? *(const f32x4*)(B + (int64_t)(k0 + br) * d + j0 + bc) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + NT * h;
      const int ar = q >> 2, ac = 4 * (q & 3), br = q >> 5, bc = 4 * (q & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) as[buf][ar * G64_AP + ac + e] = (double)ra[h][e];
      double* bp = &bs[buf][br * G64_BP + bc];
      *(f64x2*)bp = f64x2{(double)rb[h][0], (double)rb[h][1]};
      *(f64x2*)(bp + 2) = f64x2{(double)rb[h][2], (double)rb[h][3]};
    }
  };
  gload(0);
  sstore(0);
  __syncthreads();
  const int n_st = d / 16;
  for (int st = 0; st < n_st; ++st) {
    const int cur = st & 1;
    if (st + 1 < n_st) gload(16 * (st + 1));
    const double* ap = &as[cur][(64 * wm + lr) * G64_AP + lk];
    const double* bp = &bs[cur][lk * G64_BP + 64 * wn + lr];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      double af[4], bf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = ap[16 * mi * G64_AP + 4 * kk];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bf[ni] = bp[4 * kk * G64_BP + 16 * ni];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
    if (st + 1 < n_st) sstore(cur ^ 1);
    __syncthreads();
  }
  const double lam = MODE == 1 ? (double)sc->lambda : 0.0;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + 64 * wm + 16 * mi + lk + 4 * q, j = j0 + 64 * wn + 16 * ni + lr;
        if (i < d && j < d) {
          const int64_t e = (int64_t)i * d + j;
          if (MODE == 0)
            R64[e] = acc[mi][ni][q];
          else
            r[e] = (float)(R64[e] - lam * (double)B[e] - acc[mi][ni][q]);
        }
      }
}

// Partial dot products for epsilon: <D,P>, <G,P>, <W,R>, <dW,R>, <dW,dW> (fp64 per block), row by row.
// Only the lower 64-block triangle of P is formed; D and G are symmetric, so blocks below the
// diagonal count twice and the upper ones are skipped.
__global__ __launch_bounds__(NT) void dots_kernel(const float* D, const float* G, const float* P, const float* Wf,
                                                  const float* R, const float* dW, int d, double* part) {
  double s[5] = {0, 0, 0, 0, 0};
  for (int r = blockIdx.x; r < d; r += gridDim.x)
    for (int c = 4 * (int)threadIdx.x; c < d; c += 4 * NT) {
      const int64_t e = (int64_t)r * d + c;
      const f32x4 rv = *(const f32x4*)(R + e), dv = *(const f32x4*)(dW + e), wv = *(const f32x4*)(Wf + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[2] += (double)wv[u] * rv[u];
        s[3] += (double)dv[u] * rv[u];
        s[4] += (double)dv[u] * dv[u];
      }
      const int rb = r / NB, cb = c / NB;
      if (rb >= cb) {
        const double wt = rb > cb ? 2.0 : 1.0;
        const f32x4 pv = *(const f32x4*)(P + e), Dv = *(const f32x4*)(D + e), gv = *(const f32x4*)(G + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s[0] += wt * ((double)Dv[u] * pv[u]);
          s[1] += wt * ((double)gv[u] * pv[u]);
        }
      }
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
    // R = C W and (for epsilon) the lower block triangle of P = W W^T ride along, split into
    // SW_FILL_RANGES K ranges spread over the launches in order, so a range is added only after the
    // one before it is complete
    const int n_launch = nP + 1;
    const int n_out = nP * nP + (L.eps ? nP * (nP + 1) / 2 : 0);
    const int n_range = n_launch < SW_FILL_RANGES ? n_launch : SW_FILL_RANGES;   // launch k works on range k * n_range / n_launch
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
    const int tpd = (d + 127) / 128;
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
    hipLaunchKernelGGL(dots_kernel, dim3(DOT_BLOCKS), dim3(NT), 0, s, L.D, L.G, w.P, w.Wf, w.Rc, L.delta_w, d, w.part);
    ISPA_TRY(hipGetLastError());
    hipLaunchKernelGGL(eps_kernel, dim3(1), dim3(NT), 0, s, w.part, DOT_BLOCKS, w.sc, L.eps);
    ISPA_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace ispa
