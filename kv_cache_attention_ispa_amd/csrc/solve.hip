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
//   Optional iterative refinement (a given number of steps): r = C W - (G + lambda I) dW to about
//   35 bits from exact int8 products of fixed-point digits (refine.hip), then dW += (L^-1)^T (L^-1 r).
//
// "Dynamic layer selection" ranks layers by the reconstruction error epsilon;
// it is evaluated here from the statistics alone (D = dA^T dA, P = W W^T):
//   ||A_loc dW - dA W||^2 = <D, P> - <dW, R> - lambda ||dW||^2   (at the optimum)
//   ||A_full W||^2        = <G, P> + 2 <W, R> + <D, P>.
//
// Every step is a HIP kernel enqueued on the caller's stream; the host never
// waits.  A non-positive pivot sets *info to its 1-based index.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int NB = 64;          // Cholesky panel width
constexpr int NT = 256;

// Layers are solved side by side: blockIdx.y is the layer, and every array of the call is reached
// through a per-layer step in bytes (0 for arrays shared by all layers).
template <typename P>
__device__ __forceinline__ P* at_layer(P* p, int64_t step_bytes) {
  return p ? (P*)((char*)p + (int64_t)blockIdx.y * step_bytes) : p;
}

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
  int64_t sa, sb, sc, sw;   // per-layer steps (bytes) of A, B, C and of W / Wn
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
  g.A = at_layer(g.A, g.sa);
  g.B = at_layer(g.B, g.sb);
  g.C = at_layer(g.C, g.sc);
  g.W = at_layer(g.W, g.sw);
  g.Wn = at_layer(g.Wn, g.sw);
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

// Per-layer byte steps of the arrays a solve touches: the workspace and the caller's d x d matrices
// (fp32, and W / W_new in W's dtype).
struct Steps {
  int64_t ws, mat, wmat;
  int batch;
};

// C = alpha op(L) B + beta C with L = A lower triangular (op = identity or transpose), per layer
hipError_t run_trgemm(bool transA, const float* A, int64_t sa, const float* B, int64_t sb, float* C, int64_t sc,
                      int d, float alpha, float beta, int batch, hipStream_t s, const void* W = nullptr,
                      void* Wn = nullptr, int wdt = 0, int64_t sw = 0) {
  TrGemm g;
  g.W = W; g.Wn = Wn; g.wdt = wdt;
  g.A = A; g.B = B; g.C = C;
  g.sa = sa; g.sb = sb; g.sc = sc; g.sw = sw;
  g.d = d;
  g.tiles = (d + TG_TILE - 1) / TG_TILE;
  g.alpha = alpha; g.beta = beta;
  const dim3 grid(g.tiles * g.tiles, batch);
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

// Per-panel launches: Mx = G (lambda joins the diagonal blocks as the sweep factors them) and Bx = I
// (becomes L^-1).
__global__ __launch_bounds__(NT) void setup_kernel(const float* G, int d, float* Mx, float* Bx, Steps st) {
  G = at_layer(G, st.mat);
  Mx = at_layer(Mx, st.ws);
  Bx = at_layer(Bx, st.ws);
  const int64_t n = (int64_t)d * d;
  for (int64_t e = blockIdx.x * (int64_t)NT + threadIdx.x; e < n; e += (int64_t)gridDim.x * NT) {
    const int i = (int)(e / d), j = (int)(e % d);
    Mx[e] = G[e];
    Bx[e] = (i == j) ? 1.f : 0.f;
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
static_assert(SW_THREADS >= 512, "the diagonal factorization uses 512 threads");
constexpr int BP = NB + 4;   // LDS pitch of a 64 x 64 block: 16 rows of a wave hit 16 distinct 4-bank groups

struct SweepArgs {
  float* Mx;   // d x d, G + lambda I, lower blocks updated in place
  float* Bx;   // d x d, identity part, becomes L^-1
  float* Tb;   // three 64 x 64 slots: T_k in slot k % 3
  int* info;
  int d, nP, k;
  int n_a, n_i, f_row0, f_rows;   // work items: A blocks, identity blocks, final rows [f_row0, +f_rows)
  // lambda (absolute, or lam * tr(G) / d): set by the first launch's diagonal work-group (which
  // also clears *info) in sc, and added to each diagonal block as it is factored
  Scalars* sc;
  const float* G;
  float lam;
  int relative;
  float* lambda_out;
  Steps st;
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

// p-th entry (row-major) of a lower triangle: row ii, column jj <= ii.
__device__ __forceinline__ void tri_decode(int p, int& ii, int& jj) {
  int r = (int)((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= p) ++r;
  while (r * (r + 1) / 2 > p) --r;
  ii = r;
  jj = p - r * (r + 1) / 2;
}

// ------------------------------------------------------------------------------------------
// R = C W and (for epsilon) the lower block triangle of P = W W^T on bf16 MFMA (32x32x16), before
// the sweep.  An fp32 operand x is split into three bf16 parts x = x1 + x2 + x3 + r with x1 =
// bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2) (each difference is exact in fp32; the three
// parts carry 24 significant bits, so |r| is at most about 2^-24 |x|, the fp32 rounding).  A product
// term takes the parts x_i y_j with i + j <= 4, accumulated in fp32 (the dropped ones are below
// 2^-24 of the term): the result is an fp32 product up to the order of the sums.  A bf16 W (WPARTS
// 1) is its own single part: R takes three MFMAs per 16-deep step, and P one, whose bf16 x bf16
// products are exact in fp32.
// split_kernel writes the parts once per call into the workspace (bf16, [part][row][col]): C in
// three parts, W and W^T in WPARTS; both products are then NT products (k-contiguous rows on both
// sides): R[i][j] = sum_k C[i][k] W^T[j][k], P[i][j] = sum_k W[i][k] W[j][k].
// ------------------------------------------------------------------------------------------
constexpr int RP_K = 32;
constexpr int RP_PITCH = RP_K + 8;   // bf16 per LDS row (80 bytes: 16-byte aligned rows)

__device__ __forceinline__ void bf16_split3(float x, uint16_t (&part)[3]) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    part[i] = Cvt<BF16>::from_f(x);
    x -= Cvt<BF16>::to_f(part[i]);
  }
}

// Work-group (bi, bj): the 64 x 64 block (bi, bj) of C and of W (read in its own type), split; W's
// parts also go to the transposed block through LDS.  Thread t covers row t / 4, 16 columns from
// 16 (t % 4).  When state is set, the work-groups also clear the one-launch sweep's n_state state
// ints and *info.
template <int WPARTS, typename WT>
__global__ __launch_bounds__(256) void split_kernel(const float* __restrict__ C, const typename WT::storage* __restrict__ W,
                                                    uint16_t* __restrict__ sp, int d, Steps st, int* state,
                                                    int n_state, int* info) {
  C = at_layer(C, st.mat);
  W = at_layer(W, st.wmat);
  sp = at_layer(sp, st.ws);
  if (state) {
    for (int e = blockIdx.x * 256 + (int)threadIdx.x; e < n_state; e += gridDim.x * 256) state[e] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *info = 0;
  }
  const int64_t dd = (int64_t)d * d;
  __shared__ uint16_t tile[WPARTS][64][66];   // W parts of the block, [row][col]
  const int nT = (d + 63) / 64, bi = blockIdx.x / nT, bj = blockIdx.x % nT;
  const int t = threadIdx.x, r = t >> 2, c = 16 * (t & 3);
  auto put = [](uint16_t* dst, const uint16_t (&v)[16][3], int i) {
    u32x4 w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[h][e] = v[8 * h + 2 * e][i] | (uint32_t)v[8 * h + 2 * e + 1][i] << 16;
    *(u32x4*)dst = w[0];
    *(u32x4*)(dst + 8) = w[1];
  };
  // d is a multiple of 32, so a row's 16 columns are all in range or all out
  const int gr = 64 * bi + r, gc = 64 * bj + c;
  if (gr < d && gc < d) {
    uint16_t v[16][3];
    const int64_t o = (int64_t)gr * d + gc;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 x = *(const f32x4*)(C + o + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) bf16_split3(x[e], v[4 * h + e]);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) put(sp + i * dd + o, v, i);
#pragma unroll
    for (int e = 0; e < 16; ++e) bf16_split3(Cvt<WT>::to_f(W[o + e]), v[e]);
#pragma unroll
    for (int i = 0; i < WPARTS; ++i) {
      put(sp + (3 + i) * dd + o, v, i);
#pragma unroll
      for (int e = 0; e < 16; ++e) tile[i][r][c + e] = v[e][i];
    }
  }
  __syncthreads();
  // W^T block (bj, bi): row 64 bj + r holds column r of the W block, columns 64 bi + c .. + 15
  const int tr = 64 * bj + r, tc = 64 * bi + c;
  if (tr < d && tc < d) {
    uint16_t v[16][3];
#pragma unroll
    for (int i = 0; i < WPARTS; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e][i] = tile[i][c + e][r];
#pragma unroll
    for (int i = 0; i < WPARTS; ++i) put(sp + (6 + i) * dd + (int64_t)tr * d + tc, v, i);
  }
}

// One 64 x 64 output block q (R blocks first, then P's lower blocks), computed by the first 256
// threads as 4 waves of 32 x 32 (every thread of the work-group takes part in the barriers); K steps
// of 32 pass through registers, one step ahead, into LDS (every part of both operands).
template <int WPARTS>
__device__ __forceinline__ void rp_tile(const uint16_t* __restrict__ sp, float* __restrict__ R, float* __restrict__ P,
                                        int d, int n_r, int q, uint16_t (*As)[64][RP_PITCH],
                                        uint16_t (*Bs)[64][RP_PITCH]) {
  const int64_t dd = (int64_t)d * d;
  const int nT = (d + 63) / 64, t = threadIdx.x;
  const bool on = t < 256;
  const bool is_p = q >= n_r;
  int bi, bj;
  if (is_p) {
    tri_decode(q - n_r, bi, bj);
  } else {
    bi = q / nT;
    bj = q % nT;
  }
  const int a_parts = is_p ? WPARTS : 3;
  const uint16_t* A = sp + (is_p ? 3 * dd : 0) + (int64_t)64 * bi * d;        // W or C rows of block bi
  const uint16_t* B = sp + (is_p ? 3 * dd : 6 * dd) + (int64_t)64 * bj * d;   // W or W^T rows of block bj
  const int lr = (t & 255) >> 2, lk = 8 * (t & 3);
  const bool a_in = 64 * bi + lr < d, b_in = 64 * bj + lr < d;
  u32x4 ra[3], rb[WPARTS];
  auto load = [&](int k0) {
    const int64_t o = (int64_t)lr * d + k0 + lk;
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (i < a_parts) ra[i] = a_in ? *(const u32x4*)(A + i * dd + o) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < WPARTS; ++j) rb[j] = b_in ? *(const u32x4*)(B + j * dd + o) : u32x4{0u, 0u, 0u, 0u};
  };
  const int lane = t & 63, wave = (t & 255) >> 6, wm = wave >> 1, wn = wave & 1;
  const int mrow = 32 * wm + (lane & 31), nrow = 32 * wn + (lane & 31), kk = 8 * (lane >> 5);
  f32x16 acc = {};
  if (on) load(0);
  for (int k0 = 0; k0 < d; k0 += RP_K) {
    __syncthreads();
    if (on) {
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (i < a_parts) *(u32x4*)&As[i][lr][lk] = ra[i];
#pragma unroll
      for (int j = 0; j < WPARTS; ++j) *(u32x4*)&Bs[j][lr][lk] = rb[j];
    }
    __syncthreads();
    if (!on) continue;
    if (k0 + RP_K < d) load(k0 + RP_K);
#pragma unroll
    for (int s = 0; s < RP_K; s += 16) {
      u32x4 ap[3], bp[WPARTS];
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (i < a_parts) ap[i] = *(const u32x4*)&As[i][mrow][s + kk];
#pragma unroll
      for (int j = 0; j < WPARTS; ++j) bp[j] = *(const u32x4*)&Bs[j][nrow][s + kk];
      // smallest terms first
#pragma unroll
      for (int sum = 2; sum >= 0; --sum)
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int j = sum - i;
          if (j >= 0 && j < WPARTS && i < a_parts) acc = mfma32x32x16<BF16>(ap[i], bp[j], acc);
        }
    }
  }
  float* out = is_p ? P : R;
  const int col = 64 * bj + 32 * wn + (lane & 31);
  if (on && col < d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * bi + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row < d) out[(int64_t)row * d + col] = acc[r];
    }
  }
}

template <int WPARTS>
__global__ __launch_bounds__(256) void rp_kernel(const uint16_t* __restrict__ sp, float* __restrict__ R,
                                                 float* __restrict__ P, int d, int n_r, Steps st) {
  __shared__ __attribute__((aligned(16))) uint16_t As[3][64][RP_PITCH], Bs[WPARTS][64][RP_PITCH];
  rp_tile<WPARTS>(at_layer(sp, st.ws), at_layer(R, st.ws), at_layer(P, st.ws), d, n_r, blockIdx.x, As, Bs);
}

// Quadrant qd (rows 16 (qd / 4) .., columns 16 (qd % 4) ..) of X op(Y) over k < 64 (op(Y) = Y^T when
// ty): 16x16x4 MFMA, register r of lane l holds row 4 (l / 16) + r, column l % 16 of the quadrant.
// MFMA step s sums k = s, 16 + s, 32 + s, 48 + s (lane group g = l / 16 supplies k = 16 g + s), so a
// lane's sixteen X values (and Y values when ty) are one contiguous row piece: four 16-byte reads.
// sw_mm / sw_put take the quadrant of the calling wave (16 waves cover the block).
__device__ __forceinline__ f32x4 sw_mm_q(const float (*X)[BP], const float (*Y)[BP], bool ty, int qd) {
  const int lane = threadIdx.x & 63;
  const int m0 = (qd >> 2) * 16, n0 = (qd & 3) * 16;
  const int a = lane & 15, k0 = 16 * (lane >> 4);
  f32x4 xv[4], yv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    xv[u] = *(const f32x4*)&X[m0 + a][k0 + 4 * u];
    if (ty) {
      yv[u] = *(const f32x4*)&Y[n0 + a][k0 + 4 * u];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[u][e] = Y[k0 + 4 * u + e][n0 + a];
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[u][e], yv[u][e], acc, 0, 0, 0);
  return acc;
}
// Half h of sw_mm_q's MFMA steps (s = 8 h .. 8 h + 7) added to acc: the two halves in order give
// sw_mm_q's result bit for bit.
__device__ __forceinline__ f32x4 sw_mm_q_half(const float (*X)[BP], const float (*Y)[BP], bool ty, int qd, int h,
                                              f32x4 acc) {
  const int lane = threadIdx.x & 63;
  const int m0 = (qd >> 2) * 16, n0 = (qd & 3) * 16;
  const int a = lane & 15, k0 = 16 * (lane >> 4) + 8 * h;
  f32x4 xv[2], yv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    xv[u] = *(const f32x4*)&X[m0 + a][k0 + 4 * u];
    if (ty) {
      yv[u] = *(const f32x4*)&Y[n0 + a][k0 + 4 * u];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[u][e] = Y[k0 + 4 * u + e][n0 + a];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[u][e], yv[u][e], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4 sw_mm(const float (*X)[BP], const float (*Y)[BP], bool ty) {
  return sw_mm_q(X, Y, ty, threadIdx.x >> 6);
}
__device__ __forceinline__ void sw_put_q(float (*dst)[BP], f32x4 v, int qd) {
  const int lane = threadIdx.x & 63;
  const int m0 = (qd >> 2) * 16 + 4 * (lane >> 4), n = (qd & 3) * 16 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[m0 + r][n] = v[r];
}
__device__ __forceinline__ void sw_put(float (*dst)[BP], f32x4 v) { sw_put_q(dst, v, threadIdx.x >> 6); }
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
// panel) hold the identity.  T goes to Tk (global) and/or Tl (LDS), whichever is set.
// Threads 512 .. 1023 take no part in the factorization: before each step's barrier they call
// side(step) (step = 0 .. 31), so work of their own runs between the factorization's barriers.
struct NoSide {
  __device__ __forceinline__ void operator()(int) const {}
};
template <typename Side>
__device__ __forceinline__ void sw_factor(const float (*D)[BP], float (*curb)[2][2][NB], float* pivs, int nb, int k0,
                                          float* Tk, int* info, float (*Tl)[BP], Side side) {
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
    if (!act) side(s);
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
#pragma unroll
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
    if (Tk) {
      *(f32x4*)(Tk + j * NB + c0) = f32x4{o0[0], o0[1], o0[2], o0[3]};
      *(f32x4*)(Tk + (j + 1) * NB + c0) = f32x4{o1[0], o1[1], o1[2], o1[3]};
    }
    if (Tl) {
      *(f32x4*)&Tl[j][c0] = f32x4{o0[0], o0[1], o0[2], o0[3]};
      *(f32x4*)&Tl[j + 1][c0] = f32x4{o1[0], o1[1], o1[2], o1[3]};
    }
  }
}

__global__ __launch_bounds__(SW_THREADS) void sweep_kernel(SweepArgs a) {
  a.Mx = at_layer(a.Mx, a.st.ws);
  a.Bx = at_layer(a.Bx, a.st.ws);
  a.Tb = at_layer(a.Tb, a.st.ws);
  a.sc = at_layer(a.sc, a.st.ws);
  a.G = at_layer(a.G, a.st.mat);
  a.info = at_layer(a.info, (int64_t)sizeof(int));
  a.lambda_out = at_layer(a.lambda_out, (int64_t)sizeof(float));
  // three blocks (plus the factorization's few hundred bytes) keep two work-groups on a CU
  __shared__ __attribute__((aligned(16))) float L0[NB][BP], L1[NB][BP], L2[NB][BP];
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
      sw_factor(L1, curb, pivs, nb, k * NB, a.Tb + (k % 3) * NB * NB, a.info, (float(*)[BP]) nullptr, NoSide{});
      return;
    }
    --q;
  }
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

// ------------------------------------------------------------------------------------------
// One-launch sweep (one layer, nP <= PS_MAX_PANELS).  The same factorization and identity part as
// the per-panel launches above, bit for bit, with the launch boundaries replaced by version flags:
//   * work-group 0 carries the diagonal chain.  At step k it factors D_k (ready in LDS), publishes
//     T_k and X_{k+1} = (k+1, k) T_k^T, and applies panel k to (k+1, k+1), which gives D_{k+1}.
//     So the chain never waits for a launch.
//   * work-groups 1 and 2 bring row k+1 up to the chain: work-group 2 applies panel k-2 to its
//     blocks (k+1, k-1 .. k+1) from the workers' versions, work-group 1 then applies panel k-1 to
//     (k+1, k) and (k+1, k+1).  At each panel p the blocks of rows p+1 .. p+3 right of the panel are
//     these three work-groups', never the workers'.
//   * the other work-groups take tasks from a queue ordered by panel: the trailing update of a block
//     by a panel (A task), the identity-part update (B task) and the final T_r B_rc (F task, into
//     L^-1).  A task waits for the versions it reads; tasks are handed out in an order in which
//     every wait is for a task handed out earlier, so the queue always makes progress.
// A version is the number of panels applied to a block (identity part: updates applied).  Version 0
// of an A block is G itself; later versions live in Mx.
// Coherence across the XCDs: every block that one work-group writes and another reads (Mx, Bx, the
// T slots) and every flag goes through device-scope (sc1) loads and stores, which bypass the
// XCD-local caches, so no cache write-back or invalidation is needed.  A writer's stores complete
// (s_waitcnt) before its flag is set; a reader loads the data only after it has seen the flag.
// Every wait is bounded: a wait that times out sets *info = -2 (results undefined) and makes every
// later wait return at once.
// ------------------------------------------------------------------------------------------
constexpr int PS_MAX_PANELS = 32;
// Every work-group of the sweep takes a whole CU (one fits by LDS); nothing else runs beside it, so
// the chain's CU is never shared.
constexpr int PS_WORKERS = 253;
constexpr int PS_WAIT_SPINS = 1 << 21;
constexpr int PS_STATE_INTS = 64;   // [0] T blocks published, [1] next task, [2] a wait timed out

struct PsArgs {
  const float* G;
  float* Mx;     // A blocks at versions >= 1
  float* Bx;     // identity part as it is updated
  float* Linv;   // L^-1, lower blocks
  float* Tb;     // T_k in slot k
  float* Xs;     // X_{k+1} = (k+1, k) T_k^T (panels < k applied) in slot k
  int* st;       // state, then the A versions [nP][nP], then the identity-part versions [nP][nP]
  const uint16_t* sp;   // bf16 parts of C, W and W^T (split_kernel)
  float* Rc;            // R = C W
  float* P;             // lower block triangle of W W^T (with eps)
  int wparts, n_r, n_rp, rp_share;   // R blocks, R and P blocks, R/P blocks per panel
  int* info;
  Scalars* sc;
  float lam;
  int relative;
  float* lambda_out;
  int d, nP, n_tasks;
};

// one thread: wait until *f >= v; false after a time-out (of this wait or of an earlier one)
__device__ bool ps_wait(const PsArgs& a, const int* f, int v) {
  if (flag_load(f) >= v) return true;
  for (int n = 0; n < PS_WAIT_SPINS; ++n) {
    __builtin_amdgcn_s_sleep(2);
    if (flag_load(f) >= v) return true;
    if ((n & 63) == 63 && flag_load(a.st + 2)) return false;
  }
  flag_store(a.st + 2, 1);
  flag_store(a.info, -2);
  return false;
}
// one thread: wait until f[i] >= v[i] for i < n; the flags are read together, so the satisfied ones
// cost one round trip in all
template <int N>
__device__ __forceinline__ void ps_wait_all(const PsArgs& a, const int* const (&f)[N], const int (&v)[N], int n) {
  int got[N];
#pragma unroll
  for (int i = 0; i < N; ++i) got[i] = i < n ? flag_load(f[i]) : 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n && got[i] < v[i]) ps_wait(a, f[i], v[i]);
}
// all threads: this work-group's stores have completed; then thread 0 sets flag = v
__device__ __forceinline__ void ps_publish(int* flag, int v) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) flag_store(flag, v);
}

// device-scope block access through a buffer over a d x d fp32 matrix (offsets past the end read 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ps_rsrc(const float* p, int64_t elems) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(elems * 4), 0x00020000);
}
__device__ __forceinline__ float ps_ld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
}
__device__ __forceinline__ void ps_st1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kSc1);
}
constexpr uint32_t kOut = 0x80000000u;   // an offset past every buffer: loads return 0
// offset = in ? off : kOut, kept a value (v_cndmask): left visible, the compiler turns the selected
// load into two loads in branches with a wait for the first between them
__device__ __forceinline__ uint32_t ps_off(bool in, uint32_t off) {
  uint32_t o = in ? off : kOut;
  asm volatile("" : "+v"(o));
  return o;
}
// block (rb, cb) into LDS (1024 threads), zeros outside the matrix
__device__ __forceinline__ void ps_load_blk(float (*dst)[BP], __amdgpu_buffer_rsrc_t r, int d, int rb, int cb) {
  const int t = threadIdx.x;
  const int rr = t >> 4, c = (t & 15) * 4;
  const int gr = rb * NB + rr, gc = cb * NB + c;
  *(f32x4*)&dst[rr][c] = sc1_ld4(r, ps_off(gr < d && gc < d, (uint32_t)((gr * d + gc) * 4)));
}
// global block (rb, cb) = src + v (src and dst buffers may differ; accumulate = false: dst = v)
__device__ __forceinline__ void ps_store_blk(__amdgpu_buffer_rsrc_t dst, __amdgpu_buffer_rsrc_t src, int d, int rb,
                                             int cb, f32x4 v, bool accumulate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = rb * NB + (wave >> 2) * 16 + 4 * (lane >> 4), n = cb * NB + (wave & 3) * 16 + (lane & 15);
  if (n >= d) return;
  float o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = accumulate ? ps_ld1(src, ps_off(m0 + r < d, (uint32_t)(((m0 + r) * d + n) * 4))) : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (m0 + r < d) ps_st1(dst, (uint32_t)(((m0 + r) * d + n) * 4), accumulate ? o[r] + v[r] : v[r]);
}

// Tasks of panel p (m = nP - 1 - p block rows below it): A tasks over blocks (i, j), p < j <= i,
// in row order without the first six (rows p+1 .. p+3: the chain's); B tasks (i, c), i > p >= c;
// F tasks (p, c), c < p; then a share of the R = C W and W W^T blocks, which wait for nothing.
constexpr int PS_CHAIN_ENTRIES = 6;
__host__ __device__ __forceinline__ int ps_n_a(int m) {
  return m * (m + 1) / 2 > PS_CHAIN_ENTRIES ? m * (m + 1) / 2 - PS_CHAIN_ENTRIES : 0;
}
__host__ __device__ __forceinline__ int ps_count(int nP, int p) {
  const int m = nP - 1 - p;
  return ps_n_a(m) + m * (p + 1) + p;
}
__host__ __device__ __forceinline__ int ps_rp_count(int n_rp, int share, int p) {
  const int left = n_rp - p * share;
  return left <= 0 ? 0 : (left < share ? left : share);
}

__global__ __launch_bounds__(SW_THREADS) void psweep_kernel(PsArgs a) {
  __shared__ __attribute__((aligned(16))) float B0[NB][BP], B1[NB][BP], B2[NB][BP], B3[NB][BP], B4[NB][BP],
      B5[NB][BP], B6[NB][BP];
  __shared__ __attribute__((aligned(16))) float curb[2][2][2][NB];
  __shared__ float pivs[NB];
  __shared__ int sq;
  const int d = a.d, nP = a.nP, t = threadIdx.x;
  const int64_t dd = (int64_t)d * d;
  int* verA = a.st + PS_STATE_INTS;
  int* verB = verA + nP * nP;
  const int* tflag = a.st;
  const __amdgpu_buffer_rsrc_t rG = ps_rsrc(a.G, dd), rM = ps_rsrc(a.Mx, dd), rB = ps_rsrc(a.Bx, dd),
                               rT = ps_rsrc(a.Tb, (int64_t)nP * NB * NB), rX = ps_rsrc(a.Xs, (int64_t)nP * NB * NB);

  // a 64 x 64 slot (T or X) into LDS / an LDS block into a slot (1024 threads)
  auto slot_load = [&](float(*dst)[BP], __amdgpu_buffer_rsrc_t r, int k) {
    const int rr = t >> 4, c = (t & 15) * 4;
    *(f32x4*)&dst[rr][c] = sc1_ld4(r, (uint32_t)(((k * NB + rr) * NB + c) * 4));
  };
  auto slot_store = [&](__amdgpu_buffer_rsrc_t r, int k, const float(*src)[BP]) {
    const int rr = t >> 4, c = (t & 15) * 4;
    sc1_st4(r, (uint32_t)(((k * NB + rr) * NB + c) * 4), *(const f32x4*)&src[rr][c]);
  };
  // block (rb, cb) of Mx from LDS (1024 threads), inside the matrix only
  auto blk_store = [&](int rb, int cb, const float(*src)[BP]) {
    const int rr = t >> 4, c = (t & 15) * 4;
    const int gr = rb * NB + rr, gc = cb * NB + c;
    if (gr < d && gc < d) sc1_st4(rM, (uint32_t)((gr * d + gc) * 4), *(const f32x4*)&src[rr][c]);
  };
  const int lane = t & 63, wave = t >> 6;
  const int qm = (wave >> 2) * 16 + 4 * (lane >> 4), qn = (wave & 3) * 16 + (lane & 15);   // quadrant element

  if (blockIdx.x == 0) {
    // ---------------- the diagonal chain ----------------
    float(*D)[BP] = B0;    // the block being factored
    float(*Tc)[BP] = B1;   // T_k
    float(*S1)[BP] = B2;   // (k+1, k), panels < k applied
    float(*S2)[BP] = B3;   // (k+1, k+1), panels < k applied
    float(*Xk)[BP] = B4;   // X_{k+1} = S1 T_k^T
    sw_load(D, a.G, d, 0, 0);
    float lam;
    {
      // tr(G) in fp64 over the 16 waves, then lambda (S1 is free until step 0's side work)
      double tr = 0.0;
      for (int i = t; i < d; i += SW_THREADS) tr += (double)a.G[(int64_t)i * d + i];
      for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o);
      double* red = (double*)&S1[0][0];
      if ((t & 63) == 0) red[t >> 6] = tr;
      __syncthreads();
      if (t == 0) {
        double sum = 0.0;
        for (int w2 = 0; w2 < SW_THREADS / 64; ++w2) sum += red[w2];
        const float l = a.relative ? (float)((double)a.lam * sum / (double)d) : a.lam;
        a.sc->lambda = l;
        if (a.lambda_out) *a.lambda_out = l;
        red[0] = l;
      }
      __syncthreads();
      lam = (float)red[0];
      if (t < min(NB, d)) D[t][t] += lam;   // G + lambda I
      __syncthreads();
    }
    const int tt = t - 512;                     // side threads
    const int lr = tt >> 3, lc = 8 * (tt & 7);  // side loads: row lr, columns lc .. lc + 7
    for (int k = 0; k < nP; ++k) {
      const int nb = min(NB, d - k * NB);
      const bool next = k + 1 < nP;
      // side work: S1, S2 as work-group 1 leaves them (G itself for k = 0).  The flag is read at
      // step 20 and checked at step 22 (waiting only if work-group 1 is late); the blocks are
      // loaded at step 23 and put into LDS after the factorization.
      f32x4 tmp[2][2];
      int fl = 0;
      auto side = [&](int s) {
        if (!next) return;
        if (s == 20) {
          if (tt == 0 && k >= 1) fl = flag_load(verA + (k + 1) * nP + k + 1);
        } else if (s == 22) {
          if (tt == 0 && k >= 1 && fl < k) ps_wait(a, verA + (k + 1) * nP + k + 1, k);
        } else if (s == 23) {
          const __amdgpu_buffer_rsrc_t src = k == 0 ? rG : rM;   // version k
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int gr = (k + 1) * NB + lr, gc = (k + b) * NB + lc;
#pragma unroll
            for (int h = 0; h < 2; ++h)
              tmp[b][h] = sc1_ld4(src, ps_off(gr < d && gc + 4 * h < d, (uint32_t)((gr * d + gc + 4 * h) * 4)));
          }
        }
      };
      sw_factor(D, curb, pivs, nb, k * NB, (float*)nullptr, a.info, Tc, side);
      __syncthreads();
      if (t >= 512 && next) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          *(f32x4*)&S1[lr][lc + 4 * h] = tmp[0][h];
          *(f32x4*)&S2[lr][lc + 4 * h] = tmp[1][h];
        }
      }
      // T_k into its slot (read by the workers and work-groups 1 and 2) and into L^-1 block (k, k)
      slot_store(rT, k, Tc);
      {
        const int rr = t >> 4, c = (t & 15) * 4;
        const int gr = k * NB + rr, gc = k * NB + c;
        if (gr < d && gc < d) *(f32x4*)(a.Linv + (int64_t)gr * d + gc) = *(const f32x4*)&Tc[rr][c];
      }
      __syncthreads();
      // panel k on (k+1, k+1): X_{k+1} = S1 T_k^T (published with T_k) and
      // D_{k+1} = S2 - X_{k+1} X_{k+1}^T + lambda I, while the stores complete; then the flag
      if (next) {
        const f32x4 x = sw_mm(S1, Tc, true);
        sw_put(Xk, x);
        __syncthreads();
        slot_store(rX, k, Xk);
        const f32x4 xx = sw_mm(Xk, Xk, true);
        const int nb1 = min(NB, d - (k + 1) * NB);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = S2[qm + r][qn] - xx[r];
          if (qm + r == qn && qn < nb1) v += lam;
          D[qm + r][qn] = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t == 0) flag_store(a.st, k + 1);
    }
    return;
  }

  if (blockIdx.x == 1) {
    // ---------------- panel k-1 on row k+1 ----------------
    // Round k (1 <= k <= nP-2), r = k+1: from (r, k-1), (r, k), (r, r) with panels < k-1 applied
    // (work-group 2's, G for k = 1) and, once T_{k-1} is out, X_k = X slot k-1:
    //   X_r = (r, k-1) T_{k-1}^T,  (r, k) -= X_r X_k^T,  (r, r) -= X_r X_r^T,
    // published as version k ((r, k) is also the workers' panel-k block; (r, r)'s version is work-group
    // 0's flag).
    float(*T)[BP] = B0;
    float(*Xp)[BP] = B1;
    float(*R1)[BP] = B2;
    float(*R2)[BP] = B3;
    float(*R3)[BP] = B4;
    for (int k = 1; k + 1 < nP; ++k) {
      const int r = k + 1;
      if (t == 0 && k >= 2) ps_wait(a, verA + r * nP + r, k - 1);
      __syncthreads();
      const __amdgpu_buffer_rsrc_t src = k == 1 ? rG : rM;   // version k - 1
      ps_load_blk(R1, src, d, r, k - 1);
      ps_load_blk(R2, src, d, r, k);
      ps_load_blk(R3, src, d, r, r);
      if (t == 0) {
        for (int n = 0; n < 4096 && flag_load(tflag) < k; ++n) {
        }
        ps_wait(a, tflag, k);
      }
      __syncthreads();
      slot_load(T, rT, k - 1);
      slot_load(Xp, rX, k - 1);
      __syncthreads();
      const f32x4 xr = sw_mm(R1, T, true);
      __syncthreads();
      sw_put(R1, xr);
      __syncthreads();
      const f32x4 u2 = sw_mm(R1, Xp, true);
      const f32x4 u3 = sw_mm(R1, R1, true);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        R2[qm + q][qn] -= u2[q];
        R3[qm + q][qn] -= u3[q];
      }
      __syncthreads();
      blk_store(r, k, R2);
      blk_store(r, r, R3);
      ps_publish(verA + r * nP + k, k);
      if (t == 0) flag_store(verA + r * nP + r, k);
    }
    return;
  }

  if (blockIdx.x == 2) {
    // ---------------- panel k-2 on row k+1 ----------------
    // Round k (2 <= k <= nP-2), r = k+1: from the workers' versions k-2 of (r, k-2 .. k) and (r, r)
    // (G for k = 2) and, once T_{k-2} is out, X_{k-1} = X slot k-2 and (k, k-2) (kept from the
    // previous round):
    //   X_r = (r, k-2) T_{k-2}^T,  X_k = (k, k-2) T_{k-2}^T,
    //   (r, k-1) -= X_r X_{k-1}^T,  (r, k) -= X_r X_k^T,  (r, r) -= X_r X_r^T,
    // published as version k-1 ((r, k-1) is also the workers' panel-(k-1) block).
    float(*T)[BP] = B0;
    float(*Xp)[BP] = B1;   // X_{k-1}
    float(*Kp)[BP] = B2;   // (k, k-2)
    float(*R0)[BP] = B3;
    float(*R1)[BP] = B4;
    float(*R2)[BP] = B5;
    float(*R3)[BP] = B6;
    for (int k = 2; k + 1 < nP; ++k) {
      const int r = k + 1;
      if (t == 0 && k >= 3) {
        const int* const f[4] = {verA + r * nP + (k - 2), verA + r * nP + (k - 1), verA + r * nP + k, verA + r * nP + r};
        const int v[4] = {k - 2, k - 2, k - 2, k - 2};
        ps_wait_all(a, f, v, 4);
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t src = k == 2 ? rG : rM;   // version k - 2
      ps_load_blk(R0, src, d, r, k - 2);
      ps_load_blk(R1, src, d, r, k - 1);
      ps_load_blk(R2, src, d, r, k);
      ps_load_blk(R3, src, d, r, r);
      if (k == 2) ps_load_blk(Kp, rG, d, 2, 0);
      if (t == 0) ps_wait(a, tflag, k - 1);
      __syncthreads();
      slot_load(T, rT, k - 2);
      slot_load(Xp, rX, k - 2);
      __syncthreads();
      const f32x4 xk = sw_mm(Kp, T, true);
      const f32x4 xr = sw_mm(R0, T, true);
      __syncthreads();
      sw_put(Kp, xk);
      sw_put(R0, xr);
      __syncthreads();
      const f32x4 u1 = sw_mm(R0, Xp, true);
      const f32x4 u2 = sw_mm(R0, Kp, true);
      const f32x4 u3 = sw_mm(R0, R0, true);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        R1[qm + q][qn] -= u1[q];
        R2[qm + q][qn] -= u2[q];
        R3[qm + q][qn] -= u3[q];
      }
      __syncthreads();
      blk_store(r, k - 1, R1);
      blk_store(r, k, R2);
      blk_store(r, r, R3);
      ps_publish(verA + r * nP + (k - 1), k - 1);
      if (t == 0) {
        flag_store(verA + r * nP + k, k - 1);
        flag_store(verA + r * nP + r, k - 1);
      }
      // (r, k-1) is the next round's (k, k-2)
      float(*f0)[BP] = Kp;
      Kp = R1;
      R1 = f0;
    }
    return;
  }

  // ---------------- workers ----------------
  float(*L0)[BP] = B0;
  float(*L1)[BP] = B1;
  float(*L2)[BP] = B2;
  for (;;) {
    if (t == 0) sq = __hip_atomic_fetch_add(a.st + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int q = sq;
    if (q >= a.n_tasks) return;
    int p = 0;
    bool rp = false;
    for (; p < nP; ++p) {
      const int c = ps_count(nP, p);
      if (q < c) break;
      q -= c;
      const int c2 = ps_rp_count(a.n_rp, a.rp_share, p);
      if (q < c2) {
        rp = true;
        break;
      }
      q -= c2;
    }
    if (p >= nP) return;   // (n_tasks is the sum of ps_count and ps_rp_count over the panels)
    if (rp) {
      // R / P block p * share + q
      uint16_t(*As)[64][RP_PITCH] = (uint16_t(*)[64][RP_PITCH]) & B0[0][0];
      uint16_t(*Bs)[64][RP_PITCH] = (uint16_t(*)[64][RP_PITCH]) & B1[0][0];
      if (a.wparts == 1) rp_tile<1>(a.sp, a.Rc, a.P, d, a.n_r, p * a.rp_share + q, As, Bs);
      else rp_tile<3>(a.sp, a.Rc, a.P, d, a.n_r, p * a.rp_share + q, As, Bs);
      __syncthreads();
      continue;
    }
    const int m = nP - 1 - p, nA = ps_n_a(m), nBt = m * (p + 1);
    const __amdgpu_buffer_rsrc_t srcP = p == 0 ? rG : rM;   // A blocks at version p
    const uint32_t toff = (uint32_t)(p * NB * NB * 4);
    auto load_t = [&]() {   // T_p into L2
      const int rr = t >> 4, c = (t & 15) * 4;
      *(f32x4*)&L2[rr][c] = sc1_ld4(rT, toff + (uint32_t)((rr * NB + c) * 4));
    };
    if (q < nA) {
      // A task: (i, j) -= X_i X_j^T, X = (., p) T_p^T
      int ii, jj;
      tri_decode(q + PS_CHAIN_ENTRIES, ii, jj);
      const int i = p + 1 + ii, j = p + 1 + jj;
      if (t == 0) {
        const int* const f[4] = {tflag, verA + i * nP + p, verA + j * nP + p, verA + i * nP + j};
        const int v[4] = {p + 1, p, p, p};
        ps_wait_all(a, f, v, 4);
      }
      __syncthreads();
      ps_load_blk(L0, srcP, d, i, p);
      load_t();
      if (i != j) ps_load_blk(L1, srcP, d, j, p);
      __syncthreads();
      const f32x4 xi = sw_mm(L0, L2, true);
      const f32x4 xj = i != j ? sw_mm(L1, L2, true) : xi;
      __syncthreads();
      sw_put(L0, xi);
      sw_put(L1, xj);
      __syncthreads();
      const f32x4 v = sw_mm(L0, L1, true);
      ps_store_blk(rM, srcP, d, i, j, -v, true);
      ps_publish(verA + i * nP + j, p + 1);
      continue;
    }
    q -= nA;
    if (q < nBt) {
      // B task: B_ic -= X_i (T_p B_pc), with B_pp = I and B_ic = 0 before its first update
      const int i = p + 1 + q / (p + 1), c = q % (p + 1);
      if (t == 0) {
        const int* const f[4] = {tflag, verA + i * nP + p, verB + p * nP + c, verB + i * nP + c};
        const int v[4] = {p + 1, p, p - c, p - c};
        ps_wait_all(a, f, v, c < p ? 4 : 2);
      }
      __syncthreads();
      ps_load_blk(L0, srcP, d, i, p);
      load_t();
      if (c < p) ps_load_blk(L1, rB, d, p, c);
      __syncthreads();
      const f32x4 xi = sw_mm(L0, L2, true);
      f32x4 tb;
      if (c < p) {
        tb = sw_mm(L2, L1, false);
      } else {
        const int lane = t & 63, wave = t >> 6;
        const int m0 = (wave >> 2) * 16 + 4 * (lane >> 4), n = (wave & 3) * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) tb[r] = L2[m0 + r][n];
      }
      __syncthreads();
      sw_put(L0, xi);
      sw_put(L1, tb);
      __syncthreads();
      const f32x4 v = sw_mm(L0, L1, false);
      ps_store_blk(rB, rB, d, i, c, -v, c < p);
      ps_publish(verB + i * nP + c, p - c + 1);
      continue;
    }
    q -= nBt;
    {
      // F task: L^-1 block (p, c) = T_p B_pc
      const int c = q;
      if (t == 0) {
        const int* const f[2] = {tflag, verB + p * nP + c};
        const int v[2] = {p + 1, p - c};
        ps_wait_all(a, f, v, 2);
      }
      __syncthreads();
      ps_load_blk(L1, rB, d, p, c);
      load_t();
      __syncthreads();
      const f32x4 v = sw_mm(L2, L1, false);
      sw_store(a.Linv, d, p, c, v, false);
      __syncthreads();
    }
  }
}

// Partial dot products for epsilon: <D,P>, <G,P>, <W,R>, <dW,R>, <dW,dW> (fp64 per block), row by row.
// Only the lower 64-block triangle of P is formed; D and G are symmetric, so blocks below the
// diagonal count twice and the upper ones are skipped.
template <typename WT>
__global__ __launch_bounds__(NT) void dots_kernel(const float* D, const float* G, const float* P,
                                                  const typename WT::storage* W, const float* R, const float* dW,
                                                  int d, double* part, Steps st) {
  D = at_layer(D, st.mat);
  G = at_layer(G, st.mat);
  dW = at_layer(dW, st.mat);
  P = at_layer(P, st.ws);
  W = at_layer(W, st.wmat);
  R = at_layer(R, st.ws);
  part = at_layer(part, st.ws);
  double s[5] = {0, 0, 0, 0, 0};
  for (int r = blockIdx.x; r < d; r += gridDim.x)
    for (int c = 4 * (int)threadIdx.x; c < d; c += 4 * NT) {
      const int64_t e = (int64_t)r * d + c;
      const f32x4 rv = *(const f32x4*)(R + e), dv = *(const f32x4*)(dW + e);
      f32x4 wv;
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[u] = Cvt<WT>::to_f(W[e + u]);
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

__global__ __launch_bounds__(NT) void eps_kernel(const double* part, int nblk, const Scalars* sc, float* eps,
                                                 Steps st) {
  part = at_layer(part, st.ws);
  sc = at_layer(sc, st.ws);
  eps = at_layer(eps, (int64_t)sizeof(float));
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
  float* Bx;   // d x d: I, then L^-1 (per-panel launches); the identity part as updated (one launch)
  float* Rs;   // d x d: refinement residual
  float* Rc;   // d x d
  float* P;    // d x d (W W^T)
  float* T;    // NB x NB slots, one per panel (at least three)
  Scalars* sc;
  double* part;
  void* rz;    // refinement residual: int8 digit planes of [C | -G] and [W ; dW] (residual_workspace_bytes)
  uint16_t* sp; // 9 d x d bf16: three parts of C, of W and of W^T (split_kernel)
  float* Linv; // d x d: L^-1 (one-launch sweep)
  float* Xs;   // NB x NB slots, one per panel (one-launch sweep)
  int* st;     // one-launch sweep: state and block versions
};

int n_panels(int d) { return (d + NB - 1) / NB; }
size_t t_slots_bytes(int d) { return (size_t)std::max(3, n_panels(d)) * NB * NB * sizeof(float); }
size_t state_bytes(int d) { return (size_t)(PS_STATE_INTS + 2 * n_panels(d) * n_panels(d)) * sizeof(int); }

WsLayout carve(void* ws, int d) {
  char* p = (char*)ws;
  const size_t dd = (size_t)d * d * sizeof(float);
  WsLayout w;
  w.Mx = (float*)p; p += dd;
  w.Bx = (float*)p; p += dd;
  w.Rs = (float*)p; p += dd;
  w.Rc = (float*)p; p += dd;
  w.P = (float*)p; p += dd;
  w.Linv = (float*)p; p += dd;
  w.T = (float*)p; p += t_slots_bytes(d);
  w.Xs = (float*)p; p += t_slots_bytes(d);
  w.sc = (Scalars*)p; p += 256;
  w.part = (double*)p; p += DOT_BLOCKS * 5 * sizeof(double);
  w.rz = p; p += (residual_workspace_bytes(d) + 255) / 256 * 256;
  w.st = (int*)p; p += (state_bytes(d) + 255) / 256 * 256;
  w.sp = (uint16_t*)p;
  return w;
}

// One auxiliary stream per device (default priority) and a fork and a join event: work that the
// sweep does not read runs beside it.  The mutex is held from the fork to the join so that calls
// from several host threads do not interleave their records and waits.
struct AuxStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
AuxStream g_aux[kMaxDevices];

// the device's auxiliary stream, created on first use; nullptr if it cannot be (the work then stays
// on the caller's stream)
AuxStream* aux_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  AuxStream& a = g_aux[dev];
  std::lock_guard<std::mutex> lock(a.mu);
  if (!a.tried) {
    a.tried = true;
    if (hipStreamCreateWithFlags(&a.st, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess)
      a.st = nullptr;
  }
  return a.st ? &a : nullptr;
}

#define ISPA_TRY(x)                      \
  do {                                   \
    hipError_t e_ = (x);                 \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

}  // namespace

size_t solve_workspace_bytes(int d) {
  const size_t b = (size_t)d * d * sizeof(float) * 6 + 2 * t_slots_bytes(d) + 256 + DOT_BLOCKS * 5 * sizeof(double) +
                   (residual_workspace_bytes(d) + 255) / 256 * 256 + (state_bytes(d) + 255) / 256 * 256 +
                   (size_t)d * d * 18 + 256;
  return (b + 255) / 256 * 256;
}

hipError_t launch_solve(const SolveLaunch& L, hipStream_t s) {
  const int d = L.d, nb_l = L.batch;
  WsLayout w = carve(L.ws, d);
  const int64_t dd = (int64_t)d * d;
  Steps st;
  st.ws = (int64_t)solve_workspace_bytes(d);
  st.mat = dd * (int64_t)sizeof(float);
  st.wmat = dd * (L.w_dtype == DT_F32 ? 4 : 2);
  st.batch = nb_l;
  const int eb = (int)((dd + NT - 1) / NT > 2048 ? 2048 : (dd + NT - 1) / NT);
  const dim3 eg(eb, nb_l);
  const int nP = n_panels(d);
  // One layer with few panels: the whole sweep in one launch (the trailing updates then fit beside
  // the diagonal chain); otherwise one launch per panel, with the layers side by side.
  const bool one_launch = nb_l == 1 && nP <= PS_MAX_PANELS;
  int* state = one_launch ? w.st : nullptr;
  const int n_state = PS_STATE_INTS + 2 * nP * nP;

  // Mx and Bx for the per-panel launches (the one-launch sweep reads G itself and starts the identity
  // part implicitly)
  if (!one_launch) {
    hipLaunchKernelGGL(setup_kernel, eg, dim3(NT), 0, s, L.G, d, w.Mx, w.Bx, st);
    ISPA_TRY(hipGetLastError());
  }

  // R = C W and, for epsilon, the lower block triangle of P = W W^T, from bf16 parts of C and W.
  // Nothing reads them before the triangular products.  Per-panel launches: they run on the
  // auxiliary stream beside the sweep, whose launches are latency-bound and leave most of the device
  // idle.  One launch: the parts are made first on the caller's stream and the blocks of R and P
  // are tasks of the sweep's queue, run by the workers while they would otherwise wait (beside the
  // sweep, kernels would share its CUs, the diagonal chain's included).
  AuxStream* ax = one_launch ? nullptr : aux_stream();
  std::unique_lock<std::mutex> aux_lock;
  hipStream_t sr = s;
  if (ax) {
    aux_lock = std::unique_lock<std::mutex>(ax->mu);
    ISPA_TRY(hipEventRecord(ax->fork, s));
    ISPA_TRY(hipStreamWaitEvent(ax->st, ax->fork, 0));
    sr = ax->st;
  }
  {
    const int nT = (d + 63) / 64, n_r = nT * nT, n_p = L.eps ? nT * (nT + 1) / 2 : 0;
    const dim3 sg(n_r, nb_l), rg(n_r + n_p, nb_l);
    // Layers with more panels than one launch takes: R and P on the projection's NT kernel, as
    // sums of products of the bf16 planes (C0 C1 C2 | W0 W1 W2 | W^T0 W^T1 W^T2), smallest terms first
    // (the same terms as rp_tile; P in the tiles that meet its lower block triangle, which is all that
    // epsilon reads).  Its 32-bit offsets span all planes up to d = 8192.
    const bool nt_rp = nP > PS_MAX_PANELS && d % 64 == 0 && d <= 8192;
    const bool bf16w = L.w_dtype == DT_BF16;
    if (bf16w) {
      hipLaunchKernelGGL((split_kernel<1, BF16>), sg, dim3(256), 0, sr, L.C, (const uint16_t*)L.W, w.sp, d, st, state,
                         n_state, L.info);
      if (!one_launch && !nt_rp) hipLaunchKernelGGL(rp_kernel<1>, rg, dim3(256), 0, sr, w.sp, w.Rc, w.P, d, n_r, st);
    } else {
      if (L.w_dtype == DT_F16)
        hipLaunchKernelGGL((split_kernel<3, F16>), sg, dim3(256), 0, sr, L.C, (const uint16_t*)L.W, w.sp, d, st,
                           state, n_state, L.info);
      else
        hipLaunchKernelGGL((split_kernel<3, F32>), sg, dim3(256), 0, sr, L.C, (const float*)L.W, w.sp, d, st, state,
                           n_state, L.info);
      if (!one_launch && !nt_rp) hipLaunchKernelGGL(rp_kernel<3>, rg, dim3(256), 0, sr, w.sp, w.Rc, w.P, d, n_r, st);
    }
    if (nt_rp) {
      ISPA_TRY(hipGetLastError());
      // R = C W: A planes C_i (0..2), B planes W^T_j (6..8), i + j <= 2; P = W W^T: planes W_i (3..5)
      if (bf16w) {
        ISPA_TRY(launch_nt_segments(w.sp, w.Rc, d, 3, 0x012, 0x666, nb_l, st.ws, false, sr));
        if (n_p) ISPA_TRY(launch_nt_segments(w.sp, w.P, d, 1, 0x3, 0x3, nb_l, st.ws, true, sr));
      } else {
        ISPA_TRY(launch_nt_segments(w.sp, w.Rc, d, 6, 0x010210, 0x667678, nb_l, st.ws, false, sr));
        if (n_p) ISPA_TRY(launch_nt_segments(w.sp, w.P, d, 6, 0x343543, 0x334345, nb_l, st.ws, true, sr));
      }
    }
    ISPA_TRY(hipGetLastError());
    if (ax) ISPA_TRY(hipEventRecord(ax->join, sr));
  }

  if (one_launch) {
    PsArgs a;
    a.G = L.G;
    a.Mx = w.Mx;
    a.Bx = w.Bx;
    a.Linv = w.Linv;
    a.Tb = w.T;
    a.Xs = w.Xs;
    a.st = w.st;
    a.info = L.info;
    a.sc = w.sc;
    a.lam = L.lambda;
    a.relative = L.lambda_relative;
    a.lambda_out = L.lambda_out;
    a.d = d;
    a.nP = nP;
    const int nT = (d + 63) / 64;
    a.sp = w.sp;
    a.Rc = w.Rc;
    a.P = w.P;
    a.wparts = L.w_dtype == DT_BF16 ? 1 : 3;
    a.n_r = nT * nT;
    a.n_rp = a.n_r + (L.eps ? nT * (nT + 1) / 2 : 0);
    a.rp_share = (a.n_rp + nP - 1) / nP;
    int n_tasks = 0;
    for (int p = 0; p < nP; ++p) n_tasks += ps_count(nP, p) + ps_rp_count(a.n_rp, a.rp_share, p);
    a.n_tasks = n_tasks;
    const int grid = 3 + std::min(PS_WORKERS, n_tasks);
    hipLaunchKernelGGL(psweep_kernel, dim3(grid), dim3(SW_THREADS), 0, s, a);
    ISPA_TRY(hipGetLastError());
  } else {
    // Cholesky sweep (one launch per panel, plus one that finishes the last two block rows of L^-1)
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
      a.sc = w.sc;
      a.G = L.G;
      a.lam = L.lambda;
      a.relative = L.lambda_relative;
      a.lambda_out = L.lambda_out;
      a.st = st;
      const int grid = (k < nP ? 1 : 0) + a.n_a + a.n_i + n_f;
      hipLaunchKernelGGL(sweep_kernel, dim3(grid, nb_l), dim3(SW_THREADS), 0, s, a);
      ISPA_TRY(hipGetLastError());
    }
  }
  if (ax) {
    ISPA_TRY(hipStreamWaitEvent(s, ax->join, 0));
    aux_lock.unlock();
  }
  const float* Li = one_launch ? w.Linv : w.Bx;   // L^-1
  // Z = L^-1 R (L^-1 lower triangular: only k < m0 + 64 contributes), into Mx (no longer needed)
  ISPA_TRY(run_trgemm(false, Li, st.ws, w.Rc, st.ws, w.Mx, st.ws, d, 1.f, 0.f, nb_l, s));
  // dW = (L^-1)^T Z   (op(A) upper triangular: only k >= m0 contributes)
  // (W_new = W + dW is written by the last product that updates dW)
  ISPA_TRY(run_trgemm(true, Li, st.ws, w.Mx, st.ws, L.delta_w, st.mat, d, 1.f, 0.f, nb_l, s, L.W,
                      L.refine > 0 ? nullptr : L.w_new, L.w_dtype, st.wmat));
  if (L.refine > 0) {
    // iterative refinement: r = C W - (G + lambda I) dW from exact int8 products of fixed-point digits
    // (refine.hip), then dW += (L^-1)^T (L^-1 r) with the fp32 factor
    for (int it = 0; it < L.refine; ++it) {
      ResidualLaunch R;
      R.batch = nb_l;
      R.d = d;
      R.C = L.C;
      R.G = L.G;
      R.W = L.W;
      R.w_dtype = L.w_dtype;
      R.dW = L.delta_w;
      R.lambda = &w.sc->lambda;
      R.r = w.Rs;
      R.ws = w.rz;
      R.rows_too = it == 0;
      R.s_mat = st.mat;
      R.s_wmat = st.wmat;
      R.s_ws = st.ws;
      R.s_lambda = st.ws;
      ISPA_TRY(launch_residual(R, s));
      // t = L^-1 r (into Mx, no longer needed), dW += (L^-1)^T t
      ISPA_TRY(run_trgemm(false, Li, st.ws, w.Rs, st.ws, w.Mx, st.ws, d, 1.f, 0.f, nb_l, s));
      ISPA_TRY(run_trgemm(true, Li, st.ws, w.Mx, st.ws, L.delta_w, st.mat, d, 1.f, 1.f, nb_l, s, L.W,
                          it + 1 == L.refine ? L.w_new : nullptr, L.w_dtype, st.wmat));
    }
  }
  if (L.eps) {
    if (L.w_dtype == DT_BF16)
      hipLaunchKernelGGL(dots_kernel<BF16>, dim3(DOT_BLOCKS, nb_l), dim3(NT), 0, s, L.D, L.G, w.P,
                         (const uint16_t*)L.W, w.Rc, L.delta_w, d, w.part, st);
    else if (L.w_dtype == DT_F16)
      hipLaunchKernelGGL(dots_kernel<F16>, dim3(DOT_BLOCKS, nb_l), dim3(NT), 0, s, L.D, L.G, w.P,
                         (const uint16_t*)L.W, w.Rc, L.delta_w, d, w.part, st);
    else
      hipLaunchKernelGGL(dots_kernel<F32>, dim3(DOT_BLOCKS, nb_l), dim3(NT), 0, s, L.D, L.G, w.P, (const float*)L.W,
                         w.Rc, L.delta_w, d, w.part, st);
    ISPA_TRY(hipGetLastError());
    hipLaunchKernelGGL(eps_kernel, dim3(1, nb_l), dim3(NT), 0, s, w.part, DOT_BLOCKS, w.sc, L.eps, st);
    ISPA_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace ispa
