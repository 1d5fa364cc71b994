// Absorption statistics and the local-layer projection (gfx950).
//
// The closed-form absorption of the ISPA technical summary (gist.science,
// nl/pt), section 2, stage 2 "Layer Absorb", needs G = A_loc^T A_loc and
// C = A_loc^T (A_full - A_loc); the reconstruction error of "Dynamic layer
// selection" also needs D = dA^T dA.  They are sums over warmup tokens.  The
// dual-stream kernel writes A_loc and dA feature-major ([d, tokens]), so every
// statistic is a product X Y^T in which both operands are contiguous along the
// reduction (token) dimension: the MFMA operands are read as 16-byte rows.
//
// Stage 3 "Memory-Efficient Inference" projects the local attention output by
// W_new = W + dW: a plain row-major GEMM whose B operand is read through the
// transposing LDS load.
#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int NT = 256;

// ------------------------------------------------------------------------------------------
// 16-bit Gram: out (+)= X Y^T, X/Y [d, ld] (rows = features), tokens [0, n).
// 128 x 128 output tile per work-group, 4 waves as 2 x 2 of 64 x 64, k-step 32 tokens.
// ------------------------------------------------------------------------------------------
constexpr int GB = 128;
constexpr int GK = 32;
constexpr int G_ROW = GK * 2;               // 64 bytes per row of a staged tile
constexpr int G_TILE = GB * G_ROW;          // 8 KiB
constexpr int G_STAGE = 2 * G_TILE;

__device__ __forceinline__ int g_off(int row, int chunk) { return row * G_ROW + ((chunk ^ ((row >> 1) & 3)) << 4); }

struct GramArgs {
  const uint16_t* x[3];
  const uint16_t* y[3];
  float* out[3];
  int d, n, accumulate, tiles_per_dim;
  int64_t ld;
};

__device__ __forceinline__ u32x4 load_tok8(const uint16_t* row, int t0, int n) {
  if (t0 + 8 <= n) return *(const u32x4*)(row + t0);
  uint16_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = (t0 + j < n) ? row[t0 + j] : (uint16_t)0;
  return u32x4{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16),
               (uint32_t)e[4] | ((uint32_t)e[5] << 16), (uint32_t)e[6] | ((uint32_t)e[7] << 16)};
}

template <typename T>
__global__ __launch_bounds__(NT, 2) void gram16_kernel(GramArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * G_STAGE];
  const int z = blockIdx.y;
  const int tiles = a.tiles_per_dim * a.tiles_per_dim;
  const int logical = xcd_remap(blockIdx.x, tiles);
  const int bi = logical / a.tiles_per_dim, bj = logical % a.tiles_per_dim;
  const int i0 = bi * GB, j0 = bj * GB;
  const uint16_t* X = a.x[z];
  const uint16_t* Y = a.y[z];
  float* out = a.out[z];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int n_steps = (a.n + GK - 1) / GK;
  u32x4 xr[2], yr[2];
  auto gload = [&](int step) {
    const int t0 = step * GK + (tid & 3) * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 2) + 64 * i;
      xr[i] = (i0 + row < a.d) ? load_tok8(X + (int64_t)(i0 + row) * a.ld, t0, a.n) : u32x4{0, 0, 0, 0};
      yr[i] = (j0 + row < a.d) ? load_tok8(Y + (int64_t)(j0 + row) * a.ld, t0, a.n) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](char* st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 2) + 64 * i;
      *(u32x4*)(st + g_off(row, tid & 3)) = xr[i];
      *(u32x4*)(st + G_TILE + g_off(row, tid & 3)) = yr[i];
    }
  };
  gload(0);
  sstore(lds);
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    char* st = lds + (s & 1) * G_STAGE;
    const bool nxt = s + 1 < n_steps;
    if (nxt) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = *(const u32x4*)(st + g_off(64 * wm + 32 * mi + (lane & 31), 2 * kk + hi));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *(const u32x4*)(st + G_TILE + g_off(64 * wn + 32 * ni + (lane & 31), 2 * kk + hi));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16<T>(af[mi], bf[ni], acc[mi][ni]);
    }
    if (nxt) sstore(lds + ((s + 1) & 1) * G_STAGE);
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = j0 + 64 * wn + 32 * ni + (lane & 31);
      if (col >= a.d) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + 64 * wm + 32 * mi + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row >= a.d) continue;
        float* o = out + (int64_t)row * a.d + col;
        *o = a.accumulate ? *o + acc[mi][ni][r] : acc[mi][ni][r];
      }
    }
}

// fp32 Gram (small problems): VALU, 64 x 64 tile, 4 x 4 outputs per thread, k-step 16.
__global__ __launch_bounds__(NT) void gram32_kernel(GramArgs a) {
  __shared__ float xs[16][65];
  __shared__ float ys[16][65];
  const int z = blockIdx.y;
  const int tpd = (a.d + 63) / 64;
  const int bi = blockIdx.x / tpd, bj = blockIdx.x % tpd;
  const int i0 = bi * 64, j0 = bj * 64;
  const float* X = (const float*)a.x[z];
  const float* Y = (const float*)a.y[z];
  float* out = a.out[z];
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  float acc[4][4] = {};
  for (int t0 = 0; t0 < a.n; t0 += 16) {
    __syncthreads();
    for (int e = tid; e < 64 * 16; e += NT) {
      const int r = e / 16, t = e % 16;
      const bool ok = t0 + t < a.n;
      xs[t][r] = (ok && i0 + r < a.d) ? X[(int64_t)(i0 + r) * a.ld + t0 + t] : 0.f;
      ys[t][r] = (ok && j0 + r < a.d) ? Y[(int64_t)(j0 + r) * a.ld + t0 + t] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(xs[t][ti * 4 + u], ys[t][tj * 4 + w], acc[u][w]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int row = i0 + ti * 4 + u, col = j0 + tj * 4 + w;
      if (row < a.d && col < a.d) {
        float* o = out + (int64_t)row * a.d + col;
        *o = a.accumulate ? *o + acc[u][w] : acc[u][w];
      }
    }
}

// ------------------------------------------------------------------------------------------
// 16-bit projection out[m, n] = A[m, :] @ B[:, n], A [M, K], B [K, N] row-major, fp32 accumulate.
// 128 x 128 tile, k-step 32; the B operand comes from the row-major tile via transposing reads.
// ------------------------------------------------------------------------------------------
constexpr int P_BROW = 128 * 2;            // B tile row: 128 columns, 256 bytes
constexpr int P_ATILE = 128 * G_ROW;       // A tile: 128 rows x 32 k
constexpr int P_BTILE = GK * P_BROW;       // B tile: 32 rows x 128 n
constexpr int P_STAGE = P_ATILE + P_BTILE;

__device__ __forceinline__ int b_swz(int row) { return ((row & 3) << 2) | (((row >> 3) & 1) << 1); }
__device__ __forceinline__ int b_off(int row, int chunk) { return row * P_BROW + ((chunk ^ b_swz(row)) << 4); }

struct ProjArgs {
  const uint16_t* a;
  const uint16_t* b;
  uint16_t* out;
  int m, n, k, tiles_m, tiles_n;
};

template <typename T>
__global__ __launch_bounds__(NT, 2) void proj16_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * P_STAGE];
  const int logical = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  const int bn = logical / p.tiles_m, bm = logical % p.tiles_m;   // column-block major: B tile reuse per XCD
  const int m0 = bm * 128, n0 = bn * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, i16 = lane & 15;

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  u32x4 ar[2], br[2];
  auto gload = [&](int step) {
    const int k0 = step * GK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 2) + 64 * i;            // A: 128 rows x 4 chunks
      ar[i] = (m0 + row < p.m) ? *(const u32x4*)(p.a + (int64_t)(m0 + row) * p.k + k0 + (tid & 3) * 8)
                               : u32x4{0, 0, 0, 0};
      const int brow = (tid >> 4) + 16 * i;           // B: 32 rows x 16 chunks
      const int bcol = n0 + (tid & 15) * 8;
      br[i] = (bcol < p.n) ? *(const u32x4*)(p.b + (int64_t)(k0 + brow) * p.n + bcol) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](char* st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(u32x4*)(st + g_off((tid >> 2) + 64 * i, tid & 3)) = ar[i];
      *(u32x4*)(st + P_ATILE + b_off((tid >> 4) + 16 * i, tid & 15)) = br[i];
    }
  };
  const int n_steps = p.k / GK;
  gload(0);
  sstore(lds);
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    char* st = lds + (s & 1) * P_STAGE;
    const bool nxt = s + 1 < n_steps;
    if (nxt) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = *(const u32x4*)(st + g_off(64 * wm + 32 * mi + (lane & 31), 2 * kk + hi));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        u32x2 h[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int row = 16 * kk + 8 * (g >> 1) + 4 * half + (i16 >> 2);
          const int col = 64 * wn + 32 * ni + 16 * (g & 1) + 4 * (i16 & 3);
          const int off = row * P_BROW + (((col >> 3) ^ b_swz(row)) << 4) + 2 * (col & 7);
          h[half] = lds_read_tr16((const lds_void*)(st + P_ATILE + off));
        }
        bf[ni] = u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16<T>(af[mi], bf[ni], acc[mi][ni]);
    }
    if (nxt) sstore(lds + ((s + 1) & 1) * P_STAGE);
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + 64 * wn + 32 * ni + (lane & 31);
      if (col >= p.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 64 * wm + 32 * mi + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < p.m) p.out[(int64_t)row * p.n + col] = Cvt<T>::from_f(acc[mi][ni][r]);
      }
    }
}

}  // namespace

hipError_t launch_gram(const GramLaunch& L, hipStream_t s) {
  GramArgs a;
  a.x[0] = (const uint16_t*)L.a_t;  a.y[0] = (const uint16_t*)L.a_t;  a.out[0] = L.G;
  a.x[1] = (const uint16_t*)L.a_t;  a.y[1] = (const uint16_t*)L.da_t; a.out[1] = L.C;
  a.x[2] = (const uint16_t*)L.da_t; a.y[2] = (const uint16_t*)L.da_t; a.out[2] = L.D;
  a.d = L.d;
  a.n = L.n;
  a.ld = L.ld;
  a.accumulate = L.accumulate;
  const int nz = L.D ? 3 : 2;
  if (L.stat == DT_F32) {
    const int tpd = (L.d + 63) / 64;
    hipLaunchKernelGGL(gram32_kernel, dim3(tpd * tpd, nz), dim3(NT), 0, s, a);
  } else {
    a.tiles_per_dim = (L.d + GB - 1) / GB;
    dim3 grid(a.tiles_per_dim * a.tiles_per_dim, nz);
    if (L.stat == DT_BF16)
      hipLaunchKernelGGL(gram16_kernel<BF16>, grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL(gram16_kernel<F16>, grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_proj(const ProjLaunch& L, hipStream_t s) {
  ProjArgs p;
  p.a = (const uint16_t*)L.a;
  p.b = (const uint16_t*)L.b;
  p.out = (uint16_t*)L.out;
  p.m = L.m;
  p.n = L.n;
  p.k = L.k;
  p.tiles_m = (L.m + 127) / 128;
  p.tiles_n = (L.n + 127) / 128;
  dim3 grid(p.tiles_m * p.tiles_n);
  if (L.io == DT_BF16)
    hipLaunchKernelGGL(proj16_kernel<BF16>, grid, dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(proj16_kernel<F16>, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ispa
