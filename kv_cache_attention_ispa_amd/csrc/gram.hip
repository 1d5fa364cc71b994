// Absorption statistics (gfx950).
//
// The closed-form absorption of the ISPA technical summary (gist.science,
// nl/pt), section 2, stage 2 "Layer Absorb", needs G = A_loc^T A_loc and
// C = A_loc^T (A_full - A_loc); the reconstruction error of "Dynamic layer
// selection" also needs D = dA^T dA.  They are sums over warmup tokens.  The
// dual-stream kernel writes A_loc and dA feature-major ([d, tokens]), so every
// statistic is a product X Y^T in which both operands are contiguous along the
// reduction (token) dimension: the MFMA operands are read as 16-byte rows.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int NT = 256;

// ------------------------------------------------------------------------------------------
// 16-bit Gram: out (+)= X Y^T, X/Y [d, ld] (rows = features), tokens [0, n).
// A work item is a 256 x 128 output tile (256 rows of X against 128 rows of Y): 8 multiplying
// waves as 4 x 2 of 64 x 64 and 4 loading waves.  G and D are symmetric: only tiles that meet the
// lower triangle run, each 128 x 128 block strictly below the diagonal is also stored transposed,
// and blocks above it are dropped.  Tokens stream through a 3-deep LDS ring of 64-token stages
// (128 bytes of every row: a load instruction fetches whole 128-byte lines of 8 rows, which is what
// lets L2 feed a CU at ~45-60 B/clk; 64-byte pieces of 16 rows get half that), filled by
// direct-to-LDS buffer loads issued two stages ahead.  At the full MFMA rate a CU takes 48 B/clk of
// operands from L2 and reads 128 B/clk of LDS.
// ------------------------------------------------------------------------------------------
constexpr int GB = 128;
constexpr int RK = 64;                      // tokens per Gram stage
constexpr int R_ROW = RK * 2;               // 128 bytes per staged row
constexpr int R_XTILE = 2 * GB * R_ROW;     // 256 rows of X: 32 KiB
constexpr int R_YTILE = GB * R_ROW;         // 128 rows of Y: 16 KiB
constexpr int R_XLOADS = R_XTILE / 1024 / 4, R_YLOADS = R_YTILE / 1024 / 4;   // per wave: 8 and 4
constexpr int R_LOADS = R_XLOADS + R_YLOADS;
constexpr int G_TPITCH = 36;                // floats per row of a transposed 32 x 32 block in LDS

// Gram ring layout: 16-byte chunk c (tokens 8 c .. 8 c + 7) of row r at r * 128 + 16 (c ^ ((r / 2) % 8)):
// the 16 rows read by one quarter-wave of a ds_read_b128 (same logical chunk) cover all 16 chunk
// positions of 256 bytes.
__device__ __forceinline__ int r_off(int row, int chunk) { return row * R_ROW + ((chunk ^ ((row >> 1) & 7)) << 4); }

struct GramArgs {
  const uint16_t* x[3];
  const uint16_t* y[3];
  float* out[3];
  int d, n, accumulate, n_sym, rb, cb;   // rb: 256-row blocks, cb: 128-column blocks
  int64_t ld;
};

// Item q -> statistic z (0 G, 1 C, 2 D), 256-row block bi, 128-column block bj.  Items are grouped
// by bi: min(2 bi + 2, cb) tiles of G, cb tiles of C, then D like G (when n_sym == 2).
__device__ __forceinline__ void gram_item(const GramArgs& a, int q, int& z, int& bi, int& bj) {
  int b = 0;
  for (;; ++b) {
    const int g = min(2 * b + 2, a.cb);
    const int per = a.cb + a.n_sym * g;
    if (q < per || b + 1 == a.rb) {
      if (q < g) { z = 0; bj = q; }
      else if (q < g + a.cb) { z = 1; bj = q - g; }
      else { z = 2; bj = q - g - a.cb; }
      bi = b;
      return;
    }
    q -= per;
  }
}

template <typename T>
__global__ __launch_bounds__(3 * NT) void gram16_kernel(GramArgs a) {
  __shared__ __attribute__((aligned(16))) char x0[R_XTILE], x1[R_XTILE], x2[R_XTILE];
  __shared__ __attribute__((aligned(16))) char y0[R_YTILE], y1[R_YTILE], y2[R_YTILE];
  int z, bi, bj;
  gram_item(a, xcd_remap(blockIdx.x, gridDim.x), z, bi, bj);
  const int i0 = bi * 2 * GB, j0 = bj * GB;
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto xslot = [&](auto J) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return x0;
    else if constexpr (j == 1) return x1;
    else return x2;
  };
  auto yslot = [&](auto J) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return y0;
    else if constexpr (j == 1) return y1;
    else return y2;
  };
  auto barrier = [&]() { lds_barrier(); };
  const int n_steps = (a.n + RK - 1) / RK;
  const int tail_step = (a.n & 7) ? (a.n - 1) / RK : -1;   // stage holding a partly valid chunk

  // Waves 8-11 load, waves 0-7 multiply.  A wave that issues a burst of direct-to-LDS loads waits at
  // issue until the CU's load path has taken them, so loads and MFMAs belong to different waves.
  // One barrier per stage: at barrier s, stage s is in LDS and the multipliers are done with stage
  // s - 1; then the multipliers run stage s while the loaders refill slot (s - 1) % 3 with stage
  // s + 2 and wait for stage s + 1.
  if (wave >= 8) {
    const int w = wave - 8;
    // raw buffers over the tile's rows of X and of Y (rows past d fall outside: zeros)
    const int64_t row_bytes = a.ld * 2;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.x[z] + (int64_t)i0 * a.ld), (short)0, (int)(min(2 * GB, a.d - i0) * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.y[z] + (int64_t)j0 * a.ld), (short)0, (int)(min(GB, a.d - j0) * row_bytes), 0x00020000);
    // Load instruction i of a tile covers its rows 8 i .. 8 i + 7: lane l fills byte 16 l of that KiB,
    // i.e. row 8 i + l / 8, physical chunk l % 8, which holds logical chunk (l % 8) ^ (4 (i % 2) + l / 16).
    // Loader w issues X instructions 8 w .. 8 w + 7 and Y instructions 4 w .. 4 w + 3.  A chunk is
    // loaded only if its first token is below n; an out-of-range offset makes the load return zeros
    // (tokens in [n, ld) are not data).
    uint32_t xoff[R_XLOADS], yoff[R_YLOADS];
    int lim[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) lim[p] = a.n - 8 * ((lane & 7) ^ (4 * p + (lane >> 4)));
#pragma unroll
    for (int j = 0; j < R_XLOADS; ++j) {
      const int i = R_XLOADS * w + j, c = (lane & 7) ^ (4 * (i & 1) + (lane >> 4));
      xoff[j] = (uint32_t)((8 * i + (lane >> 3)) * row_bytes) + 16u * c;
    }
#pragma unroll
    for (int j = 0; j < R_YLOADS; ++j) {
      const int i = R_YLOADS * w + j, c = (lane & 7) ^ (4 * (i & 1) + (lane >> 4));
      yoff[j] = (uint32_t)((8 * i + (lane >> 3)) * row_bytes) + 16u * c;
    }
    auto issue = [&](char* xs, char* ys, int step) {
      const int t0 = step * RK;
      const bool ok0 = t0 < lim[0], ok1 = t0 < lim[1];   // instruction parity 0 / 1
#pragma unroll
      for (int j = 0; j < R_XLOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(xs + 1024 * (R_XLOADS * w + j)), 16,
                                                 ((j & 1) ? ok1 : ok0) ? xoff[j] + 2u * t0 : 0x80000000u, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < R_YLOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void*)(ys + 1024 * (R_YLOADS * w + j)), 16,
                                                 ((j & 1) ? ok1 : ok0) ? yoff[j] + 2u * t0 : 0x80000000u, 0, 0, 0);
    };
    // Zero tokens n .. of the chunk that straddles n, after this wave's own loads of that stage have
    // landed.  Every row is zeroed by the wave that loaded it: X row r by loader r / 64 (thread r of
    // the loader waves), Y row r by loader r / 32 (its lanes 0-31).
    auto fix_tail = [&](char* xs, char* ys, int step) {
      const int t = tid - 4 * GB, t0 = step * RK, c = (a.n - t0) >> 3, e0 = (a.n - t0) & 7;
      char* bx = xs + r_off(t, c);
      const bool ylane = lane < 32;
      char* by = ys + r_off(32 * w + (lane & 31), c);
      for (int e = e0; e < 8; ++e) {
        *(uint16_t*)(bx + 2 * e) = 0;
        if (ylane) *(uint16_t*)(by + 2 * e) = 0;
      }
    };
    issue(x0, y0, 0);
    issue(x1, y1, 1);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(R_LOADS));
    if (tail_step == 0) fix_tail(x0, y0, 0);
    barrier();
    auto lstep = [&](auto J, int s) {   // between barriers s and s + 1 (J = s % 3)
      constexpr int j = decltype(J)::value;
      issue(xslot(std::integral_constant<int, (j + 2) % 3>{}), yslot(std::integral_constant<int, (j + 2) % 3>{}), s + 2);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(R_LOADS));
      if (s + 1 == tail_step) fix_tail(xslot(std::integral_constant<int, (j + 1) % 3>{}),
                                       yslot(std::integral_constant<int, (j + 1) % 3>{}), s + 1);
      barrier();
    };
    for (int s = 0; s < n_steps; s += 3) {
      lstep(std::integral_constant<int, 0>{}, s);
      lstep(std::integral_constant<int, 1>{}, s + 1);
      lstep(std::integral_constant<int, 2>{}, s + 2);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // loads past the last stage (zeros) have landed
    barrier();                                   // the ring is idle
    return;
  }

  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // per-lane read offsets: A fragment m = X rows 64 wm + 32 m + l % 32, B fragment m = Y rows
  // 64 wn + 32 m + l % 32, chunk 2 kk + l / 32.  The swizzle term depends on the row only through
  // bits 1-3, the same for rows r and r + 32 m, and chunk 2 kk + h = h ^ 2 kk: offset(kk) = offset(0) ^ 32 kk.
  const int aoff = r_off(64 * wm + (lane & 31), hi);
  const int boff = r_off(64 * wn + (lane & 31), hi);
  barrier();
  // fragments of k-step kk + 1 are read while the MFMAs of k-step kk run
  auto mstep = [&](auto J) {   // between barriers s and s + 1 (J = s % 3)
    const char* xs = xslot(J);
    const char* ys = yslot(J);
    u32x4 af[2][2], bf[2][2];
    auto frags = [&](int kk, u32x4* fa, u32x4* fb) {
#pragma unroll
      for (int m = 0; m < 2; ++m) fa[m] = *(const u32x4*)(xs + (aoff ^ (kk << 5)) + 32 * m * R_ROW);
#pragma unroll
      for (int m = 0; m < 2; ++m) fb[m] = *(const u32x4*)(ys + (boff ^ (kk << 5)) + 32 * m * R_ROW);
    };
    frags(0, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < RK / 16; ++kk) {
      if (kk + 1 < RK / 16) frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16<T>(af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni]);
    }
    // order for the scheduler: reads(0) reads(1) mfma(0) reads(2) mfma(1) reads(3) mfma(2) mfma(3)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < RK / 16; ++kk) {
      if (kk + 1 < RK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    barrier();
  };
  // whole ring turns: stages past the last token hold zeros and add nothing
  for (int s = 0; s < n_steps; s += 3) {
    mstep(std::integral_constant<int, 0>{});
    mstep(std::integral_constant<int, 1>{});
    mstep(std::integral_constant<int, 2>{});
  }
  barrier();                                   // the ring is idle

  // this wave's 64 x 64 block lies in the 128 x 128 block (rb, bj), rb = 2 bi + wm / 2
  const int rb = 2 * bi + (wm >> 1);
  if (z != 1 && rb < bj) return;                // above the diagonal of G or D
  const bool mirror = z != 1 && rb > bj;
  float* out = a.out[z];
  // transposed copies go through this wave's 4.5 KiB of the (now idle) ring
  float* tb = (float*)((wave < 4 ? x0 : x1) + (wave & 3) * (G_TPITCH * 32 * 4));
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = j0 + 64 * wn + 32 * ni + (lane & 31);
      const int rowb = i0 + 64 * wm + 32 * mi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rowb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < a.d && col < a.d) {
          float* o = out + (int64_t)row * a.d + col;
          *o = a.accumulate ? *o + acc[mi][ni][r] : acc[mi][ni][r];
        }
      }
      if (mirror) {
        // block^T: LDS row c (= column col of the block) holds its 32 rows; lane l writes rows
        // 8 q + 4 hi .. +3 of column l % 32, then reads back 4 consecutive rows of column
        // 8 e + l / 8 (e = 0..3) and stores them to out[col][row .. row + 3]
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)(tb + (lane & 31) * G_TPITCH + 8 * q + 4 * hi) =
              f32x4{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        wave_lds_order();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 8 * e + (lane >> 3), r4 = 4 * (lane & 7);
          const f32x4 v = *(const f32x4*)(tb + c * G_TPITCH + r4);
          const int orow = j0 + 64 * wn + 32 * ni + c, ocol = rowb + r4;
          if (orow < a.d && ocol < a.d) {
            float* o = out + (int64_t)orow * a.d + ocol;
            *(f32x4*)o = a.accumulate ? *(const f32x4*)o + v : v;
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        wave_lds_order();   // these reads stay ahead of the next block's writes
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
    a.rb = (L.d + 2 * GB - 1) / (2 * GB);
    a.cb = (L.d + GB - 1) / GB;
    a.n_sym = nz - 1;
    int items = 0;
    for (int b = 0; b < a.rb; ++b) items += a.cb + a.n_sym * std::min(2 * b + 2, a.cb);
    if (L.stat == DT_BF16)
      hipLaunchKernelGGL(gram16_kernel<BF16>, dim3(items), dim3(3 * NT), 0, s, a);
    else
      hipLaunchKernelGGL(gram16_kernel<F16>, dim3(items), dim3(3 * NT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ispa
