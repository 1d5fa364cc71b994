// The L-layer projection out = A W_new (technical summary, section 2, stage 3 "Memory-Efficient
// Inference": converted layers attend locally and project with W + dW), for gfx950.
//
// One kernel serves the 16-bit product and the W8A8 (FP8 E4M3) product: both operands are stored
// contiguous along k -- A [m, k] row-major and W^T [n, k] -- so a 128-byte slice of a row is 64 bf16 /
// f16 values or 128 E4M3 codes, and the LDS layout, the loads and the epilogue are the same:
//  * 256 x 128 output tiles (one work-group per CU: 228 tiles at 4680 x 1536), work-groups of
//    12 waves: waves 0-7 multiply (4 x 2 of 64 x 64, 2 x 2 blocks of 32 x 32 MFMA each), waves 8-11
//    only issue loads -- a wave that issues a burst of direct-to-LDS loads stalls at issue until
//    the load path takes them, so loads and MFMAs belong to different waves;
//  * k in stages of 128 bytes per row (one load instruction fetches whole 128-byte lines of 8 rows:
//    L2 feeds a CU about twice as fast as with 64-byte halves of 16 rows) through a three-deep ring
//    of direct-to-LDS buffer loads issued two stages ahead; rows past the matrix fall outside the
//    tile's buffer range and read as zeros; 16-byte chunk c of row r sits at r*128 + 16 (c ^ ((r/2) % 8)),
//    so the 16 rows a quarter-wave reads at one chunk cover all 64 banks; every ring slot is its own
//    LDS array and the stage loop is unrolled by the ring depth, so each wait covers exactly the
//    stage it needs;
//  * per stage and multiplying wave: 16-bit: 16 v_mfma_f32_32x32x16 (lane l holds row l%32,
//    k = 8 (l/32) + 0..7 of a 16-deep step); FP8: 8 v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//    scales (k = 32 (l/32) + 0..31 of a 64-deep step), the fp32 result scaled by s_a[row] s_w[col] in
//    the epilogue; the fragments of the next k-step are read while the current one multiplies;
//  * the epilogue stages each wave's 64 x 64 part through 8 KiB of the idle ring and writes
//    16-byte pieces.
// At the full MFMA rate a CU takes 48 B/clk of operands from L2 and reads 128 B/clk of LDS.
// The 16-bit path gets W^T from transpose16_kernel (64 x 128 blocks through LDS) in the workspace.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace ispa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int NT_BK = 128;                   // bytes of a row per stage
constexpr int NT_ATILE = 256 * NT_BK;         // 32 KiB
constexpr int NT_BTILE = 128 * NT_BK;         // 16 KiB
constexpr int NT_ALOADS = NT_ATILE / 1024 / 4, NT_BLOADS = NT_BTILE / 1024 / 4;   // per loader: 8 and 4
constexpr int NT_LOADS = NT_ALOADS + NT_BLOADS;
__device__ __forceinline__ int nt_off(int row, int chunk) { return row * NT_BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// KIND 3 (segmented, for the solve's R = C W and P = W W^T): both operands are bf16 planes of one
// d x d row-major array of planes (a == b), and the k sequence is n_seg segments of d values, segment
// g pairing plane a_planes[g] of A with plane b_planes[g] of B (4 bits each); out is fp32 [m][n],
// written directly; layer blockIdx.y at a + layer * layer_bytes and out + layer * layer_bytes.
struct NtSeg {
  int n_seg, a_planes, b_planes;
  int64_t plane_bytes, layer_bytes;
  int lower;   // 1: only tiles that meet the lower triangle of 64 x 64 blocks (the others return)
};

// KIND 0: E4M3 codes (scaled epilogue); 1, 2: the 16-bit type TIn; 3: segmented (NtSeg).  TOut: type
// of out.  row_bytes: bytes of a row of either operand, a multiple of 128.
template <int KIND, typename TIn, typename TOut>
__global__ __launch_bounds__(768, 1) void gemm_nt_kernel(const uint8_t* a, const uint8_t* b, const float* sa,
                                                          const float* sw, void* out, int m, int n, int row_bytes,
                                                          int tiles_m, int tiles_n, NtSeg seg) {
  if constexpr (KIND == 3) {
    a += (int64_t)blockIdx.y * seg.layer_bytes;
    b = a;
    out = (char*)out + (int64_t)blockIdx.y * seg.layer_bytes;
  }
  __shared__ __attribute__((aligned(16))) uint8_t a0[NT_ATILE], a1[NT_ATILE], a2[NT_ATILE];
  __shared__ __attribute__((aligned(16))) uint8_t b0[NT_BTILE], b1[NT_BTILE], b2[NT_BTILE];
  __shared__ float sa_t[256], sw_t[128];
  // tiles of one 256-row block of A are consecutive, so the work-groups of one XCD share A rows
  const int logical = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int bm = logical / tiles_n, bn = logical % tiles_n;
  const int m0 = bm * 256, n0 = bn * 128;
  if constexpr (KIND == 3) {
    // the tile covers 64-blocks rows 4 bm .. 4 bm + 3 and columns 2 bn, 2 bn + 1
    if (seg.lower && 2 * bn > 4 * bm + 3) return;
  }
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
  const int seg_st = row_bytes / NT_BK;                            // stages per segment (KIND 3)
  const int n_st = KIND == 3 ? seg.n_seg * seg_st : row_bytes / NT_BK;

  // One barrier per stage: at barrier s, stage s is in LDS and the multipliers are done with stage
  // s - 1; the multipliers then run stage s while the loaders refill slot (s - 1) % 3 with stage s + 2
  // and wait for stage s + 1.
  if (wave >= 8) {
    const int w = wave - 8, t = tid - 512;
    if constexpr (KIND == 0) {
      sa_t[t] = m0 + t < m ? sa[m0 + t] : 0.f;
      if (t < 128) sw_t[t] = n0 + t < n ? sw[n0 + t] : 0.f;
    }
    // KIND 3: one buffer over all planes of the layer; rows past the matrix load zeros through an
    // out-of-range offset (the next plane follows them)
    const __amdgpu_buffer_rsrc_t ra = KIND == 3
        ? __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, (int)0xFFFFFFF0u, 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc((void*)(a + (int64_t)m0 * row_bytes), (short)0,
                                            min(256, m - m0) * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = KIND == 3
        ? __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, (int)0xFFFFFFF0u, 0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc((void*)(b + (int64_t)n0 * row_bytes), (short)0,
                                            min(128, n - n0) * row_bytes, 0x00020000);
    // load instruction i of a tile covers its rows 8 i .. 8 i + 7: lane l fills byte 16 l of that KiB,
    // i.e. row 8 i + l / 8 at physical chunk l % 8, which holds logical chunk (l % 8) ^ (4 (i % 2) + l / 16);
    // loader w issues A instructions 8 w .. 8 w + 7 and B instructions 4 w .. 4 w + 3
    uint32_t aoff[NT_ALOADS], boff[NT_BLOADS];
    bool ain[NT_ALOADS], bin[NT_BLOADS];
#pragma unroll
    for (int j = 0; j < NT_ALOADS; ++j) {
      const int i = NT_ALOADS * w + j, c = (lane & 7) ^ (4 * (i & 1) + (lane >> 4)), row = 8 * i + (lane >> 3);
      aoff[j] = (uint32_t)(((KIND == 3 ? m0 : 0) + row) * row_bytes) + 16u * c;
      ain[j] = KIND != 3 || m0 + row < m;
    }
#pragma unroll
    for (int j = 0; j < NT_BLOADS; ++j) {
      const int i = NT_BLOADS * w + j, c = (lane & 7) ^ (4 * (i & 1) + (lane >> 4)), row = 8 * i + (lane >> 3);
      boff[j] = (uint32_t)(((KIND == 3 ? n0 : 0) + row) * row_bytes) + 16u * c;
      bin[j] = KIND != 3 || n0 + row < n;
    }
    constexpr uint32_t kOutOfRange = KIND == 3 ? 0xFFFFFFF0u : 0x80000000u;
    auto issue = [&](uint8_t* as, uint8_t* bs, int st) {
      const bool ok = st < n_st;
      uint32_t ka = (uint32_t)st * NT_BK, kb = ka;
      if constexpr (KIND == 3) {
        const int g = ok ? st / seg_st : 0;
        const uint32_t k0 = (uint32_t)(st - g * seg_st) * NT_BK;
        ka = (uint32_t)(((seg.a_planes >> (4 * g)) & 15) * seg.plane_bytes) + k0;
        kb = (uint32_t)(((seg.b_planes >> (4 * g)) & 15) * seg.plane_bytes) + k0;
      }
#pragma unroll
      for (int j = 0; j < NT_ALOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(as + 1024 * (NT_ALOADS * w + j)), 16,
                                                 ok && ain[j] ? aoff[j] + ka : kOutOfRange, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NT_BLOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(bs + 1024 * (NT_BLOADS * w + j)), 16,
                                                 ok && bin[j] ? boff[j] + kb : kOutOfRange, 0, 0, 0);
    };
    issue(a0, b0, 0);
    issue(a1, b1, 1);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(NT_LOADS));
    barrier();
    auto lstep = [&](auto J, int st) {   // between barriers st and st + 1 (J = st % 3)
      constexpr int j = decltype(J)::value;
      issue(aslot(std::integral_constant<int, (j + 2) % 3>{}), bslot(std::integral_constant<int, (j + 2) % 3>{}), st + 2);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NT_LOADS));
      barrier();
    };
    for (int st = 0; st < n_st; st += 3) {
      lstep(std::integral_constant<int, 0>{}, st);
      lstep(std::integral_constant<int, 1>{}, st + 1);
      lstep(std::integral_constant<int, 2>{}, st + 2);
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
  // fragment rows 64 wm + 32 mi + l % 32 (A) and 64 wn + 32 ni + l % 32 (B); the swizzle depends on
  // the row only through bits 1-3 (the same for r and r + 32), so chunk c ^ c' sits at offset ^ 16 c'
  const int aoff = nt_off(64 * wm + (lane & 31), KIND == 0 ? 2 * hi : hi);
  const int boff = nt_off(64 * wn + (lane & 31), KIND == 0 ? 2 * hi : hi);
  barrier();
  auto mstep = [&](auto J) {   // between barriers st and st + 1 (J = st % 3)
    const uint8_t* as = aslot(J);
    const uint8_t* bs = bslot(J);
    if constexpr (KIND == 0) {
      // two 64-deep k-steps; lane l: chunks 4 kk + 2 hi and 4 kk + 2 hi + 1
      i32x8 af[2][2], bf[2][2];
      auto frags = [&](int kk, i32x8* fa, i32x8* fb) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const u32x4 lo = *(const u32x4*)(as + ((aoff ^ (kk << 6)) + 32 * mi * NT_BK));
          const u32x4 up = *(const u32x4*)(as + ((aoff ^ (kk << 6) ^ 16) + 32 * mi * NT_BK));
          fa[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const u32x4 lo = *(const u32x4*)(bs + ((boff ^ (kk << 6)) + 32 * ni * NT_BK));
          const u32x4 up = *(const u32x4*)(bs + ((boff ^ (kk << 6) ^ 16) + 32 * ni * NT_BK));
          fb[ni] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        }
      };
      frags(0, af[0], bf[0]);
      frags(1, af[1], bf[1]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[kk][mi], bf[kk][ni], acc[mi][ni], 0, 0, 0,
                                                                          127, 0, 127);
      // reads(0) reads(1) mfma(0) mfma(1)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    } else {
      // four 16-deep k-steps; lane l: chunk 2 kk + hi
      u32x4 af[2][2], bf[2][2];
      auto frags = [&](int kk, u32x4* fa, u32x4* fb) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) fa[mi] = *(const u32x4*)(as + ((aoff ^ (kk << 5)) + 32 * mi * NT_BK));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) fb[ni] = *(const u32x4*)(bs + ((boff ^ (kk << 5)) + 32 * ni * NT_BK));
      };
      frags(0, af[0], bf[0]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk + 1 < 4) frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16<TIn>(af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni]);
      }
      // reads(0) reads(1) mfma(0) reads(2) mfma(1) reads(3) mfma(2) mfma(3)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
    barrier();
  };
  // whole ring turns: stages past the last one hold zeros and add nothing
  for (int st = 0; st < n_st; st += 3) {
    mstep(std::integral_constant<int, 0>{});
    mstep(std::integral_constant<int, 1>{});
    mstep(std::integral_constant<int, 2>{});
  }
  barrier();                                   // the ring is idle
  if constexpr (KIND == 3) {
    // fp32 out, register r of lane l of block (mi, ni): row 64 wm + 32 mi + 8 (r / 4) + 4 (l / 32) + r % 4,
    // column 64 wn + 32 ni + l % 32
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = n0 + 64 * wn + 32 * ni + (lane & 31);
        if (col >= n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + 64 * wm + 32 * mi + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (row < m) ((float*)out)[(int64_t)row * n + col] = acc[mi][ni][r];
        }
      }
  } else {
    uint8_t* mine = (wave < 4 ? a0 : a1) + 8192 * (wave & 3);
    store_wave_tile_64<TOut>(acc, (char*)mine, (typename TOut::storage*)out, n, m0, n0, m, n, [&](int row, int col) {
      if constexpr (KIND == 0) return sa_t[row] * sw_t[col];
      else return 1.f;
    });
  }
}

// W [k, n] 16-bit row-major -> W^T [n, k]; k and n are multiples of 16.  A work-group moves a
// 64 (k) x 128 (n) block: thread t reads 8 columns of rows 2p and 2p + 1 (p = t / 16 and t / 16 + 16)
// and writes the eight (W[2p][j], W[2p + 1][j]) pairs to LDS as 32-bit words T[j][p]; then each
// thread of a pair writes 32 consecutive values of k of output row j from 16 words of T[j][.].
constexpr int TR_PITCH = 36;                  // words per LDS row: 16-byte aligned rows
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* w, int k, int n, uint16_t* wt) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * TR_PITCH];
  const int j0 = blockIdx.x * 128, i0 = blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int p = (t >> 4) + 16 * half, jc = 8 * (t & 15);
    const int i = i0 + 2 * p, j = j0 + jc;
    u32x4 r0 = u32x4{0, 0, 0, 0}, r1 = u32x4{0, 0, 0, 0};
    if (j < n) {
      if (i < k) r0 = *(const u32x4*)(w + (int64_t)i * n + j);
      if (i + 1 < k) r1 = *(const u32x4*)(w + (int64_t)(i + 1) * n + j);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(jc + 2 * e) * TR_PITCH + p] = (r0[e] & 0xFFFFu) | (r1[e] << 16);
      tile[(jc + 2 * e + 1) * TR_PITCH + p] = (r0[e] >> 16) | (r1[e] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  {
    const int jl = t >> 1, h = t & 1, j = j0 + jl, i = i0 + 32 * h;
    if (j < n && i < k) {
      const u32x4* src = (const u32x4*)(tile + jl * TR_PITCH + 16 * h);
      uint16_t* dst = wt + (int64_t)j * k + i;
      *(u32x4*)dst = src[0];
      *(u32x4*)(dst + 8) = src[1];
      if (i + 16 < k) {
        *(u32x4*)(dst + 16) = src[2];
        *(u32x4*)(dst + 24) = src[3];
      }
    }
  }
}

template <int KIND, typename TIn, typename TOut>
hipError_t launch_nt(const void* a, const void* b, const float* sa, const float* sw, void* out, int m, int n,
                     int row_bytes, hipStream_t s) {
  const int tm = (m + 255) / 256, tn = (n + 127) / 128;
  hipLaunchKernelGGL((gemm_nt_kernel<KIND, TIn, TOut>), dim3(tm * tn), dim3(768), 0, s, (const uint8_t*)a,
                     (const uint8_t*)b, sa, sw, out, m, n, row_bytes, tm, tn, NtSeg{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose16(const void* w, int k, int n, void* wt, hipStream_t s) {
  const dim3 gt((n + 127) / 128, (k + 63) / 64);
  hipLaunchKernelGGL(transpose16_kernel, gt, dim3(256), 0, s, (const uint16_t*)w, k, n, (uint16_t*)wt);
  return hipGetLastError();
}

hipError_t launch_proj_nt(int io, int m, int n, int k, const void* a, const void* bt, void* out, hipStream_t s) {
  if (io == DT_BF16) return launch_nt<1, BF16, BF16>(a, bt, nullptr, nullptr, out, m, n, k * 2, s);
  return launch_nt<2, F16, F16>(a, bt, nullptr, nullptr, out, m, n, k * 2, s);
}

hipError_t launch_proj(const ProjLaunch& L, hipStream_t s) {
  const hipError_t e = launch_transpose16(L.b, L.k, L.n, L.bt, s);
  if (e != hipSuccess) return e;
  return launch_proj_nt(L.io, L.m, L.n, L.k, L.a, L.bt, L.out, s);
}

hipError_t launch_nt_segments(const uint16_t* planes, float* out, int d, int n_seg, int a_planes, int b_planes,
                              int batch, int64_t layer_bytes, bool lower, hipStream_t s) {
  const int t = (d + 255) / 256, tn = (d + 127) / 128;
  NtSeg g;
  g.n_seg = n_seg;
  g.a_planes = a_planes;
  g.b_planes = b_planes;
  g.plane_bytes = (int64_t)d * d * 2;
  g.layer_bytes = layer_bytes;
  g.lower = lower ? 1 : 0;
  hipLaunchKernelGGL((gemm_nt_kernel<3, BF16, F32>), dim3(t * tn, batch), dim3(768), 0, s, (const uint8_t*)planes,
                     (const uint8_t*)planes, nullptr, nullptr, (void*)out, d, d, d * 2, t, tn, g);
  return hipGetLastError();
}

hipError_t launch_proj8(int out_dtype, const uint8_t* aq, const float* sa, const uint8_t* wq_t, const float* sw,
                        void* out, int m, int n, int k, hipStream_t s) {
  if (out_dtype == DT_BF16) return launch_nt<0, BF16, BF16>(aq, wq_t, sa, sw, out, m, n, k, s);
  return launch_nt<0, BF16, F16>(aq, wq_t, sa, sw, out, m, n, k, s);
}

}  // namespace ispa
