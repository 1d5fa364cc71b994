// W8A8 (FP8 E4M3) variant of the L-layer projection for gfx950.
//
// The ISPA pages pair the converted layers with W8A8 post-training quantisation (technical summary,
// section 4 "Results") without naming a scheme.  Reading taken here: symmetric absmax scales per
// output channel of W and per token of the activations, codes in the OCP FP8 E4M3 format (the format
// of gfx950's f8f6f4 matrix instructions and of v_cvt_pk_fp8_f32):
//   s = absmax / 448 (float32; 1 for an all-zero channel), code = E4M3(clamp(x / s, -448, 448)),
//   out[i, j] = s_a[i] s_w[j] sum_k dec(Aq[i, k]) dec(Wq[k, j]) with fp32 accumulation.
// x / s is an IEEE float32 division and the conversion rounds to nearest even, so every code is
// decided in float32.  The conversion instruction does not saturate (values past 464 become NaN),
// hence the explicit clamp.
//
// Kernels:
//  * quant_rows_kernel: one wave per row of a [rows, cols] matrix (16-bit or fp32): absmax, scale,
//    codes written row-major -- the activations, token by token;
//  * wq_colmax_kernel, wq_scale_kernel, wq_quant_kernel: the weights per output channel (block maxima,
//    scales, codes), written transposed
//    (Wq^T [d_out, d_in]) so that both operands of the product are contiguous along k;
//  * proj8_kernel: out = (Aq Wq) * s_a s_w^T on v_mfma_scale_f32_32x32x64_f8f6f4 (block scales set
//    to 1), 128 x 128 tiles of 4 waves, k in 64-deep stages through a four-deep ring of direct-to-LDS
//    loads issued three stages ahead.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace ispa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
constexpr float kE4M3Max = 448.f;

template <typename T> __device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  return Cvt<T>::to_f(((const typename T::storage*)p)[i]);
}

// four codes of four values already divided by their scale, packed low to high
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float e4m3_scale(float amax) { return amax > 0.f ? amax / kE4M3Max : 1.f; }

// ---- activations: one wave per row, 8 consecutive values per lane and step ----
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* x, int64_t ldx, int rows, int cols, uint8_t* q,
                                                         int64_t ldq, float* scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = (int64_t)row * ldx;
  float amax = 0.f;
  for (int c = 8 * lane; c < cols; c += 512)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(ld_elem<T>(x, base + c + e)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float s = e4m3_scale(amax);
  if (lane == 0) scales[row] = s;
  for (int c = 8 * lane; c < cols; c += 512) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ld_elem<T>(x, base + c + e) / s;
    *(u32x2*)(q + (int64_t)row * ldq + c) = u32x2{e4m3_pack4(v[0], v[1], v[2], v[3]), e4m3_pack4(v[4], v[5], v[6], v[7])};
  }
}

// ---- weights: per output channel (column j of W [d_in, d_out]) ----
// pass 1: the column maxima of each 64 x 64 block (coalesced 64-column row segments), written to
// part[i0 / 64][j] (scratch space inside the code buffer, overwritten by pass 3)
template <typename T>
__global__ __launch_bounds__(256) void wq_colmax_kernel(const void* w, int d_in, int d_out, float* part) {
  __shared__ float red[4][64];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + c, i0 = blockIdx.y * 64;
  float amax = 0.f;
  if (col < d_out)
    for (int i = i0 + r; i < min(i0 + 64, d_in); i += 4) amax = fmaxf(amax, fabsf(ld_elem<T>(w, (int64_t)i * d_out + col)));
  red[r][c] = amax;
  __syncthreads();
  if (r == 0 && col < d_out)
    part[(int64_t)blockIdx.y * d_out + col] = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
}
// pass 2: the scale of each column from its block maxima
__global__ __launch_bounds__(256) void wq_scale_kernel(const float* part, int n_part, int d_out, float* scales) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= d_out) return;
  float amax = 0.f;
  for (int b = 0; b < n_part; ++b) amax = fmaxf(amax, part[(int64_t)b * d_out + col]);
  scales[col] = e4m3_scale(amax);
}

// 64 x 64 blocks: read W[i0.., j0..] row-major, write the codes of W^T[j0.., i0..] through LDS
template <typename T>
__global__ __launch_bounds__(256) void wq_quant_kernel(const void* w, int d_in, int d_out, const float* scales,
                                                       uint8_t* wq_t) {
  __shared__ uint8_t tile[64][64 + 4];
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  // each thread: 4 values of one row i (columns 4(t%16) .. +3), rows t/16 and t/16 + 16, +32, +48
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = i0 + (t >> 4) + 16 * rr, jc = 4 * (t & 15);
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + jc + e;
      v[e] = (i < d_in && j < d_out) ? ld_elem<T>(w, (int64_t)i * d_out + j) / scales[j] : 0.f;
    }
    const uint32_t code = e4m3_pack4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[jc + e][(t >> 4) + 16 * rr] = (uint8_t)(code >> (8 * e));
  }
  __syncthreads();
  // write: row j of W^T, 64 codes = 16 threads x 4 bytes
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int jl = (t >> 4) + 16 * rr, il = 4 * (t & 15);
    const int j = j0 + jl, i = i0 + il;
    if (j < d_out && i < d_in)
      *(uint32_t*)(wq_t + (int64_t)j * d_in + i) =
          (uint32_t)tile[jl][il] | ((uint32_t)tile[jl][il + 1] << 8) | ((uint32_t)tile[jl][il + 2] << 16) |
          ((uint32_t)tile[jl][il + 3] << 24);
  }
}

// ---- out = (Aq Wq) s_a s_w^T ----
// A operand: lane l holds Aq[m0 + l%32][k0 + 32 (l/32) + 0..31] (32 codes, 8 dwords); B operand:
// lane l holds Wq^T[n0 + l%32][k0 + 32 (l/32) + 0..31]; accumulator register r of lane l is
// out[8 (r/4) + 4 (l/32) + r%4][l%32] of the 32 x 32 block.  A stage is k0 .. k0 + 63 of 128 rows of
// each operand, 64-byte LDS rows; 16-byte chunk c of row r sits at r*64 + 16 (c ^ ((r >> 2) & 3)), so
// the 16 rows a quarter-wave reads at one chunk hit 16 distinct 16-byte bank groups.  Stages stream
// through a four-deep ring with direct-to-LDS buffer loads issued three stages ahead (a 1 KiB load
// instruction covers 16 rows; lane l fills byte 16 l, i.e. row 16 i + l/4 at swizzled position l%4,
// so it loads logical chunk (l%4) ^ ((row >> 2) & 3)).  Every ring slot is its own LDS array and the
// stage loop is unrolled by the ring depth, so each wait covers exactly the stage it needs.
constexpr int P8_BK = 64;                        // k per stage (one MFMA)
constexpr int P8_TILE = 128 * P8_BK;             // bytes of one operand stage
__device__ __forceinline__ int p8_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <typename T>
__global__ __launch_bounds__(256, 2) void proj8_kernel(const uint8_t* aq, const float* sa, const uint8_t* wq_t,
                                                        const float* sw, void* out, int m, int n, int k, int tiles_m,
                                                        int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t a0[P8_TILE], a1[P8_TILE], a2[P8_TILE], a3[P8_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t b0[P8_TILE], b1[P8_TILE], b2[P8_TILE], b3[P8_TILE];
  const int logical = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int bn = logical / tiles_m, bm = logical % tiles_m;
  const int m0 = bm * 128, n0 = bn * 128;
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // rows past m (n) read past the end of the buffer: zeros
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, m * k, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)wq_t, (short)0, n * k, 0x00020000);
  // wave w issues A instructions 2w, 2w + 1 and B instructions 2w, 2w + 1 of a stage
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    aoff[j] = (m0 + row < m) ? (uint32_t)((m0 + row) * k + 16 * c) : 0x80000000u;
    boff[j] = (n0 + row < n) ? (uint32_t)((n0 + row) * k + 16 * c) : 0x80000000u;
  }
  const int n_st = k / P8_BK;
  auto issue = [&](uint8_t* as, uint8_t* bs, int st) {
    const bool ok = st < n_st;
    const uint32_t k0 = (uint32_t)st * P8_BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(as + 1024 * (2 * wave + j)), 16,
                                               ok && aoff[j] != 0x80000000u ? aoff[j] + k0 : 0x80000000u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(bs + 1024 * (2 * wave + j)), 16,
                                               ok && boff[j] != 0x80000000u ? boff[j] + k0 : 0x80000000u, 0, 0, 0);
    }
  };
  auto aslot = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return a0;
    else if constexpr (j == 1) return a1;
    else if constexpr (j == 2) return a2;
    else return a3;
  };
  auto bslot = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return b0;
    else if constexpr (j == 1) return b1;
    else if constexpr (j == 2) return b2;
    else return b3;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  issue(a0, b0, 0);
  issue(a1, b1, 1);
  issue(a2, b2, 2);
  // stage s (slot J = s % 4): wait for its loads, barrier, refill slot (s + 3) % 4, then 4 MFMAs
  auto step = [&](auto J, int st) {
    constexpr int j = decltype(J)::value;
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(8));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(aslot(std::integral_constant<int, (j + 3) % 4>{}), bslot(std::integral_constant<int, (j + 3) % 4>{}), st + 3);
    const uint8_t* as = aslot(J);
    const uint8_t* bs = bslot(J);
    i32x8 af[2], bf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int row = 64 * wm + 32 * mi + (lane & 31);
      const u32x4 lo = *(const u32x4*)(as + p8_off(row, 2 * hi)), h4 = *(const u32x4*)(as + p8_off(row, 2 * hi + 1));
      af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)h4[0], (int)h4[1], (int)h4[2], (int)h4[3]};
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int row = 64 * wn + 32 * ni + (lane & 31);
      const u32x4 lo = *(const u32x4*)(bs + p8_off(row, 2 * hi)), h4 = *(const u32x4*)(bs + p8_off(row, 2 * hi + 1));
      bf[ni] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)h4[0], (int)h4[1], (int)h4[2], (int)h4[3]};
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf[ni], acc[mi][ni], 0, 0, 0, 127, 0, 127);
  };
  for (int st = 0; st < n_st; st += 4) {
    step(std::integral_constant<int, 0>{}, st);
    step(std::integral_constant<int, 1>{}, st + 1);
    step(std::integral_constant<int, 2>{}, st + 2);
    step(std::integral_constant<int, 3>{}, st + 3);
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // loads past the last stage (zeros) have landed
  // per-row and per-column scales of the tile; then each wave's part through its own ring slot
  __shared__ float sa_t[128], sw_t[128];
  if (tid < 128) sa_t[tid] = m0 + tid < m ? sa[m0 + tid] : 0.f;
  else sw_t[tid - 128] = n0 + tid - 128 < n ? sw[n0 + tid - 128] : 0.f;
  __syncthreads();
  uint8_t* mine = wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? a2 : a3;
  store_wave_tile_64<T>(acc, (char*)mine, (typename T::storage*)out, n, m0, n0, m, n,
                        [&](int row, int col) { return sa_t[row] * sw_t[col]; });
}

}  // namespace

hipError_t launch_quant_rows(int dtype, const void* x, int64_t ldx, int rows, int cols, uint8_t* q, int64_t ldq,
                             float* scales, hipStream_t s) {
  const dim3 grid((rows + 3) / 4);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<BF16>, grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
  else if (dtype == DT_F16)
    hipLaunchKernelGGL(quant_rows_kernel<F16>, grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
  else
    hipLaunchKernelGGL(quant_rows_kernel<F32>, grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
  return hipGetLastError();
}

hipError_t launch_quant_weight(int dtype, const void* w, int d_in, int d_out, uint8_t* wq_t, float* scales,
                               hipStream_t s) {
  // the block maxima ((d_in / 64) x d_out floats) live in the code buffer until pass 3 writes it:
  // it holds d_out * d_in bytes, at least 4 * (d_in / 64) * d_out since d_in >= 64
  const dim3 g2((d_out + 63) / 64, (d_in + 63) / 64);
  float* part = (float*)wq_t;
  const int n_part = (d_in + 63) / 64;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(wq_colmax_kernel<BF16>, g2, dim3(256), 0, s, w, d_in, d_out, part);
  else if (dtype == DT_F16)
    hipLaunchKernelGGL(wq_colmax_kernel<F16>, g2, dim3(256), 0, s, w, d_in, d_out, part);
  else
    hipLaunchKernelGGL(wq_colmax_kernel<F32>, g2, dim3(256), 0, s, w, d_in, d_out, part);
  hipLaunchKernelGGL(wq_scale_kernel, dim3((d_out + 255) / 256), dim3(256), 0, s, part, n_part, d_out, scales);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(wq_quant_kernel<BF16>, g2, dim3(256), 0, s, w, d_in, d_out, scales, wq_t);
  else if (dtype == DT_F16)
    hipLaunchKernelGGL(wq_quant_kernel<F16>, g2, dim3(256), 0, s, w, d_in, d_out, scales, wq_t);
  else
    hipLaunchKernelGGL(wq_quant_kernel<F32>, g2, dim3(256), 0, s, w, d_in, d_out, scales, wq_t);
  return hipGetLastError();
}

hipError_t launch_proj8(int out_dtype, const uint8_t* aq, const float* sa, const uint8_t* wq_t, const float* sw,
                        void* out, int m, int n, int k, hipStream_t s) {
  const int tm = (m + 127) / 128, tn = (n + 127) / 128;
  if (out_dtype == DT_BF16)
    hipLaunchKernelGGL(proj8_kernel<BF16>, dim3(tm * tn), dim3(256), 0, s, aq, sa, wq_t, sw, out, m, n, k, tm, tn);
  else
    hipLaunchKernelGGL(proj8_kernel<F16>, dim3(tm * tn), dim3(256), 0, s, aq, sa, wq_t, sw, out, m, n, k, tm, tn);
  return hipGetLastError();
}

}  // namespace ispa
