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
//  * quant_rows_kernel: one wave per row of a [rows, cols] matrix (16-bit or fp32), read once with
//    16-byte loads and kept in registers (rows up to 5120 values): absmax, scale, codes written
//    row-major -- the activations, token by token;
//  * wq_colmax_kernel, wq_scale_kernel, wq_quant_kernel: the weights per output channel (block maxima,
//    scales, codes), written transposed
//    (Wq^T [d_out, d_in]) so that both operands of the product are contiguous along k;
//  * the product out = (Aq Wq) s_a s_w^T runs on the shared projection kernel (proj.hip).
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace ispa {
namespace {

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
// eight consecutive values of a row as floats (one 16-byte load for 16-bit types, two for fp32)
template <typename T> __device__ __forceinline__ void ld8(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (sizeof(typename T::storage) == 2) {
    const u32x4 r = *(const u32x4*)((const typename T::storage*)p + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = Cvt<T>::to_f((typename T::storage)(r[e] & 0xFFFFu));
      v[2 * e + 1] = Cvt<T>::to_f((typename T::storage)(r[e] >> 16));
    }
  } else {
    const f32x4 a = *(const f32x4*)((const float*)p + i), b = *(const f32x4*)((const float*)p + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

// The row stays in registers between the maximum and the codes when it has at most 512 NREG values
// per 64 lanes (NREG > 0); NREG = 0 reads it twice.
template <typename T, int NREG>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* x, int64_t ldx, int rows, int cols, uint8_t* q,
                                                         int64_t ldq, float* scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = (int64_t)row * ldx;
  uint8_t* qr = q + (int64_t)row * ldq;
  float amax = 0.f;
  if constexpr (NREG > 0) {
    float v[NREG][8];
#pragma unroll
    for (int j = 0; j < NREG; ++j) {
      const int c = 8 * lane + 512 * j;
      if (c < cols) ld8<T>(x, base + c, v[j]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float s = e4m3_scale(amax);
    if (lane == 0) scales[row] = s;
#pragma unroll
    for (int j = 0; j < NREG; ++j) {
      const int c = 8 * lane + 512 * j;
      if (c < cols)
        *(u32x2*)(qr + c) = u32x2{e4m3_pack4(v[j][0] / s, v[j][1] / s, v[j][2] / s, v[j][3] / s),
                                  e4m3_pack4(v[j][4] / s, v[j][5] / s, v[j][6] / s, v[j][7] / s)};
    }
  } else {
    float v[8];
    for (int c = 8 * lane; c < cols; c += 512) {
      ld8<T>(x, base + c, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float s = e4m3_scale(amax);
    if (lane == 0) scales[row] = s;
    for (int c = 8 * lane; c < cols; c += 512) {
      ld8<T>(x, base + c, v);
      *(u32x2*)(qr + c) = u32x2{e4m3_pack4(v[0] / s, v[1] / s, v[2] / s, v[3] / s),
                                e4m3_pack4(v[4] / s, v[5] / s, v[6] / s, v[7] / s)};
    }
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

template <typename T>
void quant_rows_t(const void* x, int64_t ldx, int rows, int cols, uint8_t* q, int64_t ldq, float* scales,
                  hipStream_t s) {
  const dim3 grid((rows + 3) / 4);
  if (cols <= 512 * 4)
    hipLaunchKernelGGL((quant_rows_kernel<T, 4>), grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
  else if (cols <= 512 * 10)
    hipLaunchKernelGGL((quant_rows_kernel<T, 10>), grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
  else
    hipLaunchKernelGGL((quant_rows_kernel<T, 0>), grid, dim3(256), 0, s, x, ldx, rows, cols, q, ldq, scales);
}

}  // namespace

hipError_t launch_quant_rows(int dtype, const void* x, int64_t ldx, int rows, int cols, uint8_t* q, int64_t ldq,
                             float* scales, hipStream_t s) {
  if (dtype == DT_BF16) quant_rows_t<BF16>(x, ldx, rows, cols, q, ldq, scales, s);
  else if (dtype == DT_F16) quant_rows_t<F16>(x, ldx, rows, cols, q, ldq, scales, s);
  else quant_rows_t<F32>(x, ldx, rows, cols, q, ldq, scales, s);
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


}  // namespace ispa
