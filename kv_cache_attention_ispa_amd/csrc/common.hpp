// Shared device helpers for the ISPA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ispa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, work-groups dispatched round-robin

// Element tags.  Storage is 16-bit patterns (uint16_t) for both half types.
struct BF16 { typedef uint16_t storage; };
struct F16 { typedef uint16_t storage; };
struct F32 { typedef float storage; };

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Cvt;
template <> struct Cvt<BF16> {
  static __device__ __forceinline__ float to_f(uint16_t b) { return bf16_bits_to_float(b); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return float_to_bf16_bits(f); }
};
template <> struct Cvt<F16> {
  static __device__ __forceinline__ float to_f(uint16_t b) { return f16_bits_to_float(b); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return float_to_f16_bits(f); }
};
template <> struct Cvt<F32> {
  static __device__ __forceinline__ float to_f(float b) { return b; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
};

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Pack two floats into one dword of two 16-bit values (low = a), round to nearest even;
// one v_cvt_pk_{bf16,f16}_f32 each.
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// 32x32x16 MFMA with 16-bit inputs given as raw dword quads (8 values per lane).
// A: lane l holds A[m = l%32][k = 8*(l/32) + 0..7]; B: B[k = 8*(l/32) + 0..7][n = l%32];
// C/D: register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
template <typename T> __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma32x32x16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma32x32x16<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}

// Work-group id -> logical tile id such that each XCD receives a contiguous range
// of logical ids (work-groups are dispatched round-robin over the XCDs).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  int xcd = bid % kNumXcd;
  int local = bid / kNumXcd;
  int per = n / kNumXcd;
  int rem = n % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Epilogue of a wave's 64 x 64 part of a 128-column output tile (wave w = (wm, wn) = (w / 2, w % 2) owns rows 64 wm ..
// columns 64 wn ..; accumulator register r of lane l of block (mi, ni) is element (64 wm + 32 mi +
// 8 (r/4) + 4 (l/32) + r%4, 64 wn + 32 ni + l%32), the 32x32 MFMA layout): each value times
// scale(row, col) (tile coordinates) is rounded to T into the wave's own 8 KiB of LDS, which is then
// written out as 16-byte row pieces, 8 lanes per 128-byte row.  The caller makes sure no wave still
// reads `lds` (a barrier after the last use); n % 8 == 0.
// Work-group barrier of the pipelined kernels: this wave's LDS operations complete first, while loads
// into LDS issued ahead stay in flight (no vmcnt wait, unlike __syncthreads); the wavefront-scope
// fences keep the compiler from moving memory operations across the barrier and emit no instruction.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_sched_barrier(0);
}

// Lanes of one wave exchanging data through LDS: the hardware runs a wave's LDS instructions in
// order, but the compiler, reasoning per lane, could move one lane's read above another lane's write.
// A wavefront-scope fence keeps the program order and emits no instruction.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

template <typename T, typename F>
__device__ __forceinline__ void store_wave_tile_64(const f32x16 (&acc)[2][2], char* lds, typename T::storage* out,
                                                   int64_t ld, int m0, int n0, int m, int n, F scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int c = 32 * ni + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * mi + 8 * (r >> 2) + 4 * hi + (r & 3);
        *(typename T::storage*)(lds + rr * 128 + 2 * c) = Cvt<T>::from_f(acc[mi][ni][r] * scale(64 * wm + rr, 64 * wn + c));
      }
    }
  wave_lds_order();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lane + 64 * i, rr = q >> 3, ch = q & 7;
    const int row = m0 + 64 * wm + rr, col = n0 + 64 * wn + 8 * ch;
    if (row < m && col < n) *(u32x4*)(out + (int64_t)row * ld + col) = *(const u32x4*)(lds + rr * 128 + 16 * ch);
  }
}

// Hand-overs between work-groups on different XCDs.  Device-scope (sc1) buffer accesses bypass the
// XCD-local L2s, so data that one work-group stores this way and another loads this way needs no cache
// write-back or invalidation; flags are relaxed device-wide atomics.  A writer's stores complete
// (s_waitcnt) before it sets the flag, and a reader loads the data only after it has seen the flag.
constexpr int kSc1 = 16;   // cache policy bits of a buffer access: device scope
__device__ __forceinline__ f32x4 sc1_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ void sc1_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kSc1);
}
__device__ __forceinline__ int flag_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_max_xor32(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace ispa
