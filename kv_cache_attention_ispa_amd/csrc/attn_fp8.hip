// FP8 attention of a converted (local-attention) layer for gfx950.
//
// ISPA technical summary (gist.science, nl/pt), section 4 "Results": the method combined with W8A8
// post-training quantisation gives the largest overall speed-up.  This library reads W8A8 for the
// attention of a converted layer as FP8 E4M3 operands for both matrix products:
//   * Q: one scale per query token and head, s_q = absmax / 448 (codes E4M3(q / s_q), in the kernel);
//   * K, V: one scale per head over the layer's rows (sink + current chunk), s = absmax / 448;
//   * scores in log2 units x = s_q s_k (Qq . Kq) scale log2(e); the row reference M is an integer
//     (the ceiling of the running maximum) and P = 2^(x - M) is coded as E4M3(256 P);
//   * l = sum of the decoded P codes, O = s_v sum_j dec(Pq_j) dec(Vq_j) / l.
// Because M only moves by whole powers of two, the decoded codes of a tile taken against an earlier
// reference equal, after the rescale, the codes taken against the final one (E4M3 rounding commutes
// with exact power-of-two scaling; only values below its normal range, under 2^-14 of the row's
// largest probability, can differ).
//
// Kernel design: the structure of the 16-bit attention kernel (8 waves of 32 queries, two groups
// ping-ponging between matrix and softmax phases, three-deep direct-to-LDS rings two tiles ahead)
// with FP8 tiles and v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
//   * QK^T: S^T = K Q^T, 2 x 2 MFMAs per 64-key tile; the K tile's rows are stored in LDS in the
//     order the A operand reads them (row 32 kt + m holds key 32 ((m / 4) % 2) + 16 kt + 4 (m / 8) +
//     m % 4), so that lane (query n, half h) accumulates keys 32 h + 16 kt + r in its register r --
//     its 32 consecutive keys of the PV B operand -- and a quarter-wave reads 16 consecutive rows;
//   * PV: O^T = V^T P^T, 4 MFMAs per tile from a transposed FP8 copy of V (64-byte key rows);
//   * the row sum of the decoded codes is a fifth MFMA against a register-constant row of ones.
// A pre-pass finds the per-head maxima of K and V and writes their codes (K row-major, V transposed).
#include "common.hpp"
#include "kernels.hpp"

namespace ispa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int HD = 128, BN = 64, WAVES = 8, THREADS = WAVES * 64, BM = WAVES * 32;
constexpr float kE4M3Max = 448.f;
constexpr int K8_PITCH = HD + 16;             // 144 bytes per K row (128 codes + padding)
constexpr int K8_SLOTS = K8_PITCH / 16;
constexpr int K8_TILE = BN * K8_PITCH;
constexpr int V8_PITCH = BN + 16;             // 80 bytes per head-dim row of V^T (64 codes + padding)
constexpr int V8_SLOTS = V8_PITCH / 16;
constexpr int V8_TILE = HD * V8_PITCH;
constexpr int K8_INST = BN * K8_SLOTS / 64;   // 9 wave-wide 16-byte loads per K tile
constexpr int V8_INST = HD * V8_SLOTS / 64;   // 10 per V^T tile
constexpr int LOADS8 = (K8_INST + V8_INST + WAVES - 1) / WAVES;   // 3 per wave
static_assert(K8_SLOTS * BN % 64 == 0 && V8_SLOTS * HD % 64 == 0, "tile must be whole wave loads");
constexpr int PRE_ROWS = 32;                  // rows per work-group of the absmax pre-pass

// LDS row 32 kt + m of a K tile holds key kperm(32 kt + m) of the tile
__device__ __forceinline__ int kperm(int row) {
  const int kt = row >> 5, m = row & 31;
  return 32 * ((m >> 2) & 1) + 16 * kt + 4 * (m >> 3) + (m & 3);
}

// four codes of four values already divided by their scale, packed low to high (clamped to +-448:
// the conversion does not saturate)
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}
// the same for values known to lie in [0, 448] (no clamp)
__device__ __forceinline__ uint32_t pack4_in_range(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ------------------------------------------------------------------------------------------------
// Pre-pass over the layer's own rows, numbered r = 0 .. n_loc - 1: the sink rows, then the current
// chunk (source row r + n_hist; the history rows between them are not read).  Partial maxima:
// work-group (b, y, t) covers rows [32 b, 32 b + 32) of tensor t (K, V) and 16-byte column chunks
// [256 y, +256) (16 heads); thread i keeps the running max |x| of chunk 256 y + i over those rows, and
// the 16 chunks of a head (16 consecutive lanes) reduce it to part[(t * nblk + b) * H + h].
template <typename T>
__global__ __launch_bounds__(256) void kv8_absmax_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                         int n_sink, int n_hist, int n_loc, int d, int nblk,
                                                         float* __restrict__ part) {
  const int t = blockIdx.z, b = blockIdx.x, H = d / HD, cpr = d / 8;
  const uint16_t* x = t == 0 ? k : v;
  const int c = 256 * blockIdx.y + threadIdx.x;
  const int r0 = b * PRE_ROWS, rows = min(PRE_ROWS, n_loc - r0);
  float m = 0.f;
  if (c < cpr) {
#pragma unroll 8
    for (int r = 0; r < rows; ++r) {
      const int64_t src = r0 + r < n_sink ? r0 + r : (int64_t)r0 + r + n_hist;
      const u32x4 w = *(const u32x4*)(x + src * d + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m = fmaxf(m, fabsf(Cvt<T>::to_f((uint16_t)(w[e] & 0xFFFFu))));
        m = fmaxf(m, fabsf(Cvt<T>::to_f((uint16_t)(w[e] >> 16))));
      }
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (c < cpr && (threadIdx.x & 15) == 0) part[(t * nblk + b) * H + c / 16] = m;
}

// scales of head h of K and V from the partial maxima, reduced by the whole work-group (the same
// float32 operations as the codes of the projection: absmax / 448, 1 for an all-zero head)
__device__ __forceinline__ void head_scales(const float* part, int nblk, int H, int h, float& sk, float& sv) {
  __shared__ float red[2][4];
  float mk = 0.f, mv = 0.f;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    mk = fmaxf(mk, part[b * H + h]);
    mv = fmaxf(mv, part[(nblk + b) * H + h]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, o));
    mv = fmaxf(mv, __shfl_xor(mv, o));
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = mk;
    red[1][threadIdx.x >> 6] = mv;
  }
  __syncthreads();
  mk = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  mv = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  sk = mk > 0.f ? mk / kE4M3Max : 1.f;
  sv = mv > 0.f ? mv / kE4M3Max : 1.f;
}

// Codes of the layer's own rows (numbered as in the pre-pass): work-group (kb, cb) covers keys
// [64 kb, +64) and columns [64 cb, +64) (one head): K codes row-major kq[key * d + c], V codes
// transposed vqt[c * ldv + key] (keys in [n_loc, ldv) zero), through
// an LDS tile for the transpose.  Work-groups of key block 0 also store the two scales of their head.
template <typename T>
__global__ __launch_bounds__(256) void kv8_quant_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        int n_sink, int n_hist, int n_loc, int d, int ldv, int nblk,
                                                        const float* __restrict__ part, uint8_t* __restrict__ kq,
                                                        uint8_t* __restrict__ vqt, float* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64][80];   // [key][column]
  const int key0 = blockIdx.x * 64, c0 = blockIdx.y * 64, H = d / HD, h = c0 / HD;
  float sk, sv;
  head_scales(part, nblk, H, h, sk, sv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scales[h] = sk;
    scales[H + h] = sv;
  }
  const int r = threadIdx.x >> 3, ch = threadIdx.x & 7;   // 32 rows x 8 chunks of 8 values per pass
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int key = key0 + r + 32 * pass;
    uint32_t kc[2] = {0u, 0u}, vc[2] = {0u, 0u};
    if (key < n_loc) {
      const int64_t src = key < n_sink ? key : (int64_t)key + n_hist;
      const u32x4 kw = *(const u32x4*)(k + src * d + c0 + 8 * ch);
      const u32x4 vw = *(const u32x4*)(v + src * d + c0 + 8 * ch);
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = Cvt<T>::to_f((uint16_t)(kw[e] & 0xFFFFu)) / sk;
        kf[2 * e + 1] = Cvt<T>::to_f((uint16_t)(kw[e] >> 16)) / sk;
        vf[2 * e] = Cvt<T>::to_f((uint16_t)(vw[e] & 0xFFFFu)) / sv;
        vf[2 * e + 1] = Cvt<T>::to_f((uint16_t)(vw[e] >> 16)) / sv;
      }
      kc[0] = pack4(kf[0], kf[1], kf[2], kf[3]);
      kc[1] = pack4(kf[4], kf[5], kf[6], kf[7]);
      vc[0] = pack4(vf[0], vf[1], vf[2], vf[3]);
      vc[1] = pack4(vf[4], vf[5], vf[6], vf[7]);
      *(u32x2*)(kq + (int64_t)key * d + c0 + 8 * ch) = u32x2{kc[0], kc[1]};
    }
    *(u32x2*)&tile[r + 32 * pass][8 * ch] = u32x2{vc[0], vc[1]};
  }
  __syncthreads();
  // transposed: thread -> column c (64) x 16-key group g (4): 16 codes, one 16-byte store
  const int c = threadIdx.x >> 2, g = threadIdx.x & 3;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) x |= (uint32_t)tile[16 * g + 4 * q + e][c] << (8 * e);
    w[q] = x;
  }
  *(u32x4*)(vqt + (int64_t)(c0 + c) * ldv + key0 + 16 * g) = u32x4{w[0], w[1], w[2], w[3]};
}

// ------------------------------------------------------------------------------------------------
// The attention kernel.
struct Fp8Params {
  const uint16_t* q;      // [n_q, d] io dtype
  const uint8_t* kq;      // [n_loc, d] codes of the layer's own rows (sink, then current chunk)
  const uint8_t* vqt;     // [d, ldv] codes
  const float* scales;    // s_k[H], s_v[H]
  void* out;              // [n_q, d] io dtype
  int n_q, n_loc, n_heads, d, ldv, n_qblk;
  float scale_log2;       // softmax scale * log2(e)
};

// the key tiles: 64 consecutive rows of the compacted codes (sink rows, then current chunk); the
// last tile holds n_loc - 64 (n - 1) keys
struct Sched8 {
  int n_loc, n;
  __device__ __forceinline__ void set(int rows) {
    n_loc = rows;
    n = (rows + BN - 1) / BN;
  }
  __device__ __forceinline__ int row(int t) const { return BN * t; }
  __device__ __forceinline__ int valid(int t) const { return n_loc - BN * t; }
};

// Load group k = {K tile k, V^T tile k-1}, LOADS8 wave-wide direct-to-LDS loads per wave.  Load `inst`
// of a tile puts lane l on 16-byte slot 64 inst + l: LDS row slot / SLOTS, chunk slot % SLOTS (the last
// chunk of a row is padding: a lane there loads its row's last chunk again).  K: LDS row p holds key
// kperm(p) of the tile; V^T: LDS row = head dim.
struct Loader8 {
  __amdgpu_buffer_rsrc_t rv;
  const uint8_t* kb;
  int64_t kbytes;
  uint32_t off[LOADS8];
  __device__ __forceinline__ void init(const Fp8Params& p, int n_k, int wave, int lane, int head) {
    kb = p.kq;
    kbytes = (int64_t)n_k * p.d;
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.vqt + (int64_t)head * HD * p.ldv), (short)0,
                                           (int)((int64_t)HD * p.ldv), 0x00020000);
#pragma unroll
    for (int j = 0; j < LOADS8; ++j) {
      const int idx = wave + WAVES * j;
      if (idx < K8_INST) {
        const int slot = 64 * idx + lane;
        off[j] = (uint32_t)(kperm(slot / K8_SLOTS) * p.d + min(slot % K8_SLOTS, 7) * 16);
      } else {
        const int slot = 64 * min(idx - K8_INST, V8_INST - 1) + lane;
        off[j] = (uint32_t)((slot / V8_SLOTS) * p.ldv + min(slot % V8_SLOTS, 3) * 16);
      }
    }
  }
  struct Group {
    __amdgpu_buffer_rsrc_t rk;
    uint32_t sk, sv;
    char* kt;
    char* vt;
  };
  __device__ __forceinline__ Group group(const Sched8& sc, int k, const Fp8Params& p, int head, char* kt,
                                         char* vt) const {
    const int tk = min(k, sc.n - 1);
    const int tv = min(max(k - 1, 0), sc.n - 1);
    const int64_t k0 = (int64_t)sc.row(tk) * p.d;
    const int64_t rest = kbytes - k0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kb + k0), (short)0, (int)(rest < INT32_MAX ? rest : INT32_MAX), 0x00020000);
    return Group{rk, (uint32_t)(head * HD), (uint32_t)sc.row(tv), kt, vt};
  }
  __device__ __forceinline__ void issue(const Group& g, int wave) const {
#pragma unroll
    for (int j = 0; j < LOADS8; ++j) {
      const int idx = wave + WAVES * j;
      if (idx < K8_INST)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rk, (lds_void*)(g.kt + 1024 * idx), 16, off[j], g.sk, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(g.vt + 1024 * min(idx - K8_INST, V8_INST - 1)), 16,
                                                 off[j], g.sv, 0, 0);
    }
  }
};

__device__ __forceinline__ float max_xor32_8(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ i32x8 ld32(const char* p) {
  const u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 16);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Online state of a wave's 32 queries: O^T accumulators (register r of lane l, tile t: head dim
// 32 t + 8 (r / 4) + 4 (l / 32) + r % 4), the ones-row accumulator (register 0 of lanes 0-31 holds the
// row sum), and the integer reference M (log2 units).
struct State8 {
  f32x16 o[4];
  f32x16 lacc;
  float M;
};

// Matrix phase: S^T = K Q^T for the next tile (kt, dim half) and O^T += V^T P^T, L += 1 P^T for the
// current one.  kb: this lane's K row base (LDS row = lane % 32, byte 32 (lane / 32)); vb: V^T row
// base (row lane % 32, byte 32 (lane / 32)).
__device__ __forceinline__ void matrix8(const char* kt, const char* vt, int kbase, int vbase, const i32x8 (&qf)[2],
                                        const i32x8& pf, const i32x8& ones, f32x16 (&s)[2], State8& st) {
  const char* kp = kt + kbase;
  const char* vp = vt + vbase;
  i32x8 a00 = ld32(kp), a01 = ld32(kp + 64);
  i32x8 a10 = ld32(kp + 32 * K8_PITCH), a11 = ld32(kp + 32 * K8_PITCH + 64);
  i32x8 v0 = ld32(vp), v1 = ld32(vp + 32 * V8_PITCH), v2 = ld32(vp + 64 * V8_PITCH), v3 = ld32(vp + 96 * V8_PITCH);
  s[0] = mfma8(a00, qf[0], f32x16{});
  s[1] = mfma8(a10, qf[0], f32x16{});
  st.o[0] = mfma8(v0, pf, st.o[0]);
  st.o[1] = mfma8(v1, pf, st.o[1]);
  s[0] = mfma8(a01, qf[1], s[0]);
  s[1] = mfma8(a11, qf[1], s[1]);
  st.o[2] = mfma8(v2, pf, st.o[2]);
  st.o[3] = mfma8(v3, pf, st.o[3]);
  st.lacc = mfma8(ones, pf, st.lacc);
}

// Softmax phase: mask, tile maximum, integer reference (rescale on a move), probabilities coded as
// E4M3(256 P) and packed as the PV B operand (keys 32 hi + 16 kt + r).
__device__ __forceinline__ void softmax8(f32x16 (&s)[2], int valid, float c, int hi, State8& st, i32x8& pf) {
  if (valid < BN) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * hi + 16 * kt + r >= valid) s[kt][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  mx = max_xor32_8(mx) * c;      // the row's maximum over this tile, log2 units (c > 0)
  const bool up = mx > st.M;
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float Mn = up ? ceilf(mx) : st.M;
    const float alpha = __builtin_amdgcn_exp2f(st.M - Mn);   // an exact power of two (0 on the first tile)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[t][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.lacc[r] *= alpha;
    st.M = Mn;
  }
  const float off = 8.f - st.M;    // 256 P = 2^(x - M + 8)
  uint32_t w[8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(s[kt][4 * q + j], c, off));
      // M is the ceiling of every score of the tile, so 256 P <= 256: in range without a clamp
      w[4 * kt + q] = pack4_in_range(e[0], e[1], e[2], e[3]);
    }
  pf = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

template <typename T>
__global__ __launch_bounds__(THREADS, 1) void attn_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(16))) char k0[K8_TILE];
  __shared__ __attribute__((aligned(16))) char k1[K8_TILE];
  __shared__ __attribute__((aligned(16))) char k2[K8_TILE];
  __shared__ __attribute__((aligned(16))) char v0[V8_TILE];
  __shared__ __attribute__((aligned(16))) char v1[V8_TILE];
  __shared__ __attribute__((aligned(16))) char v2[V8_TILE];
  const int n_blocks = p.n_qblk * p.n_heads;
  const int logical = xcd_remap(blockIdx.x, n_blocks);
  const int head = logical / p.n_qblk, qblk = logical % p.n_qblk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int grp = wave >> 2, hi = lane >> 5;
  const int qrow = qblk * BM + wave * 32 + (lane & 31);
  const bool qok = qrow < p.n_q;
  // a wave with no query below n_q issues its loads and meets every barrier, and multiplies nothing
  const bool live = qblk * BM + wave * 32 < p.n_q;
  const int col0 = head * HD;

  // Q codes for the B operand of MFMA h: this lane's query, head dims 64 h + 32 hi + 0..31
  float qv[64];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (qok) w = *(const u32x4*)(p.q + (int64_t)qrow * p.d + col0 + 64 * h + 32 * hi + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[32 * h + 8 * j + 2 * e] = Cvt<T>::to_f((uint16_t)(w[e] & 0xFFFFu));
        qv[32 * h + 8 * j + 2 * e + 1] = Cvt<T>::to_f((uint16_t)(w[e] >> 16));
      }
    }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) am = fmaxf(am, fabsf(qv[i]));
  am = max_xor32_8(am);
  const float sq = am > 0.f ? am / kE4M3Max : 1.f;
  i32x8 qf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j] = pack4(qv[32 * h + 4 * j] / sq, qv[32 * h + 4 * j + 1] / sq, qv[32 * h + 4 * j + 2] / sq,
                   qv[32 * h + 4 * j + 3] / sq);
    qf[h] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
  }
  const float sk = p.scales[head], sv = p.scales[p.n_heads + head];
  const float c = p.scale_log2 * sq * sk;
  const int ov = (lane & 31) == 0 ? 0x38383838 : 0;   // E4M3 1.0 in every byte of row 0
  const i32x8 ones = i32x8{ov, ov, ov, ov, ov, ov, ov, ov};

  Sched8 sc;
  sc.set(p.n_loc);

  Loader8 ld;
  ld.init(p, p.n_loc, wave, lane, head);
  auto kslot = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return k0;
    else if constexpr (decltype(J)::value == 1) return k1;
    else return k2;
  };
  auto vslot = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return v0;
    else if constexpr (decltype(J)::value == 1) return v1;
    else return v2;
  };
  ld.issue(ld.group(sc, 0, p, head, k0, v2), wave);
  ld.issue(ld.group(sc, 1, p, head, k1, v0), wave);
  ld.issue(ld.group(sc, 2, p, head, k2, v1), wave);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  lds_barrier();

  const int kbase = (lane & 31) * K8_PITCH + 32 * hi;
  const int vbase = (lane & 31) * V8_PITCH + 32 * hi;
  State8 st;
  f32x16 s[2];
  i32x8 pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  auto reset = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) st.o[t] = f32x16{};
    st.lacc = f32x16{};
    st.M = -INFINITY;
  };
  reset();

  // the schedule of the 16-bit kernel: M(t) = QK(t+1) + PV(t) reads K slot (t+1) % 3 and V slot t % 3
  auto matrix = [&](auto J, int t) {
    constexpr int j = decltype(J)::value;
    if (live) matrix8(kslot(J), vslot(std::integral_constant<int, (j + 2) % 3>{}), kbase, vbase, qf, pf, ones, s, st);
    if (t < 0) reset();
  };
  auto issue_ahead = [&](auto J, int i) {
    constexpr int j = decltype(J)::value;
    ld.issue(ld.group(sc, i + 2, p, head, kslot(std::integral_constant<int, (j + 2) % 3>{}),
                      vslot(std::integral_constant<int, (j + 1) % 3>{})), wave);
  };
  auto softmax = [&](int t) {
    if (!live || t < 0 || t >= sc.n) return;
    softmax8(s, sc.valid(t), c, hi, st, pf);
  };
  auto phase_end = [&]() { lds_barrier(); };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS8)); };
  auto iteration0 = [&](auto J, int i) {
    matrix(J, i - 1);
    phase_end();
    issue_ahead(J, i);
    softmax(i);
    wait_loads();
    phase_end();
  };
  auto iteration1 = [&](auto J, int i) {
    issue_ahead(J, i);
    softmax(i - 1);
    phase_end();
    matrix(J, i - 1);
    wait_loads();
    phase_end();
  };
  const std::integral_constant<int, 0> J0;
  const std::integral_constant<int, 1> J1;
  const std::integral_constant<int, 2> J2;
  if (grp == 0) {
    for (int i = 0; i <= sc.n; i += 3) {
      iteration0(J0, i);
      if (i + 1 > sc.n) break;
      iteration0(J1, i + 1);
      if (i + 2 > sc.n) break;
      iteration0(J2, i + 2);
    }
  } else {
    for (int i = 0; i <= sc.n; i += 3) {
      iteration1(J0, i);
      if (i + 1 > sc.n) break;
      iteration1(J1, i + 1);
      if (i + 2 > sc.n) break;
      iteration1(J2, i + 2);
    }
  }

  if (!live) return;   // no barrier follows the loop
  // O = s_v O / l; l sits in register 0 of lanes 0-31
  const uint32_t lu = __float_as_uint(st.lacc[0]);
  const auto lr = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
  const float l = hi ? __uint_as_float(lr[0]) : st.lacc[0];
  const float f = l > 0.f ? sv / l : 0.f;
  if (!qok) return;
  uint16_t* base = (uint16_t*)p.out + (int64_t)qrow * p.d + col0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int cc = 32 * t + 8 * rq + 4 * hi;
      *(u32x2*)(base + cc) = u32x2{pack2<T>(st.o[t][4 * rq] * f, st.o[t][4 * rq + 1] * f),
                                   pack2<T>(st.o[t][4 * rq + 2] * f, st.o[t][4 * rq + 3] * f)};
    }
}

}  // namespace

size_t attn_fp8_workspace_bytes(int64_t n_loc, int64_t d) {
  const int64_t nblk = (n_loc + PRE_ROWS - 1) / PRE_ROWS, H = d / HD, ldv = (n_loc + 63) / 64 * 64;
  auto al = [](int64_t b) { return (size_t)((b + 255) / 256 * 256); };
  return al(2 * nblk * H * 4) + al(2 * H * 4) + al(n_loc * d) + al(d * ldv);
}

hipError_t launch_attention_fp8(const AttnLaunch& L, hipStream_t s) {
  const int64_t n_k = (int64_t)L.n_sink + L.n_cur;   // the layer's own rows
  const int d = L.n_heads * L.head_dim, H = L.n_heads;
  const int nblk = (int)((n_k + PRE_ROWS - 1) / PRE_ROWS);
  const int ldv = (int)((n_k + 63) / 64 * 64);
  auto al = [](int64_t b) { return (size_t)((b + 255) / 256 * 256); };
  char* w = (char*)L.ws;
  float* part = (float*)w;
  w += al(2 * (int64_t)nblk * H * 4);
  float* scales = (float*)w;
  w += al(2 * (int64_t)H * 4);
  uint8_t* kq = (uint8_t*)w;
  w += al(n_k * d);
  uint8_t* vqt = (uint8_t*)w;
  const dim3 agrid(nblk, (d / 8 + 255) / 256, 2);
  if (L.io == DT_BF16) {
    hipLaunchKernelGGL(kv8_absmax_kernel<BF16>, agrid, dim3(256), 0, s, (const uint16_t*)L.k,
                       (const uint16_t*)L.v, L.n_sink, L.n_hist, (int)n_k, d, nblk, part);
    hipLaunchKernelGGL(kv8_quant_kernel<BF16>, dim3(ldv / 64, d / 64), dim3(256), 0, s, (const uint16_t*)L.k,
                       (const uint16_t*)L.v, L.n_sink, L.n_hist, (int)n_k, d, ldv, nblk, part, kq,
                       vqt, scales);
  } else {
    hipLaunchKernelGGL(kv8_absmax_kernel<F16>, agrid, dim3(256), 0, s, (const uint16_t*)L.k,
                       (const uint16_t*)L.v, L.n_sink, L.n_hist, (int)n_k, d, nblk, part);
    hipLaunchKernelGGL(kv8_quant_kernel<F16>, dim3(ldv / 64, d / 64), dim3(256), 0, s, (const uint16_t*)L.k,
                       (const uint16_t*)L.v, L.n_sink, L.n_hist, (int)n_k, d, ldv, nblk, part, kq,
                       vqt, scales);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Fp8Params p;
  p.q = (const uint16_t*)L.q;
  p.kq = kq;
  p.vqt = vqt;
  p.scales = scales;
  p.out = L.a_full;
  p.n_q = L.n_q;
  p.n_loc = (int)n_k;
  p.n_heads = L.n_heads;
  p.d = d;
  p.ldv = ldv;
  p.n_qblk = (L.n_q + BM - 1) / BM;
  p.scale_log2 = L.scale * kLog2e;
  const dim3 grid(p.n_qblk * L.n_heads);
  if (L.io == DT_BF16)
    hipLaunchKernelGGL(attn_fp8_kernel<BF16>, grid, dim3(THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<F16>, grid, dim3(THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace ispa
