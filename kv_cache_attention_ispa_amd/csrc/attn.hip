// Dual-stream (decomposable) attention for gfx950.
//
// ISPA technical summary (gist.science, nl/pt), section 2, stage 1
// "Dual-Stream Warmup": an F-layer produces A_full (attention over the whole
// cached history) and A_loc (attention over the sink tokens and the current
// chunk) in one pass, by splitting attention into a local and a historical
// branch, each with its own online-softmax state, and merging the two through
// their log-sum-exp.  The merge is exact: with LSE_F = log(e^LSE_L + e^LSE_H)
// and w = e^(LSE_H - LSE_F), A_full = A_loc + w (O_H - A_loc).
//
// Kernel design (bf16 / fp16, head_dim 128):
//  * one work-group = 128 queries of one head, 4 waves x 32 queries;
//  * keys stream through LDS in tiles of 64 rows (K and V, double-buffered,
//    padded row pitches) with direct global-to-LDS loads issued one tile ahead;
//    a branch is a virtual row range made of
//    up to two physical segments, so the sink + current-chunk local set is
//    one contiguous loop and only its last tile needs a mask;
//  * S^T = K Q^T with 32x32x16 MFMA: every lane owns one query, so the softmax
//    max/sum are in-lane plus one cross-lane step (lanes l and l^32);
//  * O^T = V^T P^T with 32x32x16 MFMA: P^T stays in registers (a lane's
//    accumulator registers are exactly its B operand, with the reduction index
//    ordered as two groups of 4 consecutive keys), V^T comes from the row-major
//    V tile through transposing LDS reads;
//  * exp2 with the softmax scale folded into log2(e); fp32 accumulation;
//  * when the statistics are requested in fp16 from bf16 inputs, V is copied to
//    fp16 first and the probabilities are rounded to fp16 (11-bit mantissa) for
//    the PV product, which keeps dA accurate enough for ill-conditioned
//    absorption problems; QK^T stays in bf16;
//  * blockIdx -> (head, query block) is XCD-aware so the work-groups of one head
//    share an L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ispa {

namespace {

constexpr int HD = 128;          // head dim of the MFMA path
constexpr int BM = 128;          // queries per work-group
constexpr int BN = 64;           // keys per tile
constexpr int NTHREADS = 256;
constexpr float kRescaleSlack = 8.f;   // log2 units: probabilities stay below 2^8 between rescales
// LDS tiles are row-major with padded pitches: every MFMA operand read is a per-lane base
// address plus an immediate offset, and the read patterns below hit distinct banks.
constexpr int K_PITCH = HD * 2 + 16;              // 272 bytes per key row
constexpr int V_PITCH = HD * 2 + 64;              // 320 bytes per value row
constexpr int K_TILE = BN * K_PITCH;
constexpr int V_TILE = BN * V_PITCH;
constexpr int STAGE_BYTES = K_TILE + V_TILE;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;        // double-buffered: 74 KiB

// A branch: virtual rows [0, len) mapped onto up to two physical row segments.
struct Branch {
  int start0, len0, start1, len;
  __device__ __forceinline__ int row(int v) const { return v < len0 ? start0 + v : start1 + (v - len0); }
};

// Global -> LDS staging of one 64-row tile of K or V for one head with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave instruction writes 16 bytes at base + 16 l).  A padded
// row of PITCH bytes is PITCH/16 slots, 16 of them data; the tile is a run of 64 * PITCH/16 slots
// filled 64 at a time by every lane.  A lane that falls on a padding slot loads its row's last
// chunk again (padding is never read).  Rows past the end of the branch are filled with the
// branch's last row, so the values stay finite (their probabilities are zero).
template <int PITCH>
struct DmaTile {
  static constexpr int SLOTS = PITCH / 16;                   // slots per row
  static constexpr int NINST = SLOTS;                        // 64 rows x SLOTS slots / 64 lanes
  static constexpr int PER_WAVE = (NINST + 3) / 4;
  uint32_t off[PER_WAVE];   // byte offset of this lane's chunk from the tile's first row
  __device__ __forceinline__ void init(int wave, int lane, int d) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int p = 64 * (wave + 4 * j) + lane;
      const int r = p / SLOTS, c = min(p % SLOTS, 15);
      off[j] = (uint32_t)(r * d + c * 8) * 2u;
    }
  }
  // Issue the loads of tile rows [tile_start, tile_start + 64) of branch br (column block col0).
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ src, int d, int col0, const Branch& br,
                                        int tile_start, char* tile, int wave, int lane) const {
    const bool contiguous = tile_start + 64 <= br.len &&
                            (tile_start + 64 <= br.len0 || tile_start >= br.len0);
    if (contiguous) {
      const char* base = (const char*)(src + (int64_t)br.row(tile_start) * d + col0);
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int inst = wave + 4 * j;
        if (inst < NINST)
          __builtin_amdgcn_global_load_lds((const void*)(base + off[j]), (lds_void*)(tile + 1024 * inst), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int inst = wave + 4 * j;
        if (inst < NINST) {
          const int p = 64 * inst + lane;
          const int r = p / SLOTS, c = min(p % SLOTS, 15);
          int vi = tile_start + r;
          vi = vi < br.len ? vi : br.len - 1;
          const uint16_t* g = src + (int64_t)br.row(vi) * d + col0 + c * 8;
          __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(tile + 1024 * inst), 16, 0, 0);
        }
      }
    }
  }
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* a_full;       // token-major, io dtype
  void* a_loc_t;      // feature-major, stat dtype
  void* delta_a_t;    // feature-major, stat dtype
  int64_t ld_stat;
  float* lse_loc;
  float* lse_hist;
  int n_q, n_sink, n_hist, n_cur, n_heads, d, n_qblk;
  float scale_log2;
};

// Online-softmax state of one branch for the 32 queries of a wave.
struct BranchState {
  f32x16 o[4];     // O^T accumulators: d tile t, lane l, reg r -> d = 32t + 8(r/4) + 4(l/32) + r%4
  float m;         // running max (log2 units), identical in lanes l and l^32
  float lsum;      // partial row sum over this lane's keys
};

// T: element type of Q and K (QK^T MFMA); TP: element type of P and V (PV MFMA).
template <typename T, typename TP>
__device__ __forceinline__ void run_branch(const AttnParams& p, const Branch& br, const u32x4 (&qf)[8], int col0,
                                           char* lds, BranchState& st) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hi = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[t][r] = 0.f;
  st.m = -INFINITY;
  st.lsum = 0.f;
  const int n_tiles = (br.len + BN - 1) / BN;
  if (n_tiles == 0) return;

  const int wave = tid >> 6;
  DmaTile<K_PITCH> kd;
  DmaTile<V_PITCH> vd;
  kd.init(wave, lane, p.d);
  vd.init(wave, lane, p.d);
  __syncthreads();  // previous users of the LDS stages are done
  kd.issue(p.k, p.d, col0, br, 0, lds, wave, lane);
  vd.issue(p.v, p.d, col0, br, 0, lds + K_TILE, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // per-lane LDS bases; every read below adds a compile-time offset
  const int kbase = (lane & 31) * K_PITCH + hi * 16;
  const int g = lane >> 4, i16 = lane & 15;
  const int vbase = (4 * (g >> 1) + (i16 >> 2)) * V_PITCH + (16 * (g & 1) + 4 * (i16 & 3)) * 2;
  for (int t = 0; t < n_tiles; ++t) {
    char* stage = lds + (t & 1) * STAGE_BYTES;
    const bool has_next = t + 1 < n_tiles;
    // the next tile streams into the other stage while this one is computed
    if (has_next) {
      char* next = lds + ((t + 1) & 1) * STAGE_BYTES;
      kd.issue(p.k, p.d, col0, br, (t + 1) * BN, next, wave, lane);
      vd.issue(p.v, p.d, col0, br, (t + 1) * BN, next + K_TILE, wave, lane);
    }

    // ---- S^T = K Q^T for two 32-key sub-tiles.  Accumulator register r of lane l holds
    // key 32 kt + 8 (r/4) + 4 (l/32) + r%4 of this tile for query l%32.
    f32x16 s[2];
    const char* kb = stage + kbase;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 a = *(const u32x4*)(kb + 32 * kt * K_PITCH + 32 * ks);
        acc = mfma32x32x16<T>(a, qf[ks], acc);
      }
      s[kt] = acc;
    }
    // ---- mask keys past the end of the branch (last tile only)
    const int valid = br.len - t * BN;
    if (valid < BN) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= valid) s[kt][r] = -INFINITY;
        }
    }
    // ---- online softmax (log2 domain).  The reference max m only moves when this tile's max
    // exceeds it by more than kRescaleSlack (then O and the row sum are rescaled, for the whole
    // wave at once); otherwise the probabilities are taken against the stale reference and stay
    // below 2^kRescaleSlack.  The final normalisation uses the same reference, so this is exact.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = wave_max_xor32(mx) * p.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(st.m, mx);
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
      st.m = m_new;
      st.lsum *= alpha;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[tt][r] *= alpha;
    }
    const float m_ref = st.m;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * u + j], p.scale_log2, -m_ref));
          rs[j & 3] += e[j];
        }
        pf[kt][u] = u32x4{pack2<TP>(e[0], e[1]), pack2<TP>(e[2], e[3]), pack2<TP>(e[4], e[5]), pack2<TP>(e[6], e[7])};
      }
    st.lsum += (rs[0] + rs[1]) + (rs[2] + rs[3]);

    // ---- O^T += V^T P^T.  MFMA step (kt, u) of lane half h uses the probabilities of keys
    // 32 kt + 16 u + 4 h + 0..3 and 32 kt + 16 u + 8 + 4 h + 0..3 (registers 8u..8u+7); the
    // matching V^T operand is two transposing reads of 4 keys x 16 columns per 16-lane group.
    const char* vb = stage + K_TILE + vbase;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const u32x2 h0 = lds_read_tr16((const lds_void*)(vb + (32 * kt + 16 * u) * V_PITCH + 64 * tt));
          const u32x2 h1 = lds_read_tr16((const lds_void*)(vb + (32 * kt + 16 * u + 8) * V_PITCH + 64 * tt));
          const u32x4 a = u32x4{h0.x, h0.y, h1.x, h1.y};
          st.o[tt] = mfma32x32x16<TP>(a, pf[kt][u], st.o[tt]);
        }
      }

    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  }
}

template <typename ST>
struct OlStash {
  uint32_t h[4][8];
  __device__ __forceinline__ void save(const f32x16 (&o)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) h[t][j] = pack2<F16>(o[t][2 * j], o[t][2 * j + 1]);
  }
  __device__ __forceinline__ float get(int t, int r) const {
    return f16_bits_to_float((uint16_t)(h[t][r >> 1] >> (16 * (r & 1))));
  }
};
template <>
struct OlStash<F32> {
  f32x16 o[4];
  __device__ __forceinline__ void save(const f32x16 (&x)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = x[t];
  }
  __device__ __forceinline__ float get(int t, int r) const { return o[t][r]; }
};

template <typename ST>
__device__ __forceinline__ void store_stat(void* base, int64_t idx, float v) {
  ((typename ST::storage*)base)[idx] = Cvt<ST>::from_f(v);
}

// Token-major store of a wave's 32 x 128 output tile: lane writes 4 consecutive columns per (t, r/4).
template <typename T>
__device__ __forceinline__ void store_token_major(void* out, int d, int col0, int qrow, bool ok, const f32x16 (&o)[4]) {
  if (!ok) return;
  const int hi = (threadIdx.x & 63) >> 5;
  uint16_t* base = (uint16_t*)out + (int64_t)qrow * d + col0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int c = 32 * t + 8 * rq + 4 * hi;
      u32x2 w = u32x2{pack2<T>(o[t][4 * rq + 0], o[t][4 * rq + 1]), pack2<T>(o[t][4 * rq + 2], o[t][4 * rq + 3])};
      *(u32x2*)(base + c) = w;
    }
}

// MODE 0: dual stream; MODE 1: single stream over all rows; MODE 2: single stream over the local rows.
// T: type of Q, K and of the token-major output; TP: type of P and V in the PV product; ST: statistics.
template <typename T, typename TP, typename ST, int MODE>
__global__ __launch_bounds__(NTHREADS, 2) void attn_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int n_blocks = p.n_qblk * p.n_heads;
  const int logical = xcd_remap(blockIdx.x, n_blocks);
  const int head = logical / p.n_qblk;
  const int qblk = logical % p.n_qblk;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int qrow = qblk * BM + wave * 32 + (lane & 31);
  const bool qok = qrow < p.n_q;
  const int col0 = head * HD;

  // Q^T B-operand fragments: lane (n = query, k = 16 ks + 8 hi + 0..7)
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = qok ? *(const u32x4*)(p.q + (int64_t)qrow * p.d + col0 + 16 * ks + 8 * hi) : u32x4{0, 0, 0, 0};

  const int n_k = p.n_sink + p.n_hist + p.n_cur;
  BranchState st;
  if (MODE == 1) {
    Branch all{0, n_k, 0, n_k};
    run_branch<T, TP>(p, all, qf, col0, lds, st);
  } else {
    Branch loc{0, p.n_sink, p.n_sink + p.n_hist, p.n_sink + p.n_cur};
    run_branch<T, TP>(p, loc, qf, col0, lds, st);
  }
  float L = st.lsum + __shfl_xor(st.lsum, 32);
  float inv = 1.f / L;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[t][r] *= inv;

  if (MODE != 0) {
    store_token_major<T>(p.a_full, p.d, col0, qrow, qok, st.o);
    return;
  }

  // ---- dual stream: local branch done
  const float m_loc = st.m, l_loc = L;
  if (p.lse_loc && qok && hi == 0) p.lse_loc[(int64_t)head * p.n_q + qrow] = (m_loc + __log2f(l_loc)) * kLn2;
  if (p.a_loc_t && qok) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = col0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        store_stat<ST>(p.a_loc_t, (int64_t)c * p.ld_stat + qrow, st.o[t][r]);
      }
  }
  // Keep A_loc for the merge while the history branch runs: fp32 when the statistics are fp32,
  // otherwise packed fp16 (the statistics are rounded to 16 bits anyway).
  OlStash<ST> ol;
  ol.save(st.o);

  Branch hist{p.n_sink, p.n_hist, 0, p.n_hist};
  run_branch<T, TP>(p, hist, qf, col0, lds, st);
  const float l_h = st.lsum + __shfl_xor(st.lsum, 32);
  const float m_h = st.m;
  // merge through the log-sum-exp states
  const float mm = fmaxf(m_loc, m_h);
  const float a = l_loc * __builtin_amdgcn_exp2f(m_loc - mm);
  const float b = l_h > 0.f ? l_h * __builtin_amdgcn_exp2f(m_h - mm) : 0.f;
  const float w = b / (a + b);
  const float inv_h = l_h > 0.f ? 1.f / l_h : 0.f;
  if (p.lse_hist && qok && hi == 0)
    p.lse_hist[(int64_t)head * p.n_q + qrow] = l_h > 0.f ? (m_h + __log2f(l_h)) * kLn2 : -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float da = w * (st.o[t][r] * inv_h - ol.get(t, r));
      st.o[t][r] = da;  // reuse as dA
    }
  if (p.delta_a_t && qok) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = col0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        store_stat<ST>(p.delta_a_t, (int64_t)c * p.ld_stat + qrow, st.o[t][r]);
      }
  }
  if (p.a_full) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[t][r] += ol.get(t, r);
    store_token_major<T>(p.a_full, p.d, col0, qrow, qok, st.o);
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 path (any head_dim in {64, 128}): plain VALU online softmax, keys staged through LDS.
// HD/32 threads share one query; each owns 32 dimensions of q and of the outputs.
// ---------------------------------------------------------------------------------------------
template <int HDF>
struct F32Cfg {
  static constexpr int TPQ = HDF / 32;          // threads per query
  static constexpr int QPB = NTHREADS / TPQ;    // queries per work-group
  static constexpr int KT = 32;                 // keys per tile
};

struct F32State {
  float o[32];
  float m, l;
};

template <int HDF>
__device__ __forceinline__ void f32_branch(const AttnParams& p, const float* __restrict__ k, const float* __restrict__ v,
                           const Branch& br, const float (&qv)[32], int col0, int dim0, float* ks, float* vs,
                           F32State& st) {
  typedef F32Cfg<HDF> C;
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 32; ++c) st.o[c] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
  for (int t0 = 0; t0 < br.len; t0 += C::KT) {
    __syncthreads();
    for (int e = tid; e < C::KT * HDF; e += NTHREADS) {
      const int rr = e / HDF, cc = e % HDF;
      const int vi = t0 + rr;
      float kv = 0.f, vv = 0.f;
      if (vi < br.len) {
        const int64_t off = (int64_t)br.row(vi) * p.d + col0 + cc;
        kv = k[off];
        vv = v[off];
      }
      ks[rr * HDF + cc] = kv;
      vs[rr * HDF + cc] = vv;
    }
    __syncthreads();
    const int nvalid = min(C::KT, br.len - t0);
    float s[C::KT];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < C::KT; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc = fmaf(qv[c], ks[j * HDF + dim0 + c], acc);
#pragma unroll
      for (int o = 1; o < C::TPQ; o <<= 1) acc += __shfl_xor(acc, o);
      s[j] = j < nvalid ? acc * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(st.m, mx);
    const float alpha = exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < 32; ++c) st.o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < C::KT; ++j) {
      const float pj = exp2f(s[j] - m_new);
      st.l += pj;
#pragma unroll
      for (int c = 0; c < 32; ++c) st.o[c] = fmaf(pj, vs[j * HDF + dim0 + c], st.o[c]);
    }
    st.m = m_new;
  }
}

template <int HDF, int MODE>
__global__ __launch_bounds__(NTHREADS) void attn_f32_kernel(AttnParams p) {
  typedef F32Cfg<HDF> C;
  __shared__ float ks[C::KT * HDF];
  __shared__ float vs[C::KT * HDF];
  const int n_blocks = p.n_qblk * p.n_heads;
  const int logical = xcd_remap(blockIdx.x, n_blocks);
  const int head = logical / p.n_qblk;
  const int qblk = logical % p.n_qblk;
  const int tid = threadIdx.x;
  const int qrow = qblk * C::QPB + tid / C::TPQ;
  const int dim0 = (tid % C::TPQ) * 32;
  const bool qok = qrow < p.n_q;
  const int col0 = head * HDF;
  const float* q = (const float*)p.q;
  const float* k = (const float*)p.k;
  const float* v = (const float*)p.v;
  float qv[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) qv[c] = qok ? q[(int64_t)qrow * p.d + col0 + dim0 + c] : 0.f;
  const int n_k = p.n_sink + p.n_hist + p.n_cur;
  F32State st;
  if (MODE == 1) {
    Branch all{0, n_k, 0, n_k};
    f32_branch<HDF>(p, k, v, all, qv, col0, dim0, ks, vs, st);
  } else {
    Branch loc{0, p.n_sink, p.n_sink + p.n_hist, p.n_sink + p.n_cur};
    f32_branch<HDF>(p, k, v, loc, qv, col0, dim0, ks, vs, st);
  }
  const float inv = 1.f / st.l;
  float ol[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) ol[c] = st.o[c] * inv;
  if (MODE != 0) {
    if (qok)
      for (int c = 0; c < 32; ++c) ((float*)p.a_full)[(int64_t)qrow * p.d + col0 + dim0 + c] = ol[c];
    return;
  }
  const float m_loc = st.m, l_loc = st.l;
  if (p.lse_loc && qok && dim0 == 0) p.lse_loc[(int64_t)head * p.n_q + qrow] = (m_loc + log2f(l_loc)) * kLn2;
  if (p.a_loc_t && qok)
    for (int c = 0; c < 32; ++c) ((float*)p.a_loc_t)[(int64_t)(col0 + dim0 + c) * p.ld_stat + qrow] = ol[c];
  Branch hist{p.n_sink, p.n_hist, 0, p.n_hist};
  f32_branch<HDF>(p, k, v, hist, qv, col0, dim0, ks, vs, st);
  const float mm = fmaxf(m_loc, st.m);
  const float a = l_loc * exp2f(m_loc - mm);
  const float b = st.l > 0.f ? st.l * exp2f(st.m - mm) : 0.f;
  const float w = b / (a + b);
  const float inv_h = st.l > 0.f ? 1.f / st.l : 0.f;
  if (p.lse_hist && qok && dim0 == 0)
    p.lse_hist[(int64_t)head * p.n_q + qrow] = st.l > 0.f ? (st.m + log2f(st.l)) * kLn2 : -INFINITY;
  if (!qok) return;
  for (int c = 0; c < 32; ++c) {
    const float da = w * (st.o[c] * inv_h - ol[c]);
    const int col = col0 + dim0 + c;
    if (p.delta_a_t) ((float*)p.delta_a_t)[(int64_t)col * p.ld_stat + qrow] = da;
    if (p.a_full) ((float*)p.a_full)[(int64_t)qrow * p.d + col] = ol[c] + da;
  }
}

AttnParams make_params(const AttnLaunch& L) {
  AttnParams p;
  p.q = (const uint16_t*)L.q;
  p.k = (const uint16_t*)L.k;
  p.v = (const uint16_t*)L.v;
  p.a_full = L.a_full;
  p.a_loc_t = L.a_loc_t;
  p.delta_a_t = L.delta_a_t;
  p.ld_stat = L.ld_stat;
  p.lse_loc = L.lse_loc;
  p.lse_hist = L.lse_hist;
  p.n_q = L.n_q;
  p.n_sink = L.n_sink;
  p.n_hist = L.n_hist;
  p.n_cur = L.n_cur;
  p.n_heads = L.n_heads;
  p.d = L.n_heads * L.head_dim;
  p.scale_log2 = L.scale * kLog2e;
  return p;
}

// bf16 -> fp16 copy of V (exact for |v| < 65504), so the PV product of the statistics path can run
// with fp16 probabilities.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                          int64_t n8) {
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 x = ((const u32x4*)in)[i];
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = pack2<F16>(bf16_bits_to_float((uint16_t)(x[j] & 0xFFFFu)), bf16_bits_to_float((uint16_t)(x[j] >> 16)));
    ((u32x4*)out)[i] = y;
  }
}

template <typename T, typename TP, int MODE>
hipError_t launch_mfma_stat(AttnParams p, int stat, hipStream_t s) {
  dim3 grid(p.n_qblk * p.n_heads), block(NTHREADS);
  if (MODE != 0 || stat == DT_F16)
    hipLaunchKernelGGL((attn_mfma_kernel<T, TP, F16, MODE>), grid, block, 0, s, p);
  else if (stat == DT_BF16)
    hipLaunchKernelGGL((attn_mfma_kernel<T, TP, BF16, MODE>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<T, TP, F32, MODE>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int MODE>
hipError_t launch_mfma_mode(AttnParams p, const AttnLaunch& L, hipStream_t s) {
  p.n_qblk = (p.n_q + BM - 1) / BM;
  if (attn_needs_f16_values(L)) {
    // statistics requested in fp16 from bf16 inputs: P and V in fp16 for the PV product
    const int64_t n = (int64_t)(L.n_sink + L.n_hist + L.n_cur) * L.n_heads * L.head_dim;
    const int64_t n8 = n / 8;
    const int blocks = (int)((n8 + 255) / 256 < 2048 ? (n8 + 255) / 256 : 2048);
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)L.v, (uint16_t*)L.ws, n8);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.v = (const uint16_t*)L.ws;
    return launch_mfma_stat<T, F16, MODE>(p, L.stat, s);
  }
  return launch_mfma_stat<T, T, MODE>(p, L.stat, s);
}

template <int HDF, int MODE>
hipError_t launch_f32_mode(AttnParams p, hipStream_t s) {
  p.n_qblk = (p.n_q + F32Cfg<HDF>::QPB - 1) / F32Cfg<HDF>::QPB;
  dim3 grid(p.n_qblk * p.n_heads), block(NTHREADS);
  hipLaunchKernelGGL((attn_f32_kernel<HDF, MODE>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& L, hipStream_t s) {
  AttnParams p = make_params(L);
  if (L.io == DT_F32) {
    if (L.head_dim == 64) {
      if (L.mode == 0) return launch_f32_mode<64, 0>(p, s);
      if (L.mode == 1) return launch_f32_mode<64, 1>(p, s);
      return launch_f32_mode<64, 2>(p, s);
    }
    if (L.mode == 0) return launch_f32_mode<128, 0>(p, s);
    if (L.mode == 1) return launch_f32_mode<128, 1>(p, s);
    return launch_f32_mode<128, 2>(p, s);
  }
  if (L.io == DT_BF16) {
    if (L.mode == 0) return launch_mfma_mode<BF16, 0>(p, L, s);
    if (L.mode == 1) return launch_mfma_mode<BF16, 1>(p, L, s);
    return launch_mfma_mode<BF16, 2>(p, L, s);
  }
  if (L.mode == 0) return launch_mfma_mode<F16, 0>(p, L, s);
  if (L.mode == 1) return launch_mfma_mode<F16, 1>(p, L, s);
  return launch_mfma_mode<F16, 2>(p, L, s);
}

}  // namespace ispa
