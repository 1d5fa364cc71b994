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
//  * one work-group = 256 queries of one head: 8 waves x 32 queries, one work-group per CU,
//    two waves per SIMD;
//  * the two groups of four waves ping-pong: while one group runs its matrix phase
//    (S^T = K Q^T of the next key tile and O^T += V^T P^T of the current one) the other
//    runs its softmax phase (VALU), and every phase ends in a work-group barrier, so the
//    matrix cores and the vector ALUs of a SIMD are busy at the same time;
//  * keys stream through three-deep LDS rings of K tiles (64 keys x 128 dims) and V^T tiles
//    (128 dims x 64 keys, read from a transposed copy of V that the call writes first), padded
//    row pitches, filled with direct global-to-LDS loads two tiles ahead; every ring slot is its
//    own LDS array, so the compiler can tell a slot being filled from a slot being read and only
//    the explicit waits below order them;
//  * a branch is a virtual row range made of up to two physical segments; the local branch
//    (sink + current chunk) and the history branch form one tile sequence, the local state is
//    closed when the first history tile is reached;
//  * S^T = K Q^T with 32x32x16 MFMA: every lane owns one query, so the softmax max/sum are
//    in-lane plus one exchange between lanes l and l^32 (v_permlane32_swap);
//  * O^T = V^T P^T with 32x32x16 MFMA: P^T stays in registers -- the K rows of the QK operand
//    are loaded in a permuted order so that a lane's accumulator registers are exactly its PV
//    B operand over 8 consecutive keys -- and V^T is one plain 16-byte LDS read per MFMA (the
//    transposing LDS read delivers a third of the bandwidth of plain reads on gfx950);
//  * exp2 with the softmax scale folded into log2(e); the reference max only moves when a
//    tile's max exceeds it by more than 2^8; with fp16 probabilities the row sum adds the
//    rounded values with packed dot products (fewer instructions than fp32 adds, although
//    v_dot2 shares the matrix pipeline);
//  * each group issues the direct-to-LDS loads of the tile two ahead at the start of its
//    softmax phase: the memory pipeline accepts a burst only at its own pace, which stalls the
//    issuing wave, and the softmax phase is the shorter one;
//  * when the statistics are requested in fp16 from bf16 inputs, V is copied to fp16 first and
//    the probabilities are rounded to fp16 (11-bit mantissa) for the PV product, which keeps dA
//    accurate enough for ill-conditioned absorption problems; QK^T stays in bf16;
//  * blockIdx -> (head, query block) is XCD-aware so the work-groups of one head share an L2.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace ispa {

namespace {

constexpr int HD = 128;          // head dim of the MFMA path
constexpr int BN = 64;           // keys per tile
constexpr int WAVES = 8;
constexpr int MFMA_THREADS = WAVES * 64;
constexpr int BM = WAVES * 32;   // queries per work-group of the MFMA path
constexpr int NTHREADS = 256;    // fp32 path
constexpr float kLazyLimit = 8192.f;   // 2^13: a lane's partial row sum that triggers a rescale
// LDS tiles are row-major with padded pitches: every MFMA operand read is a per-lane base address
// plus an immediate offset, and 16 consecutive lanes of a 16-byte read hit 16 distinct 4-bank groups.
// K tiles are 64 key rows x 128 head dims; V tiles are transposed: 128 head-dim rows x 64 keys.
constexpr int K_PITCH = HD * 2 + 16;              // 272 bytes per key row
constexpr int VT_PITCH = BN * 2 + 16;             // 144 bytes per head-dim row
constexpr int K_SLOTS = K_PITCH / 16;             // 16-byte slots per row (the last one padding)
constexpr int VT_SLOTS = VT_PITCH / 16;
constexpr int K_TILE = BN * K_PITCH;
constexpr int V_TILE = HD * VT_PITCH;
constexpr int K_INST = BN * K_SLOTS / 64;         // wave-wide 16-byte loads per K tile (17)
constexpr int V_INST = HD * VT_SLOTS / 64;        // per V^T tile (18)
constexpr int LOADS_PER_WAVE = (K_INST + V_INST + WAVES - 1) / WAVES;   // 5: every wave issues the same count
static_assert(K_SLOTS * BN % 64 == 0 && VT_SLOTS * HD % 64 == 0, "tile must be whole wave loads");


// The key tiles of one launch: up to three segments of consecutive cache rows, each cut into 64-row
// tiles (the last one partial).  Dual stream: sink rows, current-chunk rows (together the local
// branch) and history rows (the history branch, starting at tile t_hist); single stream: one
// segment of all rows, or the sink and current-chunk segments.  A tile never crosses a segment
// boundary, so every tile is 64 consecutive rows; rows past the segment's end are loaded too (the
// next segment, or zeros past the end of the buffer) and masked.
struct Sched {
  // segment g: first cache row r_g, row count l_g, one past its last tile index e_g (scalars, no
  // arrays: everything here stays in SGPRs)
  int r0, r1, r2, l0, l1, l2, e0, e1, e2;
  int n, t_hist;
  __device__ __forceinline__ void set(int ra, int la, int rb, int lb, int rc, int lc) {
    r0 = ra; l0 = la; r1 = rb; l1 = lb; r2 = rc; l2 = lc;
    e0 = (la + BN - 1) / BN;
    e1 = e0 + (lb + BN - 1) / BN;
    e2 = e1 + (lc + BN - 1) / BN;
    n = e2;
  }
  // first cache row of tile t and its number of valid rows
  __device__ __forceinline__ int row(int t) const {
    return t < e0 ? r0 + BN * t : t < e1 ? r1 + BN * (t - e0) : r2 + BN * (t - e1);
  }
  __device__ __forceinline__ int valid(int t) const {
    return t < e0 ? l0 - BN * t : t < e1 ? l1 - BN * (t - e0) : l2 - BN * (t - e1);
  }
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* vt;   // 16-bit path: V^T [d, ldv]
  int ldv;
  void* stash;          // dual stream: parked local outputs, kAttnStashBytesPerBlock per work-group
  void* a_full;       // token-major, io dtype
  void* a_loc_t;      // feature-major, stat dtype
  void* delta_a_t;    // feature-major, stat dtype
  int64_t ld_stat;
  float* lse_loc;
  float* lse_hist;
  int n_q, n_sink, n_hist, n_cur, n_heads, d, n_qblk;
  float scale_log2;
};

// Load group k = {K tile k, V^T tile k-1}: K_INST + V_INST wave-wide direct-to-LDS loads (16 bytes
// per lane, buffer addressing), dealt round-robin to the 8 waves, LOADS_PER_WAVE each (the few left
// over repeat the last V^T load, identical data).  Load `inst` of a tile with PITCH-byte rows puts
// lane l on slot 64 inst + l of the tile: row (64 inst + l) / SLOTS, 16-byte chunk (64 inst + l) % SLOTS;
// a lane on a padding slot loads its row's last chunk again (padding is never read).  A lane's byte
// offset within the tile is fixed; the tile's first key is the scalar offset.
// Buffer offsets are 32-bit, the caches are not: the V^T descriptor covers this work-group's head only
// (128 rows of the copy), and every K tile gets a descriptor based at its own first row, so no offset
// grows with the cache length (a 14B-shaped layer's K passes 2^31 bytes at 209,716 rows).
struct Loader {
  __amdgpu_buffer_rsrc_t rv;
  const char* kb;    // K [n_k, d] as bytes
  int64_t kbytes;    // n_k * d * 2
  uint32_t off[LOADS_PER_WAVE];
  __device__ __forceinline__ void init(const AttnParams& p, int n_k, int wave, int lane, int head) {
    // raw buffers: reads past the end return zeros.  Word 3 (0x00020000) is the untyped-access
    // descriptor of gfx9.
    kb = (const char*)p.k;
    kbytes = (int64_t)n_k * p.d * 2;
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.vt + (int64_t)head * HD * p.ldv), (short)0,
                                           (int)((int64_t)HD * p.ldv * 2), 0x00020000);
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) {
      const int idx = wave + WAVES * j;
      if (idx < K_INST) {
        const int slot = 64 * idx + lane;
        off[j] = (uint32_t)((slot / K_SLOTS) * p.d + min(slot % K_SLOTS, 15) * 8) * 2u;
      } else {
        const int slot = 64 * min(idx - K_INST, V_INST - 1) + lane;
        off[j] = (uint32_t)((slot / VT_SLOTS) * p.ldv + min(slot % VT_SLOTS, 7) * 8) * 2u;
      }
    }
  }
  // Every wave issues exactly LOADS_PER_WAVE loads per group, also past the ends of the tile
  // sequence (then a valid tile is loaded again into a ring slot nobody reads), so the number of
  // loads in flight is the same on every path and one wait count fits all iterations.
  struct Group {
    __amdgpu_buffer_rsrc_t rk;   // K from the tile's first row to the end of the cache
    uint32_t sk, sv;             // byte offsets of the head's columns in K and of the V^T tile
    char* kt;
    char* vt;
  };
  __device__ __forceinline__ Group group(const Sched& sc, int k, const AttnParams& p, int head, char* kt,
                                         char* vt) const {
    const int tk = min(k, sc.n - 1);
    const int tv = min(max(k - 1, 0), sc.n - 1);
    const int64_t k0 = (int64_t)sc.row(tk) * p.d * 2;
    const int64_t rest = kbytes - k0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kb + k0), (short)0, (int)(rest < INT32_MAX ? rest : INT32_MAX), 0x00020000);
    return Group{rk, (uint32_t)(head * HD * 2), (uint32_t)sc.row(tv) * 2u, kt, vt};
  }
  __device__ __forceinline__ void issue_one(const Group& g, int j, int wave) const {
    const int idx = wave + WAVES * j;
    if (idx < K_INST) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rk, (lds_void*)(g.kt + 1024 * idx), 16, off[j], g.sk, 0, 0);
    } else {
      const int vi = min(idx - K_INST, V_INST - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(g.vt + 1024 * vi), 16, off[j], g.sv, 0, 0);
    }
  }
  __device__ __forceinline__ void issue(const Group& g, int wave) const {
#pragma unroll
    for (int j = 0; j < LOADS_PER_WAVE; ++j) issue_one(g, j, wave);
  }
};

// Online-softmax state of one branch for the 32 queries of a wave.
struct BranchState {
  f32x16 o[4];     // O^T accumulators: d tile t, lane l, reg r -> d = 32t + 8(r/4) + 4(l/32) + r%4
  float m;         // running reference max (log2 units), identical in lanes l and l^32
  float lsum;      // partial row sum over this lane's keys
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    m = -INFINITY;
    lsum = 0.f;
  }
};

// value of x in lane l ^ 32, combined with x: v_permlane32_swap exchanges the two wave halves.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + lo + hi of two packed fp16 values (one v_dot2c_f32_f16).
__device__ __forceinline__ float add_f16_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
}

// Matrix phase of one wave: S^T = K Q^T for the next tile and O^T += V^T P^T for the current one.
// kt/vt are the ring slots holding that K and V tile.  The phase is 8 steps of 2 QK and 2 PV MFMAs;
// the LDS operands of step i+1 are read while step i runs, and scheduling barriers keep the compiler
// from hoisting more reads than that (registers are at their limit).
struct MatrixOps {
  u32x4 a0, a1;   // K rows of the two 32-key halves, 16 head dims
  u32x4 b[2];     // V^T operands of the two PV MFMAs
};

// K rows are read in the order key(m) = m with bits 2 and 3 swapped (lane m of the A operand loads
// key row key(m)).  Then accumulator register r of S^T holds key 32 kt + 16 (r/8) + 8 (l/32) + r%8,
// so the 8 probabilities a lane packs for PV step (kt, u) are the consecutive keys
// 32 kt + 16 u + 8 (l/32) + 0..7 -- exactly the reduction index of its B operand -- and the matching
// V^T operand is one 16-byte read of 8 consecutive keys.
__device__ __forceinline__ int key_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ MatrixOps matrix_ops(const char* kb, const char* vb, int i) {
  MatrixOps m;
  m.a0 = *(const u32x4*)(kb + 32 * i);
  m.a1 = *(const u32x4*)(kb + 32 * K_PITCH + 32 * i);
  // PV step c = (kt, u, tt): A[d = 32 tt + l%32][k = 8 (l/32) + j] = V^T[d][32 kt + 16 u + 8 (l/32) + j]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 2 * i + h;
    const int kt = c >> 3, u = (c >> 2) & 1, tt = c & 3;
    m.b[h] = *(const u32x4*)(vb + 32 * tt * VT_PITCH + (32 * kt + 16 * u) * 2);
  }
  return m;
}

template <typename T, typename TP>
__device__ __forceinline__ void matrix_phase(const char* kt, const char* vt, int kbase, int vbase,
                                             const u32x4 (&qf)[8], const u32x4 (&pf)[2][2], f32x16 (&s)[2],
                                             f32x16 (&o)[4]) {
  const char* kb = kt + kbase;
  const char* vb = vt + vbase;
  MatrixOps cur = matrix_ops(kb, vb, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    MatrixOps nxt;
    if (i < 7) nxt = matrix_ops(kb, vb, i + 1);
    // accumulator register r of lane l: key 32 kt + 8 (r/4) + 4 (l/32) + r%4 of the rows read (see key_row)
    s[0] = mfma32x32x16<T>(cur.a0, qf[i], i == 0 ? f32x16{} : s[0]);
    s[1] = mfma32x32x16<T>(cur.a1, qf[i], i == 0 ? f32x16{} : s[1]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * i + h;
      o[c & 3] = mfma32x32x16<TP>(cur.b[h], pf[c >> 3][(c >> 2) & 1], o[c & 3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i < 7) cur = nxt;
  }
}

// Softmax phase of one wave for a tile whose scores are in s: mask, running max, probabilities
// (rounded to TP and packed as the PV B operand), row sum.
template <typename TP>
__device__ __forceinline__ void softmax_phase(f32x16 (&s)[2], int valid, float scale_log2, int hi, BranchState& st,
                                              u32x4 (&pf)[2][2]) {
  if (valid < BN) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 16 * (r >> 3) + 8 * hi + (r & 7);   // see key_row
        if (key >= valid) s[kt][r] = -INFINITY;
      }
  }
  // probabilities against a reference max (packed as the PV operand) and this lane's partial row sum
  auto probs = [&](float m_ref) -> float {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * u + j], scale_log2, -m_ref));
        const u32x4 w = u32x4{pack2<TP>(e[0], e[1]), pack2<TP>(e[2], e[3]), pack2<TP>(e[4], e[5]), pack2<TP>(e[6], e[7])};
        pf[kt][u] = w;
        if (std::is_same<TP, F16>::value) {
          // fp16 probabilities: add the rounded values the PV product consumes (relative rounding
          // 2^-12 each, well inside the LSE tolerance), four packed dot products with (1, 1)
          rs0 = add_f16_pair(w[0], rs0);
          rs1 = add_f16_pair(w[1], rs1);
          rs0 = add_f16_pair(w[2], rs0);
          rs1 = add_f16_pair(w[3], rs1);
        } else {
          // bf16 rounding (2^-9) would show in the LSE: add the fp32 values
          rs0 += (e[0] + e[1]) + (e[2] + e[3]);
          rs1 += (e[4] + e[5]) + (e[6] + e[7]);
        }
      }
    return rs0 + rs1;
  };
  // The reference max is not recomputed per tile: the probabilities are taken against the running
  // reference, and only when a lane's partial sum exceeds 2^kLazyLog2 (some probability would, or
  // overflowed, or the reference is still -inf) does the tile compute its max, move the reference
  // (O and the row sum rescaled, for the whole wave at once) and redo its probabilities.  Between
  // rescales every probability stays below 2^kLazyLog2, well inside fp16.  The final normalisation
  // uses the same reference, so this is exact.
  float rs = probs(st.m);
  if (__builtin_amdgcn_ballot_w64(!(rs <= kLazyLimit)) != 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = max_xor32(mx) * scale_log2;
    const float m_new = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.lsum *= alpha;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[tt][r] *= alpha;
    rs = probs(m_new);
  }
  st.lsum += rs;
}

// The local-branch output O_L of a wave, parked in the workspace while the history branch runs
// (registers are the scarce resource there): fp16 pairs, or fp32 when the statistics are fp32.  A
// wave's slot holds NREG dwords per lane; the merge reads them back two values at a time.
template <typename ST>
struct OlStash {
  static constexpr int NREG = 32;
  static constexpr bool kInterleaved = true;   // word k of lane l at slot[64 k + l]: 256 contiguous bytes per store
  uint32_t* slot;
  __device__ __forceinline__ void save(const f32x16 (&o)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) slot[(8 * t + j) * 64] = pack2<F16>(o[t][2 * j], o[t][2 * j + 1]);
  }
  // the words of output tile t (NREG / 4), read back; then the values (t, 2j) and (t, 2j + 1)
  __device__ __forceinline__ void load_words(int t, uint32_t (&w)[NREG / 4]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = slot[(8 * t + j) * 64];
  }
  __device__ __forceinline__ void decode(const uint32_t (&w)[NREG / 4], int j, float& a, float& b) const {
    a = f16_bits_to_float((uint16_t)(w[j] & 0xFFFFu));
    b = f16_bits_to_float((uint16_t)(w[j] >> 16));
  }
};
template <>
struct OlStash<F32> {
  static constexpr int NREG = 64;
  // each lane's 64 words contiguous (one base address, 16-byte stores): the word-major layout of the
  // fp16 stash needs more address registers here than the kernel has to spare
  static constexpr bool kInterleaved = false;
  uint32_t* slot;
  __device__ __forceinline__ void save(const f32x16 (&x)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(slot + 16 * t + 4 * q) = f32x4{x[t][4 * q], x[t][4 * q + 1], x[t][4 * q + 2], x[t][4 * q + 3]};
  }
  __device__ __forceinline__ void load_words(int t, uint32_t (&w)[NREG / 4]) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *(const u32x4*)(slot + 16 * t + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * q + e] = v[e];
    }
  }
  __device__ __forceinline__ void decode(const uint32_t (&w)[NREG / 4], int j, float& a, float& b) const {
    a = __uint_as_float(w[2 * j]);
    b = __uint_as_float(w[2 * j + 1]);
  }
};
static_assert(OlStash<F32>::NREG * 64 * 4 * WAVES == kAttnStashBytesPerBlock && BM == kAttnQueriesPerBlock,
              "stash slot size");

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

// Closes a branch: O <- O / l; returns the full row sum l (both lane halves).
__device__ __forceinline__ float close_branch(BranchState& st) {
  const float L = sum_xor32(st.lsum);
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[t][r] *= inv;
  return L;
}

// MODE 0: dual stream; MODE 1: single stream over all rows; MODE 2: single stream over the local rows.
// T: type of Q, K and of the token-major output; TP: type of P and V in the PV product; ST: statistics.
template <typename T, typename TP, typename ST, int MODE>
__global__ __launch_bounds__(MFMA_THREADS, 2) void attn_mfma_kernel(AttnParams p) {
  // three-deep K and V rings, one LDS array per slot
  __shared__ __attribute__((aligned(16))) char k0[K_TILE];
  __shared__ __attribute__((aligned(16))) char k1[K_TILE];
  __shared__ __attribute__((aligned(16))) char k2[K_TILE];
  __shared__ __attribute__((aligned(16))) char v0[V_TILE];
  __shared__ __attribute__((aligned(16))) char v1[V_TILE];
  __shared__ __attribute__((aligned(16))) char v2[V_TILE];
  const int n_blocks = p.n_qblk * p.n_heads;
  const int logical = xcd_remap(blockIdx.x, n_blocks);
  const int head = logical / p.n_qblk;
  const int qblk = logical % p.n_qblk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int grp = wave >> 2;   // waves 0-3 and 4-7 alternate between matrix and softmax phases
  const int hi = lane >> 5;
  const int qrow = qblk * BM + wave * 32 + (lane & 31);
  const bool qok = qrow < p.n_q;
  // Local-only mode: a wave whose 32 queries all lie past n_q (the last query block of a head) still
  // issues its share of the tile loads and meets every barrier, but runs no matrix or softmax work
  // (the chip runs at a power-limited clock, so idle matrix cores let the busy ones run faster).  The
  // dual and full modes keep every wave working: a block that ran ahead of the other blocks of its
  // head would stop sharing their K and V lines in L2 (HBM fetches per dual call rose by a quarter).
  const bool live = MODE != 2 || qblk * BM + wave * 32 < p.n_q;
  const int col0 = head * HD;

  // Q^T B-operand fragments: lane (n = query, k = 16 ks + 8 hi + 0..7)
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = qok ? *(const u32x4*)(p.q + (int64_t)qrow * p.d + col0 + 16 * ks + 8 * hi) : u32x4{0, 0, 0, 0};

  const int n_k = p.n_sink + p.n_hist + p.n_cur;
  Sched sc;
  if (MODE == 1) {
    sc.set(0, n_k, 0, 0, 0, 0);
    sc.t_hist = sc.n;
  } else {
    sc.set(0, p.n_sink, p.n_sink + p.n_hist, p.n_cur, p.n_sink, MODE == 0 ? p.n_hist : 0);
    sc.t_hist = sc.e1;
  }

  Loader ld;
  ld.init(p, n_k, wave, lane, head);
  // Ring slots are chosen at compile time (the iteration loop below is unrolled by the ring depth),
  // so the compiler's memory-dependency analysis sees which slot each in-flight load writes.
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
  // load group k: K tile k into K slot k % 3, V^T tile k-1 into V slot (k-1) % 3
  ld.issue(ld.group(sc, 0, p, head, k0, v2), wave);
  ld.issue(ld.group(sc, 1, p, head, k1, v0), wave);
  ld.issue(ld.group(sc, 2, p, head, k2, v1), wave);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  lds_barrier();

  const int kbase = key_row(lane & 31) * K_PITCH + hi * 16;
  const int vbase = (lane & 31) * VT_PITCH + hi * 16;

  BranchState st;
  f32x16 s[2];
  u32x4 pf[2][2];
  OlStash<ST> ol;
  ol.slot = (uint32_t*)p.stash + (size_t)(blockIdx.x * WAVES + wave) * OlStash<ST>::NREG * 64 +
            (OlStash<ST>::kInterleaved ? lane : lane * OlStash<ST>::NREG);
  float m_loc = -INFINITY, l_loc = 0.f;

  // Matrix phase M(t) = QK(t+1) + PV(t) reads K slot (t+1) % 3 and V slot t % 3.  M(-1) only needs
  // QK(0): its PV runs on whatever the registers and V slot 2 hold and O is cleared afterwards;
  // M(n-1) only needs PV(n-1): its QK result is never used.
  auto matrix = [&](auto J, int t) {   // J = (t + 1) % 3
    constexpr int j = decltype(J)::value;
    if (live) matrix_phase<T, TP>(kslot(J), vslot(std::integral_constant<int, (j + 2) % 3>{}), kbase, vbase, qf, pf, s, st.o);
    if (t < 0) st.reset();
  };
  // load group i+2 (J = i % 3)
  auto issue_ahead = [&](auto J, int i) {
    constexpr int j = decltype(J)::value;
    ld.issue(ld.group(sc, i + 2, p, head, kslot(std::integral_constant<int, (j + 2) % 3>{}),
                      vslot(std::integral_constant<int, (j + 1) % 3>{})), wave);
  };
  auto softmax = [&](int t) {
    if (!live || t < 0 || t >= sc.n) return;
    if (MODE == 0 && t == sc.t_hist) {
      // first history tile: the local branch is complete
      m_loc = st.m;
      l_loc = close_branch(st);
      ol.save(st.o);
      st.reset();
    }
    softmax_phase<TP>(s, sc.valid(t), p.scale_log2, hi, st, pf);
  };
  auto phase_end = [&]() { lds_barrier(); };
  // Iteration i covers two phases.  Waves 0-3 run M(i-1) and then the softmax of tile i; waves 4-7,
  // one phase behind, run the softmax of tile i-1 and then M(i-1).  Load group k (K tile k, V^T tile
  // k-1) is issued during the softmax phases of iteration k-2 (groups 0-2 before the loop; iteration 0
  // loads group 2 again) and waited for at the end of iteration k-1, when only group k+1 may stay in
  // flight; the ring slots it overwrites were last read in the second phase of iteration k-3.
  // J = i % 3.
  auto wait_loads = [&](int) { __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_WAVE)); };
  // the two wave groups run separate copies of the loop (one branch per group, outside the loop)
  auto iteration0 = [&](auto J, int i) {
    matrix(J, i - 1);
    phase_end();
    issue_ahead(J, i);
    softmax(i);
    wait_loads(i);
    phase_end();
  };
  auto iteration1 = [&](auto J, int i) {
    issue_ahead(J, i);
    softmax(i - 1);
    phase_end();
    matrix(J, i - 1);
    wait_loads(i);
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
  if (MODE != 0) {
    close_branch(st);
    store_token_major<T>(p.a_full, p.d, col0, qrow, qok, st.o);
    return;
  }

  // ---- dual stream: merge the local and history states through their log-sum-exp
  if (!(sc.n > sc.t_hist)) {
    // no history rows: the live state is the local branch; dA = 0 and A_full = A_loc
    m_loc = st.m;
    l_loc = close_branch(st);
    if (p.lse_loc && qok && hi == 0) p.lse_loc[(int64_t)head * p.n_q + qrow] = (m_loc + __log2f(l_loc)) * kLn2;
    if (p.lse_hist && qok && hi == 0) p.lse_hist[(int64_t)head * p.n_q + qrow] = -INFINITY;
    if (qok) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t c = col0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (p.a_loc_t) store_stat<ST>(p.a_loc_t, c * p.ld_stat + qrow, st.o[t][r]);
          if (p.delta_a_t) store_stat<ST>(p.delta_a_t, c * p.ld_stat + qrow, 0.f);
        }
    }
    if (p.a_full) store_token_major<T>(p.a_full, p.d, col0, qrow, qok, st.o);
    return;
  }
  // the live state is the history branch; the local one is parked in the stash
  const float m_h = st.m;
  const float l_h = close_branch(st);
  if (p.lse_loc && qok && hi == 0) p.lse_loc[(int64_t)head * p.n_q + qrow] = (m_loc + __log2f(l_loc)) * kLn2;
  if (p.lse_hist && qok && hi == 0)
    p.lse_hist[(int64_t)head * p.n_q + qrow] = l_h > 0.f ? (m_h + __log2f(l_h)) * kLn2 : -INFINITY;
  const float mm = fmaxf(m_loc, m_h);
  const float a = l_loc * __builtin_amdgcn_exp2f(m_loc - mm);
  const float b = l_h > 0.f ? l_h * __builtin_amdgcn_exp2f(m_h - mm) : 0.f;
  const float w = b / (a + b);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // this wave's stash stores have completed
  // A_loc read back from the stash (the loads of a tile, or of all four for the fp16 stash, issued
  // together, ahead of the stores), then per pair of values dA = w (O_H - A_loc) and
  // A_full = A_loc + dA (st.o becomes A_full)
  constexpr int WPT = OlStash<ST>::NREG / 4;
  constexpr bool all_first = OlStash<ST>::NREG == 32;
  uint32_t words[4][WPT];
  if constexpr (all_first)
#pragma unroll
    for (int t = 0; t < 4; ++t) ol.load_words(t, words[t]);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (!all_first) ol.load_words(t, words[t]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float lo[2];
      ol.decode(words[t], j, lo[0], lo[1]);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * j + e;
        const int64_t c = col0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float da = l_h > 0.f ? w * (st.o[t][r] - lo[e]) : 0.f;
        if (qok && p.a_loc_t) store_stat<ST>(p.a_loc_t, c * p.ld_stat + qrow, lo[e]);
        if (qok && p.delta_a_t) store_stat<ST>(p.delta_a_t, c * p.ld_stat + qrow, da);
        st.o[t][r] = lo[e] + da;
      }
    }
  }
  if (p.a_full) store_token_major<T>(p.a_full, p.d, col0, qrow, qok, st.o);
}

// ---------------------------------------------------------------------------------------------
// fp32 path (any head_dim in {64, 128}): plain VALU online softmax, keys staged through LDS.
// HD/32 threads share one query; each owns 32 dimensions of q and of the outputs.
// ---------------------------------------------------------------------------------------------
// A branch of the fp32 path: virtual rows [0, len) mapped onto up to two physical row segments.
struct Branch {
  int start0, len0, start1, len;
  __device__ __forceinline__ int row(int v) const { return v < len0 ? start0 + v : start1 + (v - len0); }
};

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

// V^T copy for the 16-bit path: vt[c, key] = v[key, c] for c < d, key < n_k, and zero for the keys
// [n_k, 64 * gridDim.x) below n_cols (the attention kernel streams up to 63 keys past a segment's
// last row, masked, so they must be finite).  vt points at the first column written, ldv is its row
// pitch.  With CONVERT the values go from bf16 to fp16 (exact for 2^-17 <= |v| <= 65504), for the
// fp16 PV product of the dual stream.  One work-group transposes a 64-key x 64-column block through
// LDS; global reads and writes are 16 bytes per lane along rows.
template <bool CONVERT>
__global__ __launch_bounds__(256) void vt_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, int n_k,
                                                 int d, int64_t ldv, int64_t n_cols) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];   // [key][column]
  const int key0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int r = threadIdx.x >> 3, ch = threadIdx.x & 7;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int key = key0 + r + 32 * pass;
    u32x4 x = u32x4{0, 0, 0, 0};
    if (key < n_k) x = *(const u32x4*)(v + (int64_t)key * d + c0 + 8 * ch);
    if (CONVERT) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[j] = pack2<F16>(bf16_bits_to_float((uint16_t)(x[j] & 0xFFFFu)), bf16_bits_to_float((uint16_t)(x[j] >> 16)));
    }
    *(u32x4*)&tile[r + 32 * pass][8 * ch] = x;
  }
  __syncthreads();
  if (key0 + 8 * ch >= n_cols) return;   // n_cols is a multiple of 8: whole 16-byte chunks
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = r + 32 * pass;
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = (uint32_t)tile[8 * ch + 2 * j][c] | ((uint32_t)tile[8 * ch + 2 * j + 1][c] << 16);
    *(u32x4*)(vt + (int64_t)(c0 + c) * ldv + key0 + 8 * ch) = y;
  }
}

template <typename T, typename TP, int MODE>
hipError_t launch_mfma_stat(AttnParams p, int stat, hipStream_t s) {
  dim3 grid(p.n_qblk * p.n_heads), block(MFMA_THREADS);
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
  const int n_k = L.n_sink + L.n_hist + L.n_cur;
  if (L.vt) {
    // the caller's V^T, already in the PV product's type
    p.ldv = (int)L.ldv;
    p.vt = (const uint16_t*)L.vt;
    p.stash = L.ws;
  } else {
    p.ldv = (int)attn_vt_ld(n_k);
    p.vt = (const uint16_t*)L.ws;
    p.stash = (char*)L.ws + attn_vt_bytes_aligned(n_k, p.d);
    const dim3 tgrid(p.ldv / 64, p.d / 64);
    // bf16 inputs of the dual stream: P and V in fp16 for the PV product
    if (attn_needs_f16_values(L))
      hipLaunchKernelGGL(vt_kernel<true>, tgrid, dim3(256), 0, s, (const uint16_t*)L.v, (uint16_t*)L.ws, n_k, p.d,
                         (int64_t)p.ldv, (int64_t)p.ldv);
    else
      hipLaunchKernelGGL(vt_kernel<false>, tgrid, dim3(256), 0, s, (const uint16_t*)L.v, (uint16_t*)L.ws, n_k, p.d,
                         (int64_t)p.ldv, (int64_t)p.ldv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the dual stream's PV product always runs on fp16 probabilities (with an fp16 V^T copy from bf16
  // inputs); the single streams keep the input type
  if constexpr (MODE == 0)
    return launch_mfma_stat<T, F16, MODE>(p, L.stat, s);
  else
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

hipError_t launch_transpose_rows(const void* v, int rows, int d, bool convert, void* vt, int64_t ldv, int64_t col0,
                                 hipStream_t s) {
  const int64_t n_cols = ldv - col0;
  const int64_t span = ((int64_t)rows + 63) / 64 * 64 + 64;   // the rows, then at least 64 zero columns
  const int64_t cover = span < n_cols ? span : (n_cols + 63) / 64 * 64;
  if (cover == 0) return hipSuccess;   // col0 == ldv: no column to write
  const dim3 grid((unsigned)(cover / 64), (unsigned)(d / 64));
  uint16_t* dst = (uint16_t*)vt + col0;
  if (convert)
    hipLaunchKernelGGL(vt_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)v, dst, rows, d, ldv, n_cols);
  else
    hipLaunchKernelGGL(vt_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)v, dst, rows, d, ldv, n_cols);
  return hipGetLastError();
}

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
