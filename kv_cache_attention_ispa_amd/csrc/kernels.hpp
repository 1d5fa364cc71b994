// Internal launch interface between the C ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ispa {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

struct AttnLaunch {
  int mode;  // 0: dual stream, 1: single stream over all rows, 2: single stream over the local rows
  int io, stat;
  const void* q;
  const void* k;
  const void* v;
  void* a_full;
  void* a_loc_t;
  void* delta_a_t;
  int64_t ld_stat;
  float* lse_loc;
  float* lse_hist;
  int n_q, n_sink, n_hist, n_cur, n_heads, head_dim;
  float scale;
  void* ws;          // device workspace (16-bit inputs: the transposed copy of V, see attn_vt_bytes)
  size_t ws_bytes;
  // 16-bit path: a V^T [d, ldv] the caller keeps (in the PV product's type; columns [n_k, n_k + 64)
  // finite).  When set, no copy is made and the workspace holds only the parked local outputs.
  const void* vt = nullptr;
  int64_t ldv = 0;
};
// The 16-bit (MFMA) path streams V from a transposed copy V^T [d, ldv] (ldv = n_k rounded up to
// 64 keys, pad keys zero) that the call writes into the workspace first.
inline int64_t attn_vt_ld(int64_t n_k) { return (n_k + 63) / 64 * 64; }
inline size_t attn_vt_bytes(int64_t n_k, int64_t d) { return (size_t)(d * attn_vt_ld(n_k) * 2); }
// The dual stream parks each work-group's local outputs (256 queries x 128 dims, up to fp32) in the
// workspace after the V^T copy while the history branch runs.
constexpr int64_t kAttnQueriesPerBlock = 256;
constexpr size_t kAttnStashBytesPerBlock = 256 * 128 * 4;
inline size_t attn_vt_bytes_aligned(int64_t n_k, int64_t d) { return (attn_vt_bytes(n_k, d) + 255) / 256 * 256; }
inline size_t attn_stash_bytes(int64_t n_q, int64_t n_heads) {
  return (size_t)((n_q + kAttnQueriesPerBlock - 1) / kAttnQueriesPerBlock * n_heads) * kAttnStashBytesPerBlock;
}
// Dual stream from bf16 inputs: the PV product runs on fp16 probabilities and the V^T copy is
// converted to fp16 (bf16 probabilities cost the absorption about three times the error of fp16
// ones), whatever the statistics' dtype.
inline bool attn_needs_f16_values(const AttnLaunch& L) { return L.mode == 0 && L.io == DT_BF16; }
hipError_t launch_attention(const AttnLaunch& L, hipStream_t s);
// V rows [rows, d] (16-bit) into columns [col0, col0 + rows) of V^T [d, ldv] (dst[c * ldv + col0 + r]),
// converted from bf16 to fp16 when `convert`; the following 64..127 columns (up to ldv) are set to
// zero.  d % 64 == 0; col0 and ldv multiples of 8.
hipError_t launch_transpose_rows(const void* v, int rows, int d, bool convert, void* vt, int64_t ldv, int64_t col0,
                                 hipStream_t s);
// FP8 attention over the local rows (sink + current chunk; history rows are not read) into L.a_full
// (io dtype), with the codes and scales of those rows of K and V written into L.ws first
// (attn_fp8_workspace_bytes of n_sink + n_cur rows).
size_t attn_fp8_workspace_bytes(int64_t n_loc, int64_t d);
hipError_t launch_attention_fp8(const AttnLaunch& L, hipStream_t s);

// Gram statistics: out_z (+)= X_z Y_z^T for z in {G: (A, A), C: (A, dA), D: (dA, dA)}.
struct GramLaunch {
  int d, n, stat;
  const void* a_t;
  const void* da_t;
  int64_t ld;
  int accumulate;
  float* G;
  float* C;
  float* D;
};
hipError_t launch_gram(const GramLaunch& L, hipStream_t s);

// out[m, n] = a @ b for 16-bit row-major operands (local-layer projection), fp32 accumulate; b is
// first transposed into bt ([n, k], caller-provided scratch).
struct ProjLaunch {
  int io;
  int m, n, k;
  const void* a;   // [m, k]
  const void* b;   // [k, n]
  void* bt;        // [n, k] scratch
  void* out;       // [m, n]
};
hipError_t launch_proj(const ProjLaunch& L, hipStream_t s);
// W [k, n] 16-bit -> W^T [n, k] (k, n multiples of 16), and out [m, n] = A [m, k] (B^T [n, k])^T.
hipError_t launch_transpose16(const void* w, int k, int n, void* wt, hipStream_t s);
hipError_t launch_proj_nt(int io, int m, int n, int k, const void* a, const void* bt, void* out, hipStream_t s);

// W8A8 projection (fp8.hip): per-row E4M3 codes + scales of a [rows, cols] matrix; the weights per
// output channel, written transposed; out[m, n] = (Aq Wq) s_a s_w^T (k % 64 == 0).
hipError_t launch_quant_rows(int dtype, const void* x, int64_t ldx, int rows, int cols, uint8_t* q, int64_t ldq,
                             float* scales, hipStream_t s);
hipError_t launch_quant_weight(int dtype, const void* w, int d_in, int d_out, uint8_t* wq_t, float* scales,
                               hipStream_t s);
// out (fp32 d x d) = sum over n_seg segments g of A_g B_g^T, A_g / B_g the bf16 planes (d x d, row-major,
// consecutive) numbered (a_planes >> 4 g) & 15 and (b_planes >> 4 g) & 15; layer y of batch at
// planes + y layer_bytes and out + y layer_bytes.  d % 64 == 0, 9 d^2 * 2 bytes of planes < 2^32.
// lower: only the 64 x 64 blocks on and below the diagonal are needed (others may stay unwritten).
hipError_t launch_nt_segments(const uint16_t* planes, float* out, int d, int n_seg, int a_planes, int b_planes,
                              int batch, int64_t layer_bytes, bool lower, hipStream_t s);
hipError_t launch_proj8(int out_dtype, const uint8_t* aq, const float* sa, const uint8_t* wq_t, const float* sw,
                        void* out, int m, int n, int k, hipStream_t s);

// One solve per layer for `batch` layers side by side: the caller's d x d arrays (G, C, D, W, delta_w,
// w_new) are [batch, d, d] and eps, lambda_out, info [batch]; layer l's workspace starts at
// ws + l * solve_workspace_bytes(d).
struct SolveLaunch {
  int batch;
  int d;
  const float* G;
  const float* C;
  const float* D;
  int w_dtype;
  const void* W;
  float lambda;
  int lambda_relative;
  int refine;
  float* delta_w;
  void* w_new;
  float* eps;
  float* lambda_out;
  int* info;
  void* ws;
};
size_t solve_workspace_bytes(int d);
hipError_t launch_solve(const SolveLaunch& L, hipStream_t s);

// Refinement residual r = C W - (G + lambda I) dW from int8 digit products (refine.hip), per layer
// (blockIdx.y) with byte steps s_mat (C, G, dW), s_wmat (W), s_ws (ws, r) and s_lambda (lambda).
struct ResidualLaunch {
  int batch, d;
  const float* C;
  const float* G;
  const void* W;
  int w_dtype;
  const float* dW;
  const float* lambda;   // device
  float* r;
  void* ws;              // residual_workspace_bytes(d) per layer
  int rows_too;          // 1: (re)form the digits of [C | -G] (once per solve)
  int64_t s_mat, s_wmat, s_ws, s_lambda;
};
size_t residual_workspace_bytes(int d);
hipError_t launch_residual(const ResidualLaunch& L, hipStream_t s);

}  // namespace ispa
