/*
 * ispa.h -- C ABI of the ISPA hot path for AMD Instinct MI355X (gfx950).
 *
 * Instance-Specific Parametric Absorption ("Towards Memory-Efficient
 * Autoregressive Video Generation via Instance-Specific Parametric
 * Absorption"; gist.science technical summary, section 2 "Methodology")
 * turns selected full-attention layers of an autoregressive video model into
 * local-attention layers.  During a short warmup each layer computes, in one
 * pass, the attention output over the whole KV cache (A_full) and over local
 * context only (A_loc: sink tokens + current chunk); at the transition point
 * a closed-form ridge regression absorbs the missing history into the
 * layer's output projection, dW = (A_loc^T A_loc + lambda I)^-1
 * A_loc^T (A_full - A_loc) W; converted layers then run on local context with
 * W + dW.
 *
 * Conventions for every call
 * --------------------------
 *  * Pointers to tensors are DEVICE pointers owned by the caller; the library
 *    never frees them and never keeps them after the call returns.
 *  * Every call only enqueues work on `stream` (a hipStream_t, 0 = the null
 *    stream) and returns without synchronising.  Outputs are ready when the
 *    stream reaches that point.  The solves that factorise panel by panel
 *    (ispa_absorb_solve_batched, and ispa_absorb_solve for d > 2048) fork the
 *    part that the factorisation does not read to an auxiliary stream of the
 *    current device (owned by the library, created on first use, default
 *    priority) and join it back onto `stream` by events before they return,
 *    so under graph capture it joins the capture.
 *  * Dense row-major layouts.  Token tensors are [tokens, d] with heads as
 *    contiguous column blocks: head h owns columns [h*head_dim, (h+1)*head_dim).
 *    The projection convention is y = A W with W [d_in, d_out] (a PyTorch
 *    nn.Linear stores W^T).
 *  * Device pointers must be 16-byte aligned.
 *  * Return value: ISPA_OK or an error status for everything the host can
 *    check (arguments, sizes, workspace, launch errors).  When a call returns
 *    an error nothing has been enqueued, except ISPA_EHIP, which reports a
 *    failed launch.  NaN/Inf inputs are propagated, not detected.
 *  * Calls are reentrant; calls on different streams may run concurrently if
 *    their outputs do not overlap.  The only global state is per device: the
 *    solves' auxiliary stream (its fork-join sequence runs under a mutex) and
 *    the scratch array of ispa_local_attn_fused_proj_noalloc.
 */
#ifndef ISPA_H
#define ISPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { ISPA_F32 = 0, ISPA_BF16 = 1, ISPA_F16 = 2 };

/* status codes */
enum {
  ISPA_OK = 0,
  ISPA_EINVAL = 1,        /* NULL required pointer, bad size, misaligned pointer */
  ISPA_EUNSUPPORTED = 2,  /* head_dim or dtype combination not implemented      */
  ISPA_EWORKSPACE = 3,    /* workspace missing or smaller than required         */
  ISPA_EHIP = 4           /* a kernel launch or HIP runtime call failed         */
};

/* call ids for ispa_workspace_bytes */
enum { ISPA_CALL_DUAL_ATTN = 0, ISPA_CALL_ABSORB_SOLVE = 1, ISPA_CALL_LOCAL_ATTN_PROJ = 2,
       ISPA_CALL_LOCAL_ATTN_PROJ_W8A8 = 3, ISPA_CALL_LOCAL_ATTN_FP8 = 4, ISPA_CALL_LOCAL_ATTN_FP8_PROJ_W8A8 = 5,
       ISPA_CALL_DUAL_ATTN_VT = 6 };

/*
 * One layer's KV cache, rows in this order:
 *   [0, n_sink)                          sink tokens (e.g. the first latent frame)
 *   [n_sink, n_sink + n_hist)            cached history
 *   [n_sink + n_hist, n_k)               the current chunk,  n_k = n_sink + n_hist + n_cur
 * The local set is sink + current chunk ("current frame and sink tokens",
 * technical summary section 2, stage 1 "Dual-Stream Warmup"); the history set
 * is the rows in between.  Queries are the n_q tokens of the current chunk
 * and attend to every row of their set (no mask).
 */
typedef struct ispa_attn_shape {
  int32_t n_q;
  int32_t n_sink;
  int32_t n_hist;
  int32_t n_cur;
  int32_t n_heads;
  int32_t head_dim;  /* 64 or 128 */
  float scale;       /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
} ispa_attn_shape;

/*
 * ispa_dual_attn -- dual-stream (decomposable) attention.
 * Technical summary section 2, stage 1 "Dual-Stream Warmup": A_full (whole
 * history, the ground truth) and A_loc (sink + current chunk) from one pass,
 * by running online softmax separately over the local and the history rows
 * and merging the two partial results through their log-sum-exp states.
 *
 *   q      [n_q, d]  io_dtype          k, v  [n_k, d]  io_dtype
 *   a_full [n_q, d]  io_dtype          attention over all n_k rows (nullable in dual mode)
 *   a_loc_t, delta_a_t : FEATURE-MAJOR [d, ld_stat] in stat_dtype, columns [0, n_q) written:
 *          a_loc_t[c*ld_stat + i]   = A_loc[i, c]
 *          delta_a_t[c*ld_stat + i] = (A_full - A_loc)[i, c], computed as
 *                                     w_hist * (O_hist - A_loc) (no cancellation)
 *          ld_stat >= n_q and a multiple of 8.  Pointing at column offset j0 of a
 *          wider buffer lets warmup chunks be stacked for one Gram call.
 *   lse_loc, lse_hist  [n_heads, n_q] fp32, natural log; lse_hist = -inf when n_hist = 0.
 *
 * Modes: if a_loc_t, delta_a_t, lse_loc and lse_hist are all NULL the call runs
 * single-stream attention over all n_k rows into a_full (an F-layer after the
 * warmup); otherwise it runs the dual stream and writes the non-NULL outputs.
 * dtypes: io_dtype BF16 or F16 (MFMA path; stat_dtype F16, BF16 or F32) or
 * F32 (stat_dtype F32).  Requires n_q >= 1, n_sink + n_cur >= 1 (an empty local
 * set is EINVAL), n_hist >= 0.
 * Workspace: BF16/F16 inputs need ispa_workspace_bytes(ISPA_CALL_DUAL_ATTN,
 * shape, 0) bytes (16-byte aligned; EWORKSPACE otherwise): the call first writes
 * a transposed copy of V there, which the attention kernel streams, and the dual
 * stream parks the local-branch outputs there while the history branch runs.
 * Calls that share a workspace must not overlap in time.  F32 inputs
 * need none (workspace may be NULL).  The 16-bit path addresses one head's
 * rows of the copy with 32-bit byte offsets: n_k must stay below 8,388,544
 * (EUNSUPPORTED); K and V themselves may exceed 2^31 bytes.
 * Precision: QK^T and PV run on MFMA with fp32 accumulation.  In dual mode
 * (any statistics dtype, or none) the PV product uses fp16 probabilities; with
 * BF16 inputs the V copy is converted to fp16, for all outputs, A_full
 * included.  That conversion is exact for bf16 values with
 * 2^-17 <= |v| <= 65504 and for 0; smaller magnitudes become fp16 subnormals and
 * lose low bits (below 2^-25 they become 0) and larger ones become inf.  The
 * single-stream mode and F16 inputs use the input type for P and V.
 */
int ispa_dual_attn(const ispa_attn_shape* shape, int io_dtype,
                   const void* q, const void* k, const void* v,
                   void* a_full,
                   int stat_dtype, void* a_loc_t, void* delta_a_t, int64_t ld_stat,
                   float* lse_loc, float* lse_hist,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_dual_attn_vt -- ispa_dual_attn with V supplied transposed by the caller.
 * The same operation (technical summary section 2, stage 1 "Dual-Stream
 * Warmup"), for callers that keep V^T next to their cache: the cached rows of
 * V are then transposed once, when they are appended (ispa_transpose_rows),
 * instead of on every call.  Outputs are bit-identical to ispa_dual_attn's on
 * the same values.
 *
 *   vt      [d, ldv] in vt_dtype: vt[c*ldv + r] = V[r, c] for the n_k cache rows
 *           r (same row order as ispa_dual_attn's v).  vt_dtype is the type the
 *           PV product runs on: F16 in dual mode (BF16 or F16 inputs; bf16 values
 *           converted as ispa_dual_attn does), io_dtype in single-stream mode;
 *           EINVAL otherwise.  ldv >= n_k, ldv % 8 == 0, 128 * ldv * 2 < 2^31
 *           (EUNSUPPORTED).  The kernel streams up to 63 columns past a
 *           segment's last row as masked keys, whose probabilities are zero:
 *           columns [n_k, min(ldv, n_k + 64)) must hold finite values (the zeros
 *           ispa_transpose_rows leaves after the rows it writes qualify).
 *   Other arguments as ispa_dual_attn; io_dtype BF16 or F16 only (F32:
 *   EUNSUPPORTED).  Workspace: ispa_workspace_bytes(ISPA_CALL_DUAL_ATTN_VT,
 *   shape, 0) bytes in dual mode (the parked local outputs); none (NULL) in
 *   single-stream mode.  vt is only read.
 */
int ispa_dual_attn_vt(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, int vt_dtype,
                      const void* vt, int64_t ldv, void* a_full, int stat_dtype, void* a_loc_t, void* delta_a_t,
                      int64_t ld_stat, float* lse_loc, float* lse_hist, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * ispa_transpose_rows -- appends cache rows to a caller-owned V^T.
 * Writes vt[c*ldv + col0 + r] = V[r, c] for r < rows, c < d, from v [rows, d]
 * (row-major, v_dtype BF16 or F16), converted to vt_dtype (F16, or v_dtype;
 * bf16 -> fp16 as ispa_dual_attn converts), then sets the next 64 to 127
 * columns (those below ldv) to zero, so the columns past the last rows a call
 * wrote are finite for ispa_dual_attn_vt.  Requires d % 64 == 0, d <= 65536,
 * rows >= 0, col0 and ldv multiples of 8, col0 + rows <= ldv, v and vt 16-byte
 * aligned.  Stream-ordered, no workspace.
 */
int ispa_transpose_rows(int rows, int d, int v_dtype, const void* v, int vt_dtype, void* vt, int64_t ldv,
                        int64_t col0, void* stream);

/*
 * ispa_gram_accum -- the absorption statistics over warmup tokens.
 * The closed form of technical summary section 2, stage 2 "Layer Absorb"
 * needs G = A_loc^T A_loc and C = A_loc^T (A_full - A_loc); the reconstruction
 * error used by the layer selection also needs D = dA^T dA.  All three are sums
 * over tokens, so chunks can be accumulated call by call.
 *
 *   a_loc_t, delta_a_t : [d, ld] feature-major, stat_dtype (F16, BF16 or F32),
 *                        columns [0, n) are the tokens; ld >= n, ld % 8 == 0.
 *   G, C, D            : [d, d] fp32 row-major.  accumulate = 0 overwrites,
 *                        1 adds.  G and D are symmetric and written in full.
 *   D may be NULL.  d % 32 == 0 and d <= 16384; n >= 1.  16-bit statistics are
 *   read in 256-row slices with 32-bit byte offsets: 512 * ld must stay below
 *   2^31 (EUNSUPPORTED).  Token columns [n, ld) are never read as data (they may
 *   hold anything, NaN included).
 */
int ispa_gram_accum(int d, int n, int stat_dtype, const void* a_loc_t, const void* delta_a_t, int64_t ld,
                    int accumulate, float* G, float* C, float* D, void* stream);

/*
 * ispa_absorb_solve -- closed-form ridge absorption.
 * Technical summary section 2, stage 2 "Layer Absorb": the minimiser of
 * ||A_loc (W + dW) - A_full W||_F^2 + lambda ||dW||_F^2 is
 * dW = (G + lambda I)^-1 C W, obtained without iteration.  Computed as
 * R = C W, a blocked Cholesky factorisation G + lambda I = L L^T, and the two
 * triangular solves, all to fp32 accuracy (R, and W W^T for eps, on the bf16
 * matrix cores from three-part bf16 splits of C and W that carry all 24 bits
 * of their fp32 values); refine = n (0..8) adds n steps of iterative
 * refinement.  Each forms the residual C W - (G + lambda I) dW as exact int8
 * products of 7-bit fixed-point digits (5 per value, scaled per row of C and G
 * and per column of W and dW), about 35 bits relative to those rows' and
 * columns' largest entries, and corrects dW with the fp32 factor.  Refinement
 * reduces dW's error down to the residual's accuracy (not to that of an fp64
 * solve): one step brings an ill-conditioned layer (features > warmup tokens,
 * cond ~ 2e6 at d = 5120) from the fp32 solve's error to within 4e-3 of the
 * float64 dW, as an fp64 residual does.
 *
 *   G, C [d, d] fp32 (from ispa_gram_accum); D [d, d] fp32, needed only for eps.
 *   W [d, d] in w_dtype (F32, BF16 or F16).
 *   lambda_relative = 0: lambda as given; 1: lambda * tr(G) / d.
 *   delta_w [d, d] fp32 out.
 *   w_new  [d, d] w_dtype out, W + dW rounded to nearest (nullable).
 *   eps    device fp32 scalar out (nullable; requires D): the reconstruction error
 *          ||A_loc (W + dW) - A_full W||_F / ||A_full W||_F of section 2
 *          "Dynamic layer selection", evaluated from G, C, D, W and dW alone.
 *   lambda_out device fp32 scalar out: the lambda used (nullable).
 *   info   device int out (required): 0 on success; k > 0 when the leading
 *          minor of order k of G + lambda I is not positive definite (LAPACK
 *          potrf convention); then delta_w, w_new and eps are undefined.
 *          -2: a wait inside the one-launch factorisation (one layer,
 *          d <= 2048) timed out, which needs the device to be held by other
 *          work for about a second; the outputs are then undefined.
 *   Execution: for one layer with d <= 2048 the factorisation runs as one
 *   launch whose work-groups exchange blocks through device memory and
 *   version flags (each work-group takes a CU; work-group 0 carries the
 *   chain of diagonal blocks); otherwise, and for every batched call, as one
 *   launch per 64-wide panel.  Both give the same results bit for bit.
 *   workspace: at least ispa_workspace_bytes(ISPA_CALL_ABSORB_SOLVE, NULL, d) bytes.
 *   d % 32 == 0, 32 <= d <= 16384.
 */
int ispa_absorb_solve(int d, const float* G, const float* C, const float* D,
                      int w_dtype, const void* W,
                      float lambda, int lambda_relative, int refine,
                      float* delta_w, void* w_new, float* eps, float* lambda_out, int* info,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_absorb_solve_batched -- ispa_absorb_solve for n_layers independent
 * layers in one call (the transition absorbs every layer at once; each layer's
 * solve alone leaves most of the GPU idle, since its Cholesky panels are a
 * sequential chain).  Same arguments, results and errors as ispa_absorb_solve,
 * per layer l:
 *   G, C, D, W, delta_w, w_new  [n_layers, d, d] contiguous (layer l at l*d*d),
 *   eps, lambda_out, info       [n_layers] (nullable as in ispa_absorb_solve),
 *   workspace: n_layers * ispa_workspace_bytes(ISPA_CALL_ABSORB_SOLVE, NULL, d)
 *   bytes, layer l's part at l times that size.  1 <= n_layers <= 65535.
 * Layer l's results equal those of ispa_absorb_solve on layer l's arrays, bit for
 * bit (the same kernels with the layer as a grid dimension).
 */
int ispa_absorb_solve_batched(int n_layers, int d, const float* G, const float* C, const float* D,
                              int w_dtype, const void* W, float lambda, int lambda_relative, int refine,
                              float* delta_w, void* w_new, float* eps, float* lambda_out, int* info,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_select_layers -- which layers become local-attention layers.
 * Technical summary section 2, "Dynamic layer selection": after the warmup the
 * layers are ranked by their reconstruction error epsilon (ispa_absorb_solve's
 * eps output) and the lowest-error ones are converted.
 *
 *   eps   [n_layers] fp32, device: the per-layer errors.
 *   info  [n_layers] int32, device (nullable): the solves' info words; a layer
 *         with info != 0 (its factorisation failed, its eps is undefined) ranks
 *         as if its eps were NaN.
 *   k     how many layers to convert, 0 <= k <= n_layers.
 *   role  [n_layers] int32, device, out: 1 for the converted layers -- the first
 *         k in rank order whose eps is a number (a layer with NaN eps or info != 0
 *         is never converted, so fewer than k are when fewer than k errors are
 *         numbers) -- and 0 for the layers that keep full attention.
 *   order [n_layers] int32, device, out (nullable): the layer indices in rank order.
 * Ranking: ascending eps; equal values rank the lower layer index first (a
 * stable sort); NaN ranks after every number.  1 <= n_layers <= 4096.
 */
int ispa_select_layers(int n_layers, const float* eps, const int32_t* info, int k, int32_t* role, int32_t* order,
                       void* stream);

/*
 * ispa_local_attn_fused_proj -- one step of a converted L-layer.
 * Technical summary section 2, stage 3 "Memory-Efficient Inference": after the
 * warmup the selected layers attend to local context only (sink + current
 * chunk) and project with the updated weights W_new = W + dW.
 *
 *   out = softmax(Q K_loc^T * scale) V_loc  @  w_new
 *   q [n_q, d], k/v [n_k, d] with the layout of ispa_attn_shape (history rows,
 *   if any, are skipped), w_new [d, d], out [n_q, d]; all io_dtype BF16 or F16.
 *   workspace: at least ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_PROJ, shape, d)
 *   bytes, 16-byte aligned (the local attention output between the two kernels,
 *   the transposed copy of V and a transposed copy of w_new); n_k below
 *   8,388,544 and n_q * d * 2 below 2^31 (ISPA_EUNSUPPORTED otherwise).
 */
int ispa_local_attn_fused_proj(const ispa_attn_shape* shape, int io_dtype,
                               const void* q, const void* k, const void* v, const void* w_new,
                               void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_local_attn_fused_proj_wt -- the same L-layer step with the projection
 * given transposed: w_new_t [d_out, d_in] = W_new^T (io_dtype), as
 * ispa_transpose16 writes it once per converted layer at the fold (W_new does
 * not change after the transition, so the per-call transpose of
 * ispa_local_attn_fused_proj is skipped).  Arguments, limits and workspace as
 * ispa_local_attn_fused_proj; the output is bit-identical to it.
 */
int ispa_local_attn_fused_proj_wt(const ispa_attn_shape* shape, int io_dtype,
                                  const void* q, const void* k, const void* v, const void* w_new_t,
                                  void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_transpose16 -- dst [cols, rows] = src [rows, cols]^T for BF16 or F16
 * (dtype), both row-major device arrays, 16-byte aligned, not overlapping;
 * rows and cols multiples of 16, at most 65536 (ISPA_EINVAL otherwise).
 */
int ispa_transpose16(int rows, int cols, int dtype, const void* src, void* dst, void* stream);

/*
 * ispa_local_attn_fused_proj_noalloc -- ispa_local_attn_fused_proj without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and checks as ispa_local_attn_fused_proj
 * (bit for bit: the same kernels run), but the scratch is a fixed array of
 * ispa_noalloc_scratch_bytes() = 64 MiB that the library holds on each GPU it
 * runs on until the process ends; the call allocates nothing.  A shape whose
 * scratch (ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_PROJ, shape, 0)) exceeds
 * it returns ISPA_EWORKSPACE (e.g. n_q 4680, sink 1560, current 4680, d 1536
 * needs 38 MiB and fits; d 5120 does not).  Every call on one GPU uses that
 * GPU's array: calls that overlap in time on one GPU (other streams or host
 * threads) race and must be ordered by the caller.  The first call on a device
 * looks the array's address up (hipGetSymbolAddress) and keeps it; ISPA_EHIP if
 * that fails.
 */
int ispa_local_attn_fused_proj_noalloc(const ispa_attn_shape* shape, int io_dtype,
                                       const void* q, const void* k, const void* v, const void* w_new,
                                       void* out, void* stream);
size_t ispa_noalloc_scratch_bytes(void);

/*
 * W8A8 variant of the L-layer step (FP8 weights and activations).
 * Technical summary section 4 "Results": the method combined with W8A8
 * post-training quantisation gives the largest overall speed-up; the pages
 * name no scheme.  This library reads it as symmetric absmax scaling per
 * channel into OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite value 448):
 *   s = absmax / 448 in float32 (1 for an all-zero channel),
 *   code = E4M3(clamp(x / s, -448, 448)), rounded to nearest even, x / s an
 *   IEEE float32 division.
 * Weights get one scale per output channel, activations one per token; the
 * product is out[i, j] = s_a[i] s_w[j] sum_k dec(Aq[i, k]) dec(Wq[k, j]) with
 * fp32 accumulation, rounded to the io dtype.
 *
 *   ispa_quantize_weight_fp8: W [d_in, d_out] (F32, BF16 or F16) ->
 *     wq_t [d_out, d_in] E4M3 codes (one byte each; W TRANSPOSED, so both
 *     operands of the product are contiguous along d_in) and w_scales [d_out]
 *     fp32.  d_in % 64 == 0, d_out % 4 == 0, both <= 65536.  Run once per
 *     converted layer on W_new.
 *   ispa_local_attn_fused_proj_w8a8: as ispa_local_attn_fused_proj, but the
 *     local attention output (rounded to io_dtype) is quantised per token and
 *     multiplied by the quantised W_new: out = W8A8(LocalAttn(Q; sink +
 *     current), W_new).  workspace: ispa_workspace_bytes(
 *     ISPA_CALL_LOCAL_ATTN_PROJ_W8A8, shape, 0) bytes, 16-byte aligned.  The
 *     attention itself stays in io_dtype (the pages do not say how attention
 *     would be quantised).  n_q * d must stay below 2^31 (EUNSUPPORTED).
 */
int ispa_quantize_weight_fp8(int d_in, int d_out, int w_dtype, const void* w, void* wq_t, float* w_scales,
                             void* stream);
/*   ispa_quantize_rows_fp8: the activation side on its own: x [rows, cols] (row
 *     stride ldx elements; F32, BF16 or F16) -> q [rows, cols] E4M3 codes (row
 *     stride ldq bytes) and scales [rows] fp32, one scale per row.  cols % 8
 *     == 0, ldx % 8 == 0, ldq % 8 == 0 (EINVAL otherwise). */
int ispa_quantize_rows_fp8(int rows, int cols, int dtype, const void* x, int64_t ldx, void* q, int64_t ldq,
                           float* scales, void* stream);
int ispa_local_attn_fused_proj_w8a8(const ispa_attn_shape* shape, int io_dtype,
                                    const void* q, const void* k, const void* v,
                                    const void* wq_t, const float* w_scales,
                                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 attention of a converted layer (the W8A8 variant extended to the attention).
 * Technical summary section 4 "Results" pairs the method with W8A8 quantisation
 * without naming a scheme; read here for the attention of an L-layer as FP8 E4M3
 * operands of both products:
 *   Q: one scale per query token and head, s_q = absmax / 448, codes E4M3(q / s_q);
 *   K, V: one scale per head over the call's key rows (sink + current chunk);
 *   scores in log2 units x = s_q s_k (Qq . Kq) * scale * log2(e);
 *   P = 2^(x - M), M the integer ceiling of the row maximum, coded as E4M3(256 P);
 *   l = sum of the decoded P codes, out = s_v sum_j dec(Pq_j) dec(Vq_j) / l.
 * Scales and quotients are float32 operations (absmax / 448, 1 for an all-zero
 * head or token).  The kernel moves its reference M by whole powers of two only,
 * so its codes equal those taken against the row's final M (up to probabilities
 * below 2^-14 of the row's largest, which E4M3 holds as subnormals).
 *
 *   ispa_local_attn_fp8: out [n_q, d] (io dtype BF16 or F16) = that attention over
 *     the local rows of `shape` (history rows, if any, are not read); q, k, v as in
 *     ispa_local_attn_fused_proj.  workspace: ispa_workspace_bytes(
 *     ISPA_CALL_LOCAL_ATTN_FP8, shape, 0) bytes (K codes, transposed V codes,
 *     scales of the local rows), 16-byte aligned.  head_dim 128; n_sink + n_cur
 *     below 8,388,544 and
 *     n_q * d * 2 below 2^31 (EUNSUPPORTED).
 *   ispa_local_attn_fp8_proj_w8a8: the converted layer in W8A8 end to end: the FP8
 *     attention, its output rounded to the io dtype, then the W8A8 projection of
 *     ispa_local_attn_fused_proj_w8a8 (wq_t, w_scales from
 *     ispa_quantize_weight_fp8).  workspace: ispa_workspace_bytes(
 *     ISPA_CALL_LOCAL_ATTN_FP8_PROJ_W8A8, shape, 0) bytes.
 */
int ispa_local_attn_fp8(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                        void* out, void* workspace, size_t workspace_bytes, void* stream);
int ispa_local_attn_fp8_proj_w8a8(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                                  const void* v, const void* wq_t, const float* w_scales, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV-cache manager -- the K/V storage on either side of the hot path.
 * Technical summary section 2, stage 3 "Memory-Efficient Inference": after the
 * warmup the F-layers keep attending to the whole growing cache while the
 * converted L-layers keep only the sink tokens and the current chunk; their
 * history rows are what the method frees.  A cache object holds, per layer,
 * K and V rows in the order of ispa_attn_shape (sink | history | current),
 * ready to pass to ispa_dual_attn / ispa_local_attn_fused_proj.
 *
 * Unlike the calls above, a cache OWNS device memory.  Each layer's K rows and
 * V rows live in virtual address ranges reserved by ispa_kv_create for
 * sink_rows + max_chunks * chunk_rows rows (address space only); physical
 * memory is mapped behind them as rows arrive (HIP virtual memory management,
 * in whole allocation granules; the sink rows of every layer are mapped by
 * ispa_kv_create) and the pieces past the sink and current chunk are released
 * when a layer is converted.  So the device memory a cache uses follows the
 * rows it holds: nothing beyond the sink rows is committed up front, and the
 * peak over a rollout is the peak of the rows held.  Rows keep their addresses: a
 * layer's K and V pointers stay valid until ispa_kv_destroy.  The calls that
 * map or release memory (write_sink, append_chunk and release_history when they
 * grow or shrink a layer, destroy) may synchronise the device.  A handle is not
 * thread-safe: calls on one handle must come from one host thread at a time.
 * Row data is copied with hipMemcpyAsync on `stream`; the caller's source rows
 * must stay valid until the stream reaches the copy.  HIP failures (mapping,
 * copies) return ISPA_EHIP.
 *
 *   ispa_kv_create: n_layers >= 1 layers of rows of width d (d % 8 == 0) in
 *     dtype (F32, BF16 or F16) on the current device; sink_rows >= 0 sink
 *     rows, chunks of chunk_rows >= 1 rows, at most max_chunks >= 1 chunks per
 *     full layer (total below 2^31 rows).  *out receives the handle (NULL on
 *     error).
 *   ispa_kv_destroy: waits for the device, then frees the handle and its
 *     memory (NULL is a no-op).
 *   ispa_kv_write_sink: copies sink_rows rows of k and v ([sink_rows, d]
 *     each) into the sink rows of `layer`.
 *   ispa_kv_append_chunk: copies one chunk (chunk_rows rows of k and v).  A
 *     full layer appends it after its rows (the previous current chunk becomes
 *     history; EINVAL once max_chunks chunks are held); a converted layer
 *     overwrites its current chunk.
 *   ispa_kv_release_history: converts a full layer: its current chunk is
 *     copied next to the sink rows, the stream is synchronised (earlier work may
 *     still read the history) and the memory past sink + current chunk is
 *     released.  EINVAL if the layer is already converted.
 *   ispa_kv_layer: the layer's K and V base pointers and rows[0..2] = n_sink,
 *     n_hist, n_cur for ispa_attn_shape.
 *   ispa_kv_bytes: *held_bytes = bytes of K and V rows the layers hold
 *     (sink + history + current of full layers, sink + current of converted
 *     ones: the quantity the method reduces); *reserved_bytes = bytes of device
 *     memory mapped behind them (held bytes rounded up to allocation granules).
 */
typedef struct ispa_kv_cache ispa_kv_cache;

int ispa_kv_create(int n_layers, int d, int dtype, int32_t sink_rows, int32_t chunk_rows, int32_t max_chunks,
                   ispa_kv_cache** out);
int ispa_kv_destroy(ispa_kv_cache* kv);
int ispa_kv_write_sink(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream);
int ispa_kv_append_chunk(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream);
int ispa_kv_release_history(ispa_kv_cache* kv, int layer, void* stream);
int ispa_kv_layer(const ispa_kv_cache* kv, int layer, void** k, void** v, int32_t* rows);
int ispa_kv_bytes(const ispa_kv_cache* kv, int64_t* held_bytes, int64_t* reserved_bytes);

/* Workspace bytes a call needs (0 if none).  `shape` is used by the attention
 * calls, `d` by ISPA_CALL_ABSORB_SOLVE.  Returns (size_t)-1 for an unknown call. */
size_t ispa_workspace_bytes(int call_id, const ispa_attn_shape* shape, int d);

/* Static string for a status code. */
const char* ispa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int ispa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ISPA_H */
