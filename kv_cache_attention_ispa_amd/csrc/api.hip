// C ABI of the ISPA hot path: argument validation, workspace sizing and launches.
// The operations, layouts and error behaviour are documented in include/ispa.h.
#include "../../include/ispa.h"
#include "kernels.hpp"

#include <math.h>

#include <mutex>

using namespace ispa;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool valid_dtype(int t) { return t == ISPA_F32 || t == ISPA_BF16 || t == ISPA_F16; }

int check_shape(const ispa_attn_shape* s) {
  if (!s) return ISPA_EINVAL;
  if (s->n_q < 1 || s->n_sink < 0 || s->n_hist < 0 || s->n_cur < 0 || s->n_heads < 1) return ISPA_EINVAL;
  if ((int64_t)s->n_sink + s->n_cur < 1) return ISPA_EINVAL;
  if ((int64_t)s->n_sink + s->n_hist + s->n_cur > INT32_MAX) return ISPA_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return ISPA_EUNSUPPORTED;
  if ((int64_t)s->n_heads * s->head_dim > 65536) return ISPA_EINVAL;
  if (!(s->scale == s->scale)) return ISPA_EINVAL;
  return ISPA_OK;
}

float eff_scale(const ispa_attn_shape* s) { return s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim); }

int hip_status(hipError_t e) { return e == hipSuccess ? ISPA_OK : ISPA_EHIP; }

// The local attention output between the two kernels of ispa_local_attn_fused_proj, rounded up to
// 256 bytes; the V^T copy follows it in the workspace.
size_t local_a_bytes(const ispa_attn_shape* s) {
  return ((size_t)s->n_q * s->n_heads * s->head_dim * 2 + 255) / 256 * 256;
}

// The transposed copy of W_new the 16-bit projection reads ([d, d] 16-bit).
size_t w_t_bytes(const ispa_attn_shape* s) {
  const size_t d = (size_t)s->n_heads * s->head_dim;
  return (d * d * 2 + 255) / 256 * 256;
}

// The E4M3 codes of the local attention output and their per-token scales (W8A8 projection).
size_t w8a8_codes_bytes(const ispa_attn_shape* s) {
  return ((size_t)s->n_q * s->n_heads * s->head_dim + 255) / 256 * 256;
}
size_t w8a8_act_bytes(const ispa_attn_shape* s) {
  return w8a8_codes_bytes(s) + ((size_t)s->n_q * 4 + 255) / 256 * 256;
}

// The FP8 attention's codes of K and V and their scales.
size_t fp8_attn_ws(const ispa_attn_shape* s) {
  return attn_fp8_workspace_bytes((int64_t)s->n_sink + s->n_cur, (int64_t)s->n_heads * s->head_dim);
}

// ispa_dual_attn's workspace (16-bit inputs): the V^T copy, then the parked local outputs.
size_t dual_ws_bytes(const ispa_attn_shape* s) {
  return attn_vt_bytes_aligned((int64_t)s->n_sink + s->n_hist + s->n_cur, (int64_t)s->n_heads * s->head_dim) +
         attn_stash_bytes(s->n_q, s->n_heads);
}

// ispa_dual_attn_vt's workspace: only the dual stream's parked local outputs.
size_t dual_vt_ws_bytes(const ispa_attn_shape* s, bool dual) { return dual ? attn_stash_bytes(s->n_q, s->n_heads) : 0; }

// The 16-bit path addresses one head's 128 rows of the V^T copy with 32-bit byte offsets (K tiles get
// descriptors of their own, so K has no such limit).
bool fits_buffer(const ispa_attn_shape* s) {
  const int64_t n_k = (int64_t)s->n_sink + s->n_hist + s->n_cur;
  return 128 * attn_vt_ld(n_k) * 2 < INT32_MAX;
}

// Scratch of ispa_local_attn_fused_proj_noalloc: one array per GPU, part of the code object (so it
// exists once the library is loaded on a device and is never allocated by a call).  Its host-side
// name is only a stand-in; the device address comes from hipGetSymbolAddress, looked up once per
// device on that device's first call and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr when the lookup failed.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// ispa_dual_attn and ispa_dual_attn_vt: V row-major (v, copied to V^T in the workspace by the call)
// or the caller's V^T (vt, ldv, in vt_dtype).
int dual_attn_call(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                   const void* vt, int64_t ldv, int vt_dtype, void* a_full, int stat_dtype, void* a_loc_t,
                   void* delta_a_t, int64_t ld_stat, float* lse_loc, float* lse_hist, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (!valid_dtype(io_dtype)) return ISPA_EUNSUPPORTED;
  if (!q || !k || (!v && !vt)) return ISPA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(vt) || !aligned16(a_full)) return ISPA_EINVAL;
  const bool dual = a_loc_t || delta_a_t || lse_loc || lse_hist;
  if (!dual && !a_full) return ISPA_EINVAL;
  if (a_loc_t || delta_a_t) {
    if (!valid_dtype(stat_dtype)) return ISPA_EUNSUPPORTED;
    if (ld_stat < shape->n_q || ld_stat % 8 != 0) return ISPA_EINVAL;
    if (!aligned16(a_loc_t) || !aligned16(delta_a_t)) return ISPA_EINVAL;
  }
  if (!aligned4(lse_loc) || !aligned4(lse_hist)) return ISPA_EINVAL;
  if (io_dtype == ISPA_F32) {
    if (vt) return ISPA_EUNSUPPORTED;
    if ((a_loc_t || delta_a_t) && stat_dtype != ISPA_F32) return ISPA_EUNSUPPORTED;
  } else {
    if (shape->head_dim != 128 || !fits_buffer(shape)) return ISPA_EUNSUPPORTED;
  }
  const int64_t n_k = (int64_t)shape->n_sink + shape->n_hist + shape->n_cur;
  if (vt) {
    // the PV product's type: fp16 for the dual stream, the input type for the single stream
    if (vt_dtype != (dual ? ISPA_F16 : io_dtype)) return ISPA_EINVAL;
    if (ldv < n_k || ldv % 8 != 0) return ISPA_EINVAL;
    if (128 * ldv * 2 >= INT32_MAX) return ISPA_EUNSUPPORTED;
  }
  AttnLaunch L;
  L.mode = dual ? 0 : 1;
  L.io = io_dtype;
  L.stat = stat_dtype;
  L.q = q;
  L.k = k;
  L.v = v;
  L.vt = vt;
  L.ldv = ldv;
  L.a_full = a_full;
  L.a_loc_t = a_loc_t;
  L.delta_a_t = delta_a_t;
  L.ld_stat = ld_stat;
  L.lse_loc = lse_loc;
  L.lse_hist = lse_hist;
  L.n_q = shape->n_q;
  L.n_sink = shape->n_sink;
  L.n_hist = shape->n_hist;
  L.n_cur = shape->n_cur;
  L.n_heads = shape->n_heads;
  L.head_dim = shape->head_dim;
  L.scale = eff_scale(shape);
  L.ws = workspace;
  L.ws_bytes = workspace_bytes;
  if (io_dtype != ISPA_F32) {
    const size_t need = vt ? dual_vt_ws_bytes(shape, dual) : dual_ws_bytes(shape);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return ISPA_EWORKSPACE;
  }
  return hip_status(launch_attention(L, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int ispa_version(void) { return 100; }

const char* ispa_status_string(int status) {
  switch (status) {
    case ISPA_OK: return "ok";
    case ISPA_EINVAL: return "invalid argument";
    case ISPA_EUNSUPPORTED: return "unsupported head_dim or dtype combination";
    case ISPA_EWORKSPACE: return "workspace missing or too small";
    case ISPA_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

size_t ispa_workspace_bytes(int call_id, const ispa_attn_shape* shape, int d) {
  switch (call_id) {
    case ISPA_CALL_DUAL_ATTN:
      if (!shape || shape->n_heads < 1) return 0;
      return dual_ws_bytes(shape);
    case ISPA_CALL_DUAL_ATTN_VT:
      if (!shape || shape->n_heads < 1) return 0;
      return dual_vt_ws_bytes(shape, true);
    case ISPA_CALL_ABSORB_SOLVE: return d > 0 ? solve_workspace_bytes(d) : 0;
    case ISPA_CALL_LOCAL_ATTN_PROJ:
      if (!shape || shape->n_q < 1 || shape->n_heads < 1) return 0;
      return local_a_bytes(shape) + attn_vt_bytes_aligned((int64_t)shape->n_sink + shape->n_hist + shape->n_cur,
                                                          (int64_t)shape->n_heads * shape->head_dim) +
             w_t_bytes(shape);
    case ISPA_CALL_LOCAL_ATTN_PROJ_W8A8:
      if (!shape || shape->n_q < 1 || shape->n_heads < 1) return 0;
      return local_a_bytes(shape) + attn_vt_bytes_aligned((int64_t)shape->n_sink + shape->n_hist + shape->n_cur,
                                                          (int64_t)shape->n_heads * shape->head_dim) +
             w8a8_act_bytes(shape);
    case ISPA_CALL_LOCAL_ATTN_FP8:
      if (!shape || shape->n_q < 1 || shape->n_heads < 1) return 0;
      return fp8_attn_ws(shape);
    case ISPA_CALL_LOCAL_ATTN_FP8_PROJ_W8A8:
      if (!shape || shape->n_q < 1 || shape->n_heads < 1) return 0;
      return local_a_bytes(shape) + fp8_attn_ws(shape) + w8a8_act_bytes(shape);
    default: return (size_t)-1;
  }
}

int ispa_dual_attn(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                   void* a_full, int stat_dtype, void* a_loc_t, void* delta_a_t, int64_t ld_stat, float* lse_loc,
                   float* lse_hist, void* workspace, size_t workspace_bytes, void* stream) {
  return dual_attn_call(shape, io_dtype, q, k, v, nullptr, 0, 0, a_full, stat_dtype, a_loc_t, delta_a_t, ld_stat,
                        lse_loc, lse_hist, workspace, workspace_bytes, stream);
}

int ispa_dual_attn_vt(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, int vt_dtype,
                      const void* vt, int64_t ldv, void* a_full, int stat_dtype, void* a_loc_t, void* delta_a_t,
                      int64_t ld_stat, float* lse_loc, float* lse_hist, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!vt) return ISPA_EINVAL;
  return dual_attn_call(shape, io_dtype, q, k, nullptr, vt, ldv, vt_dtype, a_full, stat_dtype, a_loc_t, delta_a_t,
                        ld_stat, lse_loc, lse_hist, workspace, workspace_bytes, stream);
}

int ispa_transpose_rows(int rows, int d, int v_dtype, const void* v, int vt_dtype, void* vt, int64_t ldv,
                        int64_t col0, void* stream) {
  if (rows < 0 || d < 64 || d % 64 != 0 || d > 65536) return ISPA_EINVAL;
  if (v_dtype != ISPA_BF16 && v_dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (vt_dtype != ISPA_F16 && vt_dtype != v_dtype) return ISPA_EUNSUPPORTED;
  if ((rows > 0 && !v) || !vt || !aligned16(v) || !aligned16(vt)) return ISPA_EINVAL;
  if (col0 < 0 || col0 % 8 != 0 || ldv % 8 != 0 || col0 + rows > ldv) return ISPA_EINVAL;
  if (ldv - col0 > (int64_t)64 * 65536 * 64) return ISPA_EUNSUPPORTED;
  return hip_status(launch_transpose_rows(v, rows, d, v_dtype == ISPA_BF16 && vt_dtype == ISPA_F16, vt, ldv, col0,
                                          (hipStream_t)stream));
}

int ispa_gram_accum(int d, int n, int stat_dtype, const void* a_loc_t, const void* delta_a_t, int64_t ld,
                    int accumulate, float* G, float* C, float* D, void* stream) {
  if (d < 32 || d > 16384 || d % 32 != 0 || n < 1) return ISPA_EINVAL;
  if (!valid_dtype(stat_dtype)) return ISPA_EUNSUPPORTED;
  if (!a_loc_t || !delta_a_t || !G || !C) return ISPA_EINVAL;
  if (ld < n || ld % 8 != 0) return ISPA_EINVAL;
  // the 16-bit kernel addresses a 256-row slice of a statistic with 32-bit byte offsets, and an offset
  // of 2^31 must fall outside that slice (it is how a load of tokens past n returns zeros)
  if (stat_dtype != ISPA_F32 && ld * 2 * 256 >= INT32_MAX) return ISPA_EUNSUPPORTED;
  if (!aligned16(a_loc_t) || !aligned16(delta_a_t) || !aligned16(G) || !aligned16(C) || !aligned16(D))
    return ISPA_EINVAL;
  if (accumulate != 0 && accumulate != 1) return ISPA_EINVAL;
  GramLaunch L;
  L.d = d;
  L.n = n;
  L.stat = stat_dtype;
  L.a_t = a_loc_t;
  L.da_t = delta_a_t;
  L.ld = ld;
  L.accumulate = accumulate;
  L.G = G;
  L.C = C;
  L.D = D;
  return hip_status(launch_gram(L, (hipStream_t)stream));
}

int ispa_absorb_solve_batched(int n_layers, int d, const float* G, const float* C, const float* D, int w_dtype,
                              const void* W, float lambda, int lambda_relative, int refine, float* delta_w,
                              void* w_new, float* eps, float* lambda_out, int* info, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (n_layers < 1 || n_layers > 65535) return ISPA_EINVAL;
  if (d < 32 || d > 16384 || d % 32 != 0) return ISPA_EINVAL;
  if (!valid_dtype(w_dtype)) return ISPA_EUNSUPPORTED;
  if (!G || !C || !W || !delta_w || !info) return ISPA_EINVAL;
  if (eps && !D) return ISPA_EINVAL;
  if (!(lambda == lambda) || (lambda_relative != 0 && lambda_relative != 1) || refine < 0 || refine > 8)
    return ISPA_EINVAL;
  if (!aligned16(G) || !aligned16(C) || !aligned16(D) || !aligned16(W) || !aligned16(delta_w) || !aligned16(w_new) ||
      !aligned4(eps) || !aligned4(lambda_out) || !aligned4(info))
    return ISPA_EINVAL;
  if (!workspace || workspace_bytes / (size_t)n_layers < solve_workspace_bytes(d) ||
      workspace_bytes < (size_t)n_layers * solve_workspace_bytes(d) || !aligned16(workspace))
    return ISPA_EWORKSPACE;
  SolveLaunch L;
  L.batch = n_layers;
  L.d = d;
  L.G = G;
  L.C = C;
  L.D = D;
  L.w_dtype = w_dtype;
  L.W = W;
  L.lambda = lambda;
  L.lambda_relative = lambda_relative;
  L.refine = refine;
  L.delta_w = delta_w;
  L.w_new = w_new;
  L.eps = eps;
  L.lambda_out = lambda_out;
  L.info = info;
  L.ws = workspace;
  return hip_status(launch_solve(L, (hipStream_t)stream));
}

int ispa_absorb_solve(int d, const float* G, const float* C, const float* D, int w_dtype, const void* W,
                      float lambda, int lambda_relative, int refine, float* delta_w, void* w_new, float* eps,
                      float* lambda_out, int* info, void* workspace, size_t workspace_bytes, void* stream) {
  return ispa_absorb_solve_batched(1, d, G, C, D, w_dtype, W, lambda, lambda_relative, refine, delta_w, w_new, eps,
                                   lambda_out, info, workspace, workspace_bytes, stream);
}

// The 16-bit L-layer step: local attention into the workspace, then the projection by W_new (w_new
// transposed into the workspace first) or by a W_new^T the caller already holds (w_new_t).
static int local_attn_proj16(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                             const void* w_new, const void* w_new_t, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (io_dtype != ISPA_BF16 && io_dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (shape->head_dim != 128 || !fits_buffer(shape)) return ISPA_EUNSUPPORTED;
  if ((int64_t)shape->n_q * shape->n_heads * shape->head_dim * 2 >= INT32_MAX) return ISPA_EUNSUPPORTED;
  const void* w = w_new ? w_new : w_new_t;
  if (!q || !k || !v || !w || !out) return ISPA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(out)) return ISPA_EINVAL;
  const size_t need = ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_PROJ, shape, 0);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ISPA_EWORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  AttnLaunch L;
  L.mode = 2;
  L.io = io_dtype;
  L.stat = ISPA_F16;
  L.q = q;
  L.k = k;
  L.v = v;
  L.a_full = workspace;
  L.a_loc_t = nullptr;
  L.delta_a_t = nullptr;
  L.ld_stat = 0;
  L.lse_loc = nullptr;
  L.lse_hist = nullptr;
  L.n_q = shape->n_q;
  L.n_sink = shape->n_sink;
  L.n_hist = shape->n_hist;
  L.n_cur = shape->n_cur;
  L.n_heads = shape->n_heads;
  L.head_dim = shape->head_dim;
  L.scale = eff_scale(shape);
  const size_t vt_bytes = attn_vt_bytes_aligned((int64_t)shape->n_sink + shape->n_hist + shape->n_cur,
                                                (int64_t)shape->n_heads * shape->head_dim);
  L.ws = (char*)workspace + local_a_bytes(shape);
  L.ws_bytes = vt_bytes;
  hipError_t e = launch_attention(L, s);
  if (e != hipSuccess) return ISPA_EHIP;
  const int d = shape->n_heads * shape->head_dim;
  if (w_new_t) return hip_status(launch_proj_nt(io_dtype, shape->n_q, d, d, workspace, w_new_t, out, s));
  ProjLaunch P;
  P.bt = (char*)workspace + local_a_bytes(shape) + vt_bytes;
  P.io = io_dtype;
  P.m = shape->n_q;
  P.n = d;
  P.k = d;
  P.a = workspace;
  P.b = w_new;
  P.out = out;
  return hip_status(launch_proj(P, s));
}

int ispa_local_attn_fused_proj(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                               const void* v, const void* w_new, void* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!w_new) return ISPA_EINVAL;
  return local_attn_proj16(shape, io_dtype, q, k, v, w_new, nullptr, out, workspace, workspace_bytes, stream);
}

int ispa_local_attn_fused_proj_wt(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                                  const void* v, const void* w_new_t, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!w_new_t) return ISPA_EINVAL;
  return local_attn_proj16(shape, io_dtype, q, k, v, nullptr, w_new_t, out, workspace, workspace_bytes, stream);
}

int ispa_transpose16(int rows, int cols, int dtype, const void* src, void* dst, void* stream) {
  if (dtype != ISPA_BF16 && dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (rows < 16 || cols < 16 || rows % 16 != 0 || cols % 16 != 0 || rows > 65536 || cols > 65536)
    return ISPA_EINVAL;
  if (!src || !dst || src == dst || !aligned16(src) || !aligned16(dst)) return ISPA_EINVAL;
  return hip_status(launch_transpose16(src, rows, cols, dst, (hipStream_t)stream));
}

size_t ispa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int ispa_local_attn_fused_proj_noalloc(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                                       const void* v, const void* w_new, void* out, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  const size_t need = ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_PROJ, shape, 0);
  if (need > kNoAllocScratchBytes) return ISPA_EWORKSPACE;
  // the remaining checks are those of the workspace variant; argument errors come before the lookup
  if (io_dtype != ISPA_BF16 && io_dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (shape->head_dim != 128 || !fits_buffer(shape)) return ISPA_EUNSUPPORTED;
  if (!q || !k || !v || !w_new || !out) return ISPA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w_new) || !aligned16(out)) return ISPA_EINVAL;
  void* ws = noalloc_scratch();
  if (!ws) return ISPA_EHIP;
  return ispa_local_attn_fused_proj(shape, io_dtype, q, k, v, w_new, out, ws, kNoAllocScratchBytes, stream);
}

// shared by the two FP8-attention calls: argument checks and the attention launch into `a` (io dtype)
static int fp8_attention(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                         void* a, void* ws, hipStream_t s) {
  AttnLaunch L;
  L.mode = 2;
  L.io = io_dtype;
  L.stat = ISPA_F16;
  L.q = q;
  L.k = k;
  L.v = v;
  L.a_full = a;
  L.a_loc_t = nullptr;
  L.delta_a_t = nullptr;
  L.ld_stat = 0;
  L.lse_loc = nullptr;
  L.lse_hist = nullptr;
  L.n_q = shape->n_q;
  L.n_sink = shape->n_sink;
  L.n_hist = shape->n_hist;
  L.n_cur = shape->n_cur;
  L.n_heads = shape->n_heads;
  L.head_dim = shape->head_dim;
  L.scale = eff_scale(shape);
  L.ws = ws;
  L.ws_bytes = fp8_attn_ws(shape);
  return hip_status(launch_attention_fp8(L, s));
}

static int fp8_attn_checks(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                           const void* out) {
  int st = check_shape(shape);
  if (st) return st;
  if (io_dtype != ISPA_BF16 && io_dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (shape->head_dim != 128) return ISPA_EUNSUPPORTED;
  const int64_t n_loc = (int64_t)shape->n_sink + shape->n_cur;
  const int64_t d = (int64_t)shape->n_heads * shape->head_dim;
  if (128 * attn_vt_ld(n_loc) >= INT32_MAX || (int64_t)shape->n_q * d * 2 >= INT32_MAX) return ISPA_EUNSUPPORTED;
  if (!q || !k || !v || !out) return ISPA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ISPA_EINVAL;
  return ISPA_OK;
}

int ispa_local_attn_fp8(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k, const void* v,
                        void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = fp8_attn_checks(shape, io_dtype, q, k, v, out);
  if (st) return st;
  if (!workspace || workspace_bytes < fp8_attn_ws(shape) || !aligned16(workspace)) return ISPA_EWORKSPACE;
  return fp8_attention(shape, io_dtype, q, k, v, out, workspace, (hipStream_t)stream);
}

int ispa_local_attn_fp8_proj_w8a8(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                                  const void* v, const void* wq_t, const float* w_scales, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int st = fp8_attn_checks(shape, io_dtype, q, k, v, out);
  if (st) return st;
  if (!wq_t || !w_scales || !aligned16(wq_t) || !aligned4(w_scales)) return ISPA_EINVAL;
  const size_t need = ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_FP8_PROJ_W8A8, shape, 0);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ISPA_EWORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const int d = shape->n_heads * shape->head_dim;
  char* a = (char*)workspace;
  char* fws = a + local_a_bytes(shape);
  uint8_t* aq = (uint8_t*)(fws + fp8_attn_ws(shape));
  float* sa = (float*)(aq + w8a8_codes_bytes(shape));
  st = fp8_attention(shape, io_dtype, q, k, v, a, fws, s);
  if (st) return st;
  if (launch_quant_rows(io_dtype, a, d, shape->n_q, d, aq, d, sa, s) != hipSuccess) return ISPA_EHIP;
  return hip_status(launch_proj8(io_dtype, aq, sa, (const uint8_t*)wq_t, w_scales, out, shape->n_q, d, d, s));
}

int ispa_quantize_weight_fp8(int d_in, int d_out, int w_dtype, const void* w, void* wq_t, float* w_scales,
                             void* stream) {
  if (d_in < 1 || d_out < 1 || d_in % 64 != 0 || d_out % 4 != 0 || d_in > 65536 || d_out > 65536)
    return ISPA_EINVAL;
  if (!valid_dtype(w_dtype)) return ISPA_EINVAL;
  if (!w || !wq_t || !w_scales) return ISPA_EINVAL;
  if (!aligned16(w) || !aligned16(wq_t) || !aligned4(w_scales)) return ISPA_EINVAL;
  return hip_status(launch_quant_weight(w_dtype, w, d_in, d_out, (uint8_t*)wq_t, w_scales, (hipStream_t)stream));
}

int ispa_quantize_rows_fp8(int rows, int cols, int dtype, const void* x, int64_t ldx, void* q, int64_t ldq,
                           float* scales, void* stream) {
  if (rows < 1 || cols < 1 || cols % 8 != 0 || ldx < cols || ldx % 8 != 0 || ldq < cols || ldq % 8 != 0)
    return ISPA_EINVAL;
  if (!valid_dtype(dtype)) return ISPA_EINVAL;
  if (!x || !q || !scales) return ISPA_EINVAL;
  if (!aligned16(x) || !aligned16(q) || !aligned4(scales)) return ISPA_EINVAL;
  return hip_status(launch_quant_rows(dtype, x, ldx, rows, cols, (uint8_t*)q, ldq, scales, (hipStream_t)stream));
}

int ispa_local_attn_fused_proj_w8a8(const ispa_attn_shape* shape, int io_dtype, const void* q, const void* k,
                                    const void* v, const void* wq_t, const float* w_scales, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (io_dtype != ISPA_BF16 && io_dtype != ISPA_F16) return ISPA_EUNSUPPORTED;
  if (shape->head_dim != 128 || !fits_buffer(shape)) return ISPA_EUNSUPPORTED;
  if (!q || !k || !v || !wq_t || !w_scales || !out) return ISPA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wq_t) || !aligned4(w_scales) || !aligned16(out))
    return ISPA_EINVAL;
  const size_t need = ispa_workspace_bytes(ISPA_CALL_LOCAL_ATTN_PROJ_W8A8, shape, 0);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ISPA_EWORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const int d = shape->n_heads * shape->head_dim;
  if ((int64_t)shape->n_q * d >= INT32_MAX) return ISPA_EUNSUPPORTED;   // 32-bit buffer offsets of the product
  const size_t a_bytes = local_a_bytes(shape);
  const size_t vt_bytes = attn_vt_bytes_aligned((int64_t)shape->n_sink + shape->n_hist + shape->n_cur, d);
  uint8_t* aq = (uint8_t*)workspace + a_bytes + vt_bytes;
  float* sa = (float*)(aq + w8a8_codes_bytes(shape));
  AttnLaunch L;
  L.mode = 2;
  L.io = io_dtype;
  L.stat = ISPA_F16;
  L.q = q;
  L.k = k;
  L.v = v;
  L.a_full = workspace;
  L.a_loc_t = nullptr;
  L.delta_a_t = nullptr;
  L.ld_stat = 0;
  L.lse_loc = nullptr;
  L.lse_hist = nullptr;
  L.n_q = shape->n_q;
  L.n_sink = shape->n_sink;
  L.n_hist = shape->n_hist;
  L.n_cur = shape->n_cur;
  L.n_heads = shape->n_heads;
  L.head_dim = shape->head_dim;
  L.scale = eff_scale(shape);
  L.ws = (char*)workspace + a_bytes;
  L.ws_bytes = vt_bytes;
  if (launch_attention(L, s) != hipSuccess) return ISPA_EHIP;
  if (launch_quant_rows(io_dtype, workspace, d, shape->n_q, d, aq, d, sa, s) != hipSuccess) return ISPA_EHIP;
  return hip_status(launch_proj8(io_dtype, aq, sa, (const uint8_t*)wq_t, w_scales, out, shape->n_q, d, d, s));
}

}  // extern "C"
