"""Python binding of the ISPA hot-path library (libispa.so, C ABI in include/ispa.h).

Argument marshalling only: every call passes device pointers of PyTorch tensors,
sizes and the current HIP stream to the C ABI, and every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["IspaError", "AttnShape", "lib", "dual_attn", "gram_accum", "absorb_solve",
           "local_attn_fused_proj", "workspace_bytes", "CALL_DUAL_ATTN", "CALL_ABSORB_SOLVE",
           "CALL_LOCAL_ATTN_PROJ", "CALL_LOCAL_ATTN_PROJ_W8A8", "library_path", "KVCache",
           "quantize_weight_fp8", "quantize_rows_fp8", "local_attn_fused_proj_w8a8", "select_layers",
           "local_attn_fused_proj_noalloc", "absorb_solve_batched", "local_attn_fp8", "local_attn_fp8_proj_w8a8",
           "CALL_LOCAL_ATTN_FP8", "CALL_LOCAL_ATTN_FP8_PROJ_W8A8", "dual_attn_vt", "transpose_rows",
           "CALL_DUAL_ATTN_VT", "local_attn_fused_proj_wt", "transpose16"]

F32, BF16, F16 = 0, 1, 2
CALL_DUAL_ATTN, CALL_ABSORB_SOLVE, CALL_LOCAL_ATTN_PROJ, CALL_LOCAL_ATTN_PROJ_W8A8 = 0, 1, 2, 3
CALL_LOCAL_ATTN_FP8, CALL_LOCAL_ATTN_FP8_PROJ_W8A8, CALL_DUAL_ATTN_VT = 4, 5, 6
_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libispa.so")


class IspaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().ispa_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_hist", ctypes.c_int32),
                ("n_cur", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float)]

    @classmethod
    def of(cls, s, scale: float = 0.0) -> "AttnShape":
        """From any object with n_q, n_sink, n_hist, n_cur, n_heads, head_dim attributes."""
        return cls(s.n_q, s.n_sink, s.n_hist, s.n_cur, s.n_heads, s.head_dim, scale)


_LIB: Optional[ctypes.CDLL] = None
_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


def lib() -> ctypes.CDLL:
    """Load libispa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m kv_cache_attention_ispa_amd.build`")
        L = ctypes.CDLL(path)
        L.ispa_dual_attn.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _vp,
                                     _vp, _vp, _sz, _vp]
        L.ispa_dual_attn_vt.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _i32, _vp, _i64, _vp, _i32, _vp,
                                        _vp, _i64, _vp, _vp, _vp, _sz, _vp]
        L.ispa_transpose_rows.argtypes = [_i32, _i32, _i32, _vp, _i32, _vp, _i64, _i64, _vp]
        L.ispa_gram_accum.argtypes = [_i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp]
        L.ispa_absorb_solve.argtypes = [_i32, _vp, _vp, _vp, _i32, _vp, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp]
        L.ispa_local_attn_fused_proj.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                 _vp]
        L.ispa_local_attn_fused_proj_wt.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _sz, _vp]
        L.ispa_transpose16.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp]
        L.ispa_workspace_bytes.argtypes = [_i32, ctypes.POINTER(AttnShape), _i32]
        L.ispa_workspace_bytes.restype = ctypes.c_size_t
        L.ispa_status_string.argtypes = [_i32]
        L.ispa_status_string.restype = ctypes.c_char_p
        L.ispa_version.restype = ctypes.c_int
        L.ispa_quantize_weight_fp8.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _vp]
        L.ispa_quantize_rows_fp8.argtypes = [_i32, _i32, _i32, _vp, _i64, _vp, _i64, _vp, _vp]
        L.ispa_local_attn_fused_proj_w8a8.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _vp, _sz, _vp]
        L.ispa_kv_create.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp)]
        L.ispa_kv_destroy.argtypes = [_vp]
        L.ispa_kv_write_sink.argtypes = [_vp, _i32, _vp, _vp, _vp]
        L.ispa_kv_append_chunk.argtypes = [_vp, _i32, _vp, _vp, _vp]
        L.ispa_kv_release_history.argtypes = [_vp, _i32, _vp]
        L.ispa_kv_layer.argtypes = [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_i32)]
        L.ispa_kv_bytes.argtypes = [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.ispa_select_layers.argtypes = [_i32, _vp, _vp, _i32, _vp, _vp, _vp]
        L.ispa_local_attn_fp8.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.ispa_local_attn_fp8_proj_w8a8.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _vp, _sz, _vp]
        L.ispa_absorb_solve_batched.argtypes = [_i32, _i32, _vp, _vp, _vp, _i32, _vp, _f32, _i32, _i32, _vp, _vp, _vp,
                                                _vp, _vp, _vp, _sz, _vp]
        L.ispa_local_attn_fused_proj_noalloc.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp,
                                                         _vp]
        L.ispa_noalloc_scratch_bytes.restype = ctypes.c_size_t
        for f in ("ispa_dual_attn", "ispa_dual_attn_vt", "ispa_transpose_rows", "ispa_gram_accum", "ispa_absorb_solve", "ispa_local_attn_fused_proj",
                  "ispa_quantize_weight_fp8", "ispa_quantize_rows_fp8", "ispa_local_attn_fused_proj_w8a8",
                  "ispa_kv_create", "ispa_kv_destroy", "ispa_kv_write_sink", "ispa_kv_append_chunk",
                  "ispa_kv_release_history", "ispa_kv_layer", "ispa_kv_bytes", "ispa_select_layers",
                  "ispa_local_attn_fused_proj_noalloc", "ispa_absorb_solve_batched", "ispa_local_attn_fp8",
                  "ispa_local_attn_fp8_proj_w8a8"):
            getattr(L, f).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in codes:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want(t, name, dtypes=None, shape=None, min_numel=None, contiguous=True):
    """Check one tensor argument before anything reaches the C ABI: dtype, exact shape (None entries
    are free), size and layout.  Raises ValueError; `t = None` passes (optional arguments)."""
    if t is None:
        return
    if dtypes is not None:
        import torch
        ds = (dtypes,) if isinstance(dtypes, torch.dtype) else tuple(dtypes)
        if t.dtype not in ds:
            raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in ds)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} must have shape {tuple('*' if w is None else w for w in shape)}, "
                             f"got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements, got {t.numel()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(str(d) for d in devs)}")
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _io_dtypes():
    import torch
    return (torch.float32, torch.bfloat16, torch.float16)


def _stat_view(t, name, d, n):
    """A feature-major statistic: [d, >= n] with unit stride along tokens; returns its row stride."""
    if t is None:
        return None
    if t.dim() != 2 or t.shape[0] != d or t.shape[1] < n:
        raise ValueError(f"{name} must be a [{d}, >= {n}] feature-major view, got {tuple(t.shape)}")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along tokens")
    return t.stride(0)


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise IspaError(status, where)


def _ws_bytes(workspace) -> int:
    if workspace is None:
        return 0
    import torch
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return workspace.numel()


def workspace_bytes(call_id: int, shape: Optional[AttnShape] = None, d: int = 0) -> int:
    return int(lib().ispa_workspace_bytes(call_id, ctypes.byref(shape) if shape is not None else None, d))


def _dual_outputs(shape, q, a_full, a_loc_t, delta_a_t, ld_stat, lse_loc, lse_hist):
    """Checks the outputs of ispa_dual_attn(_vt); returns (stat dtype code, ld_stat)."""
    import torch
    d = shape.n_heads * shape.head_dim
    _want(a_full, "a_full", q.dtype, (shape.n_q, d))
    for n_, t in (("lse_loc", lse_loc), ("lse_hist", lse_hist)):
        _want(t, n_, torch.float32, (shape.n_heads, shape.n_q))
    if a_loc_t is not None and delta_a_t is not None and a_loc_t.dtype != delta_a_t.dtype:
        raise ValueError("a_loc_t and delta_a_t must share a dtype")
    lds = [x for x in (_stat_view(a_loc_t, "a_loc_t", d, shape.n_q), _stat_view(delta_a_t, "delta_a_t", d, shape.n_q))
           if x is not None]
    if len(set(lds)) > 1:
        raise ValueError("a_loc_t and delta_a_t must have the same leading dimension")
    stat = a_loc_t if a_loc_t is not None else delta_a_t
    if stat is not None:
        _want(stat, "statistics", _io_dtypes(), contiguous=False)
        if ld_stat is None:
            ld_stat = lds[0]
        elif ld_stat != lds[0]:
            raise ValueError(f"ld_stat {ld_stat} differs from the statistics' row stride {lds[0]}")
    return (_dtype_code(stat) if stat is not None else F16), int(ld_stat or 0)


def dual_attn(shape: AttnShape, q, k, v, a_full=None, a_loc_t=None, delta_a_t=None, ld_stat: Optional[int] = None,
              lse_loc=None, lse_hist=None, workspace=None, stream=None) -> None:
    """ispa_dual_attn: see include/ispa.h.  Stat outputs are feature-major [d, ld_stat] views;
    workspace (bytes from workspace_bytes(CALL_DUAL_ATTN, shape)) is needed for bf16/fp16 inputs."""
    d = shape.n_heads * shape.head_dim
    n_k = shape.n_sink + shape.n_hist + shape.n_cur
    _want(q, "q", _io_dtypes(), (shape.n_q, d))
    _want(k, "k", q.dtype, (n_k, d))
    _want(v, "v", q.dtype, (n_k, d))
    st, ld = _dual_outputs(shape, q, a_full, a_loc_t, delta_a_t, ld_stat, lse_loc, lse_hist)
    _same_device(q, k, v, a_full, a_loc_t, delta_a_t, lse_loc, lse_hist, workspace)
    _check(lib().ispa_dual_attn(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(a_full), st,
                                _ptr(a_loc_t), _ptr(delta_a_t), ld, _ptr(lse_loc), _ptr(lse_hist),
                                _ptr(workspace), _ws_bytes(workspace), _stream(stream)), "ispa_dual_attn")


def dual_attn_vt(shape: AttnShape, q, k, vt, a_full=None, a_loc_t=None, delta_a_t=None,
                 ld_stat: Optional[int] = None, lse_loc=None, lse_hist=None, workspace=None, stream=None) -> None:
    """ispa_dual_attn_vt: V given as the caller's V^T, a [d, ldv] tensor (unit stride along rows of
    the cache, ldv = its row stride) in fp16 for the dual stream or the input dtype for the single
    stream.  Workspace (workspace_bytes(CALL_DUAL_ATTN_VT, shape)) only in dual mode."""
    import torch
    d = shape.n_heads * shape.head_dim
    n_k = shape.n_sink + shape.n_hist + shape.n_cur
    _want(q, "q", (torch.bfloat16, torch.float16), (shape.n_q, d))
    _want(k, "k", q.dtype, (n_k, d))
    _want(vt, "vt", (torch.bfloat16, torch.float16), contiguous=False)
    ldv = _stat_view(vt, "vt", d, n_k)
    st, ld = _dual_outputs(shape, q, a_full, a_loc_t, delta_a_t, ld_stat, lse_loc, lse_hist)
    _same_device(q, k, vt, a_full, a_loc_t, delta_a_t, lse_loc, lse_hist, workspace)
    _check(lib().ispa_dual_attn_vt(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _dtype_code(vt), _ptr(vt),
                                   int(ldv), _ptr(a_full), st, _ptr(a_loc_t), _ptr(delta_a_t), ld, _ptr(lse_loc),
                                   _ptr(lse_hist), _ptr(workspace), _ws_bytes(workspace), _stream(stream)),
           "ispa_dual_attn_vt")


def transpose_rows(v, vt, col0: int, stream=None) -> None:
    """ispa_transpose_rows: the rows of v [rows, d] (bf16/fp16) into columns [col0, col0 + rows) of
    the V^T view vt [d, ldv] (fp16 or v's dtype, unit stride along columns), zeros after them."""
    import torch
    _want(v, "v", (torch.bfloat16, torch.float16))
    if v.dim() != 2:
        raise ValueError("v must be 2-D")
    rows, d = v.shape
    _want(vt, "vt", (torch.float16, v.dtype), contiguous=False)
    ldv = _stat_view(vt, "vt", d, 0)
    if col0 < 0 or col0 + rows > vt.shape[1]:
        raise ValueError(f"columns [{col0}, {col0 + rows}) do not fit in vt of {vt.shape[1]} columns")
    _same_device(v, vt)
    _check(lib().ispa_transpose_rows(rows, d, _dtype_code(v), _ptr(v), _dtype_code(vt), _ptr(vt), int(ldv),
                                     int(col0), _stream(stream)), "ispa_transpose_rows")


def gram_accum(a_loc_t, delta_a_t, n: int, G, C, D=None, accumulate: bool = False, stream=None) -> None:
    """ispa_gram_accum over tokens [0, n) of feature-major [d, ld] statistics."""
    import torch
    if G.dim() != 2:
        raise ValueError("G must be [d, d]")
    d = G.shape[0]
    for n_, t in (("G", G), ("C", C), ("D", D)):
        _want(t, n_, torch.float32, (d, d))
    if a_loc_t.dtype != delta_a_t.dtype:
        raise ValueError("a_loc_t and delta_a_t must share a dtype")
    _want(a_loc_t, "a_loc_t", _io_dtypes(), contiguous=False)
    if _stat_view(a_loc_t, "a_loc_t", d, n) != _stat_view(delta_a_t, "delta_a_t", d, n):
        raise ValueError("statistics must be feature-major views with one leading dimension")
    _same_device(a_loc_t, delta_a_t, G, C, D)
    _check(lib().ispa_gram_accum(d, int(n), _dtype_code(a_loc_t), _ptr(a_loc_t), _ptr(delta_a_t), a_loc_t.stride(0),
                                 int(bool(accumulate)), _ptr(G), _ptr(C), _ptr(D), _stream(stream)), "ispa_gram_accum")


def absorb_solve(G, C, W, lam: float, relative: bool, delta_w, info, workspace, D=None, w_new=None, eps=None,
                 lambda_out=None, refine: int = 0, stream=None) -> None:
    """ispa_absorb_solve: dW = (G + lambda I)^-1 C W (+ eps, W_new); refine = refinement steps."""
    import torch
    if G.dim() != 2:
        raise ValueError("G must be [d, d]")
    d = G.shape[0]
    for n_, t in (("G", G), ("C", C), ("D", D), ("delta_w", delta_w)):
        _want(t, n_, torch.float32, (d, d))
    _want(W, "W", _io_dtypes(), (d, d))
    _want(w_new, "w_new", W.dtype, (d, d))
    _want(info, "info", torch.int32, min_numel=1)
    _want(eps, "eps", torch.float32, min_numel=1)
    _want(lambda_out, "lambda_out", torch.float32, min_numel=1)
    _same_device(G, C, D, W, delta_w, w_new, info, eps, lambda_out, workspace)
    _check(lib().ispa_absorb_solve(d, _ptr(G), _ptr(C), _ptr(D), _dtype_code(W), _ptr(W), float(lam), int(relative),
                                   int(refine), _ptr(delta_w), _ptr(w_new), _ptr(eps), _ptr(lambda_out), _ptr(info),
                                   _ptr(workspace), _ws_bytes(workspace), _stream(stream)),
           "ispa_absorb_solve")


def absorb_solve_batched(G, C, W, lam: float, relative: bool, delta_w, info, workspace, D=None, w_new=None,
                         eps=None, lambda_out=None, refine: int = 0, stream=None) -> None:
    """ispa_absorb_solve_batched: one absorption per layer for [n_layers, d, d] statistics and weights;
    eps, lambda_out, info are [n_layers]."""
    import torch
    if G.dim() != 3 or G.shape[1] != G.shape[2]:
        raise ValueError("G must be [n_layers, d, d]")
    n, d = G.shape[0], G.shape[1]
    for n_, t in (("G", G), ("C", C), ("D", D), ("delta_w", delta_w)):
        _want(t, n_, torch.float32, (n, d, d))
    _want(W, "W", _io_dtypes(), (n, d, d))
    _want(w_new, "w_new", W.dtype, (n, d, d))
    _want(info, "info", torch.int32, (n,))
    _want(eps, "eps", torch.float32, (n,))
    _want(lambda_out, "lambda_out", torch.float32, (n,))
    _same_device(G, C, D, W, delta_w, w_new, info, eps, lambda_out, workspace)
    _check(lib().ispa_absorb_solve_batched(n, d, _ptr(G), _ptr(C), _ptr(D), _dtype_code(W), _ptr(W), float(lam),
                                           int(relative), int(refine), _ptr(delta_w), _ptr(w_new), _ptr(eps),
                                           _ptr(lambda_out), _ptr(info), _ptr(workspace), _ws_bytes(workspace),
                                           _stream(stream)), "ispa_absorb_solve_batched")


def _l_layer_args(shape, q, k, v, out):
    import torch
    d = shape.n_heads * shape.head_dim
    n_k = shape.n_sink + shape.n_hist + shape.n_cur
    _want(q, "q", (torch.bfloat16, torch.float16), (shape.n_q, d))
    _want(k, "k", q.dtype, (n_k, d))
    _want(v, "v", q.dtype, (n_k, d))
    _want(out, "out", q.dtype, (shape.n_q, d))
    return d


def local_attn_fused_proj(shape: AttnShape, q, k, v, w_new, out, workspace, stream=None) -> None:
    """ispa_local_attn_fused_proj: out = LocalAttn(q; sink + current) @ w_new."""
    d = _l_layer_args(shape, q, k, v, out)
    _want(w_new, "w_new", q.dtype, (d, d))
    _same_device(q, k, v, w_new, out, workspace)
    _check(lib().ispa_local_attn_fused_proj(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(w_new), _ptr(out), _ptr(workspace), _ws_bytes(workspace),
                                            _stream(stream)),
           "ispa_local_attn_fused_proj")


def local_attn_fused_proj_wt(shape: AttnShape, q, k, v, w_new_t, out, workspace, stream=None) -> None:
    """ispa_local_attn_fused_proj_wt: the L-layer step with W_new given transposed (w_new_t = W_new^T,
    e.g. from transpose16 once at the fold)."""
    d = _l_layer_args(shape, q, k, v, out)
    _want(w_new_t, "w_new_t", q.dtype, (d, d))
    _same_device(q, k, v, w_new_t, out, workspace)
    _check(lib().ispa_local_attn_fused_proj_wt(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(w_new_t), _ptr(out), _ptr(workspace), _ws_bytes(workspace),
                                               _stream(stream)),
           "ispa_local_attn_fused_proj_wt")


def transpose16(src, dst, stream=None) -> None:
    """ispa_transpose16: dst = src^T for 2-D bf16/fp16 device tensors (dims multiples of 16)."""
    import torch
    if src.dim() != 2:
        raise ValueError("src must be 2-D")
    rows, cols = src.shape
    _want(src, "src", (torch.bfloat16, torch.float16))
    _want(dst, "dst", src.dtype, (cols, rows))
    _same_device(src, dst)
    _check(lib().ispa_transpose16(rows, cols, _dtype_code(src), _ptr(src), _ptr(dst), _stream(stream)),
           "ispa_transpose16")


def local_attn_fused_proj_noalloc(shape: AttnShape, q, k, v, w_new, out, stream=None) -> None:
    """ispa_local_attn_fused_proj_noalloc: the L-layer step with the library's fixed per-GPU scratch
    instead of a workspace (allocates nothing; calls overlapping on one GPU race)."""
    d = _l_layer_args(shape, q, k, v, out)
    _want(w_new, "w_new", q.dtype, (d, d))
    _same_device(q, k, v, w_new, out)
    _check(lib().ispa_local_attn_fused_proj_noalloc(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                                    _ptr(w_new), _ptr(out), _stream(stream)),
           "ispa_local_attn_fused_proj_noalloc")


def local_attn_fp8(shape: AttnShape, q, k, v, out, workspace, stream=None) -> None:
    """ispa_local_attn_fp8: out = FP8 attention over the local rows (sink + current chunk)."""
    _l_layer_args(shape, q, k, v, out)
    _same_device(q, k, v, out, workspace)
    _check(lib().ispa_local_attn_fp8(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     _ptr(workspace), _ws_bytes(workspace), _stream(stream)), "ispa_local_attn_fp8")


def local_attn_fp8_proj_w8a8(shape: AttnShape, q, k, v, wq_t, w_scales, out, workspace, stream=None) -> None:
    """ispa_local_attn_fp8_proj_w8a8: the converted layer in W8A8 end to end (FP8 attention, then the W8A8
    projection by the codes and scales of quantize_weight_fp8)."""
    import torch
    d = _l_layer_args(shape, q, k, v, out)
    _want(wq_t, "wq_t", torch.uint8, (d, d))
    _want(w_scales, "w_scales", torch.float32, (d,))
    _same_device(q, k, v, wq_t, w_scales, out, workspace)
    _check(lib().ispa_local_attn_fp8_proj_w8a8(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(wq_t), _ptr(w_scales), _ptr(out), _ptr(workspace),
                                               _ws_bytes(workspace), _stream(stream)),
           "ispa_local_attn_fp8_proj_w8a8")


def quantize_weight_fp8(w, wq_t, w_scales, stream=None) -> None:
    """ispa_quantize_weight_fp8: w [d_in, d_out] -> wq_t [d_out, d_in] E4M3 codes (uint8), w_scales [d_out]."""
    import torch
    if w.dim() != 2:
        raise ValueError("w must be [d_in, d_out]")
    d_in, d_out = w.shape
    _want(w, "w", _io_dtypes())
    _want(wq_t, "wq_t", torch.uint8, (d_out, d_in))
    _want(w_scales, "w_scales", torch.float32, (d_out,))
    _same_device(w, wq_t, w_scales)
    _check(lib().ispa_quantize_weight_fp8(d_in, d_out, _dtype_code(w), _ptr(w), _ptr(wq_t), _ptr(w_scales),
                                          _stream(stream)), "ispa_quantize_weight_fp8")


def quantize_rows_fp8(x, q, scales, stream=None) -> None:
    """ispa_quantize_rows_fp8: x [rows, cols] -> q [rows, cols] E4M3 codes (uint8), scales [rows]."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    _want(x, "x", _io_dtypes(), contiguous=False)
    _want(q, "q", torch.uint8, (rows, cols), contiguous=False)
    _want(scales, "scales", torch.float32, (rows,))
    if x.stride(1) != 1 or q.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    _same_device(x, q, scales)
    _check(lib().ispa_quantize_rows_fp8(rows, cols, _dtype_code(x), _ptr(x), x.stride(0), _ptr(q), q.stride(0),
                                        _ptr(scales), _stream(stream)), "ispa_quantize_rows_fp8")


def local_attn_fused_proj_w8a8(shape: AttnShape, q, k, v, wq_t, w_scales, out, workspace, stream=None) -> None:
    """ispa_local_attn_fused_proj_w8a8: out = W8A8(LocalAttn(q; sink + current), W_new) with W_new given as
    the codes and scales of quantize_weight_fp8."""
    import torch
    d = _l_layer_args(shape, q, k, v, out)
    _want(wq_t, "wq_t", torch.uint8, (d, d))
    _want(w_scales, "w_scales", torch.float32, (d,))
    _same_device(q, k, v, wq_t, w_scales, out, workspace)
    _check(lib().ispa_local_attn_fused_proj_w8a8(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                                 _ptr(wq_t), _ptr(w_scales), _ptr(out), _ptr(workspace),
                                                 _ws_bytes(workspace), _stream(stream)),
           "ispa_local_attn_fused_proj_w8a8")


def select_layers(eps, k: int, role, order=None, info=None, stream=None) -> None:
    """ispa_select_layers: role[i] = 1 for the k layers with the lowest eps (stable; NaN, and layers whose
    info is non-zero, last), else 0; order (optional) receives the layer indices in rank order."""
    import torch
    _want(eps, "eps", torch.float32)
    if eps.dim() != 1:
        raise ValueError("eps must be [n_layers]")
    n = eps.shape[0]
    _want(info, "info", torch.int32, (n,))
    _want(role, "role", torch.int32, (n,))
    _want(order, "order", torch.int32, (n,))
    _same_device(eps, info, role, order)
    _check(lib().ispa_select_layers(n, _ptr(eps), _ptr(info), int(k), _ptr(role), _ptr(order), _stream(stream)),
           "ispa_select_layers")


class _DeviceRows:
    """A [rows, d] view of device memory the library owns, for torch.as_tensor (no copy)."""

    def __init__(self, ptr: int, rows: int, d: int, dtype: int):
        self.__cuda_array_interface__ = {"shape": (rows, d), "typestr": {F32: "<f4", F16: "<f2", BF16: "<i2"}[dtype],
                                         "data": (ptr, False), "version": 3}


class KVCache:
    """ispa_kv_*: per-layer K/V rows (sink | history | current) on the device, owned by the library.

    A full layer grows by one chunk per append_chunk; release_history converts a layer to sink +
    current chunk only.  See include/ispa.h for the contract."""

    def __init__(self, n_layers: int, d: int, dtype, sink_rows: int, chunk_rows: int, max_chunks: int):
        import torch
        self.dtype = dtype
        self.d = d
        self._code = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[dtype]
        h = _vp()
        _check(lib().ispa_kv_create(n_layers, d, self._code, sink_rows, chunk_rows, max_chunks, ctypes.byref(h)),
               "ispa_kv_create")
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(lib().ispa_kv_destroy(self._h), "ispa_kv_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _rows(self, t, name):
        if not t.is_contiguous() or t.dtype != self.dtype or t.shape[-1] != self.d:
            raise ValueError(f"{name} must be contiguous [rows, {self.d}] {self.dtype}")
        return _ptr(t)

    def write_sink(self, layer: int, k, v, stream=None) -> None:
        _check(lib().ispa_kv_write_sink(self._h, layer, self._rows(k, "k"), self._rows(v, "v"), _stream(stream)),
               "ispa_kv_write_sink")

    def append_chunk(self, layer: int, k, v, stream=None) -> None:
        _check(lib().ispa_kv_append_chunk(self._h, layer, self._rows(k, "k"), self._rows(v, "v"), _stream(stream)),
               "ispa_kv_append_chunk")

    def release_history(self, layer: int, stream=None) -> None:
        _check(lib().ispa_kv_release_history(self._h, layer, _stream(stream)), "ispa_kv_release_history")

    def layer(self, layer: int):
        """(k, v, (n_sink, n_hist, n_cur)): k and v are torch views of the layer's rows (no copy),
        valid until release_history of that layer or close()."""
        import torch
        kp, vp, rows = _vp(), _vp(), (_i32 * 3)()
        _check(lib().ispa_kv_layer(self._h, layer, ctypes.byref(kp), ctypes.byref(vp), rows), "ispa_kv_layer")
        n = rows[0] + rows[1] + rows[2]
        if n == 0:
            e = torch.empty((0, self.d), dtype=self.dtype, device="cuda")
            return e, e, (0, 0, 0)
        views = []
        for p in (kp.value, vp.value):
            t = torch.as_tensor(_DeviceRows(p, n, self.d, self._code), device="cuda")
            views.append(t.view(self.dtype) if self._code == BF16 else t)
        return views[0], views[1], (rows[0], rows[1], rows[2])

    def bytes(self):
        """(held, reserved): bytes of K and V rows held, bytes of device memory allocated."""
        held, reserved = _i64(), _i64()
        _check(lib().ispa_kv_bytes(self._h, ctypes.byref(held), ctypes.byref(reserved)), "ispa_kv_bytes")
        return held.value, reserved.value
