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
           "CALL_LOCAL_ATTN_PROJ", "library_path"]

F32, BF16, F16 = 0, 1, 2
CALL_DUAL_ATTN, CALL_ABSORB_SOLVE, CALL_LOCAL_ATTN_PROJ = 0, 1, 2
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
        L.ispa_gram_accum.argtypes = [_i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp]
        L.ispa_absorb_solve.argtypes = [_i32, _vp, _vp, _vp, _i32, _vp, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp]
        L.ispa_local_attn_fused_proj.argtypes = [ctypes.POINTER(AttnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                 _vp]
        L.ispa_workspace_bytes.argtypes = [_i32, ctypes.POINTER(AttnShape), _i32]
        L.ispa_workspace_bytes.restype = ctypes.c_size_t
        L.ispa_status_string.argtypes = [_i32]
        L.ispa_status_string.restype = ctypes.c_char_p
        L.ispa_version.restype = ctypes.c_int
        for f in ("ispa_dual_attn", "ispa_gram_accum", "ispa_absorb_solve", "ispa_local_attn_fused_proj"):
            getattr(L, f).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise IspaError(status, where)


def workspace_bytes(call_id: int, shape: Optional[AttnShape] = None, d: int = 0) -> int:
    return int(lib().ispa_workspace_bytes(call_id, ctypes.byref(shape) if shape is not None else None, d))


def dual_attn(shape: AttnShape, q, k, v, a_full=None, a_loc_t=None, delta_a_t=None, ld_stat: Optional[int] = None,
              lse_loc=None, lse_hist=None, workspace=None, stream=None) -> None:
    """ispa_dual_attn: see include/ispa.h.  Stat outputs are feature-major [d, ld_stat] views;
    workspace (bytes from workspace_bytes(CALL_DUAL_ATTN, shape)) is needed for bf16/fp16 inputs."""
    for n, t in (("q", q), ("k", k), ("v", v), ("a_full", a_full), ("lse_loc", lse_loc), ("lse_hist", lse_hist)):
        _dense(t, n)
    stat = a_loc_t if a_loc_t is not None else delta_a_t
    if stat is not None:
        if stat.stride(1) != 1:
            raise ValueError("stat outputs must have unit stride along tokens")
        if ld_stat is None:
            ld_stat = stat.stride(0)
    st = _dtype_code(stat) if stat is not None else F16
    _check(lib().ispa_dual_attn(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(a_full), st,
                                _ptr(a_loc_t), _ptr(delta_a_t), int(ld_stat or 0), _ptr(lse_loc), _ptr(lse_hist),
                                _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream(stream)), "ispa_dual_attn")


def gram_accum(a_loc_t, delta_a_t, n: int, G, C, D=None, accumulate: bool = False, stream=None) -> None:
    """ispa_gram_accum over tokens [0, n) of feature-major [d, ld] statistics."""
    for n_, t in (("G", G), ("C", C), ("D", D)):
        _dense(t, n_)
    if a_loc_t.stride(1) != 1 or delta_a_t.stride(1) != 1 or a_loc_t.stride(0) != delta_a_t.stride(0):
        raise ValueError("statistics must be feature-major views with one leading dimension")
    d = G.shape[0]
    _check(lib().ispa_gram_accum(d, int(n), _dtype_code(a_loc_t), _ptr(a_loc_t), _ptr(delta_a_t), a_loc_t.stride(0),
                                 int(bool(accumulate)), _ptr(G), _ptr(C), _ptr(D), _stream(stream)), "ispa_gram_accum")


def absorb_solve(G, C, W, lam: float, relative: bool, delta_w, info, workspace, D=None, w_new=None, eps=None,
                 lambda_out=None, refine: int = 0, stream=None) -> None:
    """ispa_absorb_solve: dW = (G + lambda I)^-1 C W (+ eps, W_new); refine = refinement steps."""
    for n_, t in (("G", G), ("C", C), ("D", D), ("W", W), ("delta_w", delta_w), ("w_new", w_new)):
        _dense(t, n_)
    d = G.shape[0]
    _check(lib().ispa_absorb_solve(d, _ptr(G), _ptr(C), _ptr(D), _dtype_code(W), _ptr(W), float(lam), int(relative),
                                   int(refine), _ptr(delta_w), _ptr(w_new), _ptr(eps), _ptr(lambda_out), _ptr(info),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "ispa_absorb_solve")


def local_attn_fused_proj(shape: AttnShape, q, k, v, w_new, out, workspace, stream=None) -> None:
    """ispa_local_attn_fused_proj: out = LocalAttn(q; sink + current) @ w_new."""
    for n_, t in (("q", q), ("k", k), ("v", v), ("w_new", w_new), ("out", out)):
        _dense(t, n_)
    _check(lib().ispa_local_attn_fused_proj(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(w_new), _ptr(out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream)),
           "ispa_local_attn_fused_proj")
