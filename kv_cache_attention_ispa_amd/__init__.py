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
           "quantize_weight_fp8", "quantize_rows_fp8", "local_attn_fused_proj_w8a8"]

F32, BF16, F16 = 0, 1, 2
CALL_DUAL_ATTN, CALL_ABSORB_SOLVE, CALL_LOCAL_ATTN_PROJ, CALL_LOCAL_ATTN_PROJ_W8A8 = 0, 1, 2, 3
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
        for f in ("ispa_dual_attn", "ispa_gram_accum", "ispa_absorb_solve", "ispa_local_attn_fused_proj",
                  "ispa_quantize_weight_fp8", "ispa_quantize_rows_fp8", "ispa_local_attn_fused_proj_w8a8",
                  "ispa_kv_create", "ispa_kv_destroy", "ispa_kv_write_sink", "ispa_kv_append_chunk",
                  "ispa_kv_release_history", "ispa_kv_layer", "ispa_kv_bytes"):
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


def quantize_weight_fp8(w, wq_t, w_scales, stream=None) -> None:
    """ispa_quantize_weight_fp8: w [d_in, d_out] -> wq_t [d_out, d_in] E4M3 codes (uint8), w_scales [d_out]."""
    for n_, t in (("w", w), ("wq_t", wq_t), ("w_scales", w_scales)):
        _dense(t, n_)
    d_in, d_out = w.shape
    _check(lib().ispa_quantize_weight_fp8(d_in, d_out, _dtype_code(w), _ptr(w), _ptr(wq_t), _ptr(w_scales),
                                          _stream(stream)), "ispa_quantize_weight_fp8")


def quantize_rows_fp8(x, q, scales, stream=None) -> None:
    """ispa_quantize_rows_fp8: x [rows, cols] -> q [rows, cols] E4M3 codes (uint8), scales [rows]."""
    for n_, t in (("q", q), ("scales", scales)):
        _dense(t, n_)
    if x.stride(1) != 1 or q.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    rows, cols = x.shape
    _check(lib().ispa_quantize_rows_fp8(rows, cols, _dtype_code(x), _ptr(x), x.stride(0), _ptr(q), q.stride(0),
                                        _ptr(scales), _stream(stream)), "ispa_quantize_rows_fp8")


def local_attn_fused_proj_w8a8(shape: AttnShape, q, k, v, wq_t, w_scales, out, workspace, stream=None) -> None:
    """ispa_local_attn_fused_proj_w8a8: out = W8A8(LocalAttn(q; sink + current), W_new) with W_new given as
    the codes and scales of quantize_weight_fp8."""
    for n_, t in (("q", q), ("k", k), ("v", v), ("wq_t", wq_t), ("w_scales", w_scales), ("out", out)):
        _dense(t, n_)
    _check(lib().ispa_local_attn_fused_proj_w8a8(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                                 _ptr(wq_t), _ptr(w_scales), _ptr(out), _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "ispa_local_attn_fused_proj_w8a8")


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
