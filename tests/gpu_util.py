"""Helpers for the GPU parity tests: device upload, calls through the C ABI, metrics."""
from __future__ import annotations

import numpy as np

_TORCH = None


def torch():
    global _TORCH
    if _TORCH is None:
        import torch as t
        _TORCH = t
    return _TORCH


def tdtype(name: str):
    t = torch()
    return {"f32": t.float32, "bf16": t.bfloat16, "f16": t.float16}[name]


def dev(x: np.ndarray, dtype: str):
    """Upload values that are exactly representable in `dtype` (they come from workloads.round_to)."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(tdtype(dtype))


def host(x) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def maxrel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def relfro(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def run_dual(shape, q, k, v, io: str, stat: str, ld_extra: int = 0, want=("a_full", "a_loc", "delta_a", "lse")):
    """Call ispa_dual_attn; return host float64 arrays (stat outputs transposed back to [n_q, d])."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    d = shape.d
    qd, kd, vd = dev(q, io), dev(k, io), dev(v, io)
    ld = ((shape.n_q + ld_extra + 7) // 8) * 8
    a_full = t.full((shape.n_q, d), float("nan"), device="cuda", dtype=tdtype(io)) if "a_full" in want else None
    a_loc_t = t.full((d, ld), float("nan"), device="cuda", dtype=tdtype(stat)) if "a_loc" in want else None
    da_t = t.full((d, ld), float("nan"), device="cuda", dtype=tdtype(stat)) if "delta_a" in want else None
    lse_l = t.full((shape.n_heads, shape.n_q), float("nan"), device="cuda") if "lse" in want else None
    lse_h = t.full((shape.n_heads, shape.n_q), float("nan"), device="cuda") if "lse" in want else None
    s = ispa.AttnShape.of(shape)
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, s), dtype=t.uint8, device="cuda")
    ispa.dual_attn(s, qd, kd, vd, a_full=a_full, a_loc_t=a_loc_t, delta_a_t=da_t,
                   ld_stat=ld if (a_loc_t is not None or da_t is not None) else 0, lse_loc=lse_l, lse_hist=lse_h,
                   workspace=ws)
    t.cuda.synchronize()
    out = {}
    if a_full is not None:
        out["a_full"] = host(a_full)
    if a_loc_t is not None:
        out["a_loc"] = host(a_loc_t)[:, :shape.n_q].T.copy()
        out["a_loc_pad"] = host(a_loc_t)[:, shape.n_q:]
    if da_t is not None:
        out["delta_a"] = host(da_t)[:, :shape.n_q].T.copy()
    if lse_l is not None:
        out["lse_loc"] = host(lse_l)
        out["lse_hist"] = host(lse_h)
    return out
