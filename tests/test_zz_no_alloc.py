"""GPU: ispa_local_attn_fused_proj_noalloc (the L-layer step on the library's fixed per-GPU scratch)
against ispa_local_attn_fused_proj with a workspace: two calls in a row, the second on a smaller
input, each bit-identical to the workspace variant (the same kernels run), plus the oracle on
sampled rows of the first."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import dev, host, maxrel, torch

pytestmark = pytest.mark.gpu


def _inputs(shape, seed):
    rng = np.random.default_rng(seed)
    q = wl.round_to(rng.standard_normal((shape.n_q, shape.d)), "bf16")
    k = wl.round_to(rng.standard_normal((shape.n_k, shape.d)), "bf16")
    v = wl.round_to(rng.standard_normal((shape.n_k, shape.d)), "bf16")
    w = wl.round_to(rng.standard_normal((shape.d, shape.d)) / math.sqrt(shape.d), "bf16")
    return q, k, v, w


def test_noalloc_matches_workspace_variant_twice():
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    # the 1.3B L-layer (sink 1560 + current 4680, d 1536), then a smaller ragged one
    shapes = [wl.AttnShape(4680, 1560, 0, 4680, 12, 128), wl.AttnShape(333, 100, 0, 333, 4, 128)]
    for i, shape in enumerate(shapes):
        print(f"noalloc call {i}: n_q {shape.n_q}, n_k {shape.n_k}, d {shape.d}", flush=True)
        q, k, v, w = _inputs(shape, 40 + i)
        qd, kd, vd, wd = (dev(x, "bf16") for x in (q, k, v, w))
        s = ispa.AttnShape.of(shape)
        out_na = t.full((shape.n_q, shape.d), float("nan"), dtype=t.bfloat16, device="cuda")
        ispa.local_attn_fused_proj_noalloc(s, qd, kd, vd, wd, out_na)
        ws = t.empty(ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, s), dtype=t.uint8, device="cuda")
        out_ws = t.full((shape.n_q, shape.d), float("nan"), dtype=t.bfloat16, device="cuda")
        ispa.local_attn_fused_proj(s, qd, kd, vd, wd, out_ws, ws)
        t.cuda.synchronize()
        assert t.equal(out_na, out_ws)
        rows = np.linspace(0, shape.n_q - 1, 5).astype(int)
        ref = oracle.local_layer_output(q[rows], k, v, shape.n_sink, shape.n_cur, shape.n_heads, w, threads=8)
        assert maxrel(host(out_na)[rows], ref) <= 2e-2


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    s = ispa.AttnShape(4680, 1560, 0, 4680, 40, 128, 0.0)      # d = 5120: 164 MiB of scratch
    assert ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, s) > ispa.lib().ispa_noalloc_scratch_bytes()
    x = t.empty((8,), dtype=t.bfloat16, device="cuda")
    p = x.data_ptr()
    st = ispa.lib().ispa_local_attn_fused_proj_noalloc(s, 1, p, p, p, p, p, None)
    assert st == 3   # ISPA_EWORKSPACE, nothing launched
