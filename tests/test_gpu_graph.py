"""The hot path under HIP graph capture: every call only enqueues kernels on the caller's stream (the
solve forks part of its work to the library's auxiliary stream and joins it back by events, which
brings that stream into the capture; no allocation, copy, memset or host synchronisation), so the
whole step -- dual attention (with the per-call V copy, and over a kept V^T with the current chunk
appended in the graph), Gram statistics, solve with epsilon and W_new, and the L-layer variants
(16-bit, W8A8, W8A8 with FP8 attention) -- can be captured once and replayed.  Each replay, with eager work and synchronisation between replays, must reproduce the eager
results bit for bit (the kernels are deterministic)."""
import math

import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, torch

pytestmark = pytest.mark.gpu


def test_whole_step_graph_replays_match_eager():
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    sh = wl.AttnShape(600, 200, 400, 600, 4, 128)
    d = sh.d
    rng = np.random.default_rng(77)
    q = dev(wl.round_to(rng.standard_normal((sh.n_q, d)), "bf16"), "bf16")
    k = dev(wl.round_to(rng.standard_normal((sh.n_k, d)), "bf16"), "bf16")
    v = dev(wl.round_to(rng.standard_normal((sh.n_k, d)), "bf16"), "bf16")
    W = dev(wl.round_to(rng.standard_normal((d, d)) / math.sqrt(d), "bf16"), "bf16")
    loc = np.concatenate([np.arange(sh.n_sink), np.arange(sh.n_sink + sh.n_hist, sh.n_k)])
    loc_t = t.from_numpy(loc).cuda()
    k_loc, v_loc = k[loc_t].contiguous(), v[loc_t].contiguous()
    s = ispa.AttnShape.of(sh)
    sl = ispa.AttnShape(sh.n_q, sh.n_sink, 0, sh.n_cur, sh.n_heads, sh.head_dim, 0.0)
    ld = ((sh.n_q + 7) // 8) * 8
    out = {
        "a_full": t.empty((sh.n_q, d), dtype=t.bfloat16, device="cuda"),
        "a_t": t.empty((d, ld), dtype=t.float16, device="cuda"),
        "da_t": t.empty((d, ld), dtype=t.float16, device="cuda"),
        "lse_l": t.empty((sh.n_heads, sh.n_q), device="cuda"),
        "lse_h": t.empty((sh.n_heads, sh.n_q), device="cuda"),
        "G": t.empty((d, d), device="cuda"), "C": t.empty((d, d), device="cuda"), "D": t.empty((d, d), device="cuda"),
        "dW": t.empty((d, d), device="cuda"), "w_new": t.empty((d, d), dtype=t.bfloat16, device="cuda"),
        "eps": t.empty((1,), device="cuda"), "info": t.zeros((1,), dtype=t.int32, device="cuda"),
        "y16": t.empty((sh.n_q, d), dtype=t.bfloat16, device="cuda"),
        "wq": t.empty((d, d), dtype=t.uint8, device="cuda"), "sw": t.empty((d,), device="cuda"),
        "y8": t.empty((sh.n_q, d), dtype=t.bfloat16, device="cuda"),
        "y8f": t.empty((sh.n_q, d), dtype=t.bfloat16, device="cuda"),
        "a_full_vt": t.empty((sh.n_q, d), dtype=t.bfloat16, device="cuda"),
        "a_t_vt": t.empty((d, ld), dtype=t.float16, device="cuda"),
        "da_t_vt": t.empty((d, ld), dtype=t.float16, device="cuda"),
    }
    ws_a = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, s), dtype=t.uint8, device="cuda")
    ws_s = t.empty(ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d), dtype=t.uint8, device="cuda")
    ws_l = t.empty(ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, sl), dtype=t.uint8, device="cuda")
    ws_8 = t.empty(ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ_W8A8, sl), dtype=t.uint8, device="cuda")
    ws_8f = t.empty(ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_FP8_PROJ_W8A8, sl), dtype=t.uint8, device="cuda")
    ws_vt = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN_VT, s), dtype=t.uint8, device="cuda")
    # the layer's V^T: sink and history rows written before the capture, the current chunk in it
    n_old = sh.n_sink + sh.n_hist
    vt = t.zeros((d, (sh.n_k + 7) // 8 * 8 + 64), dtype=t.float16, device="cuda")
    ispa.transpose_rows(v[:n_old], vt, 0)
    st = t.cuda.Stream()
    o = out

    def step():
        ispa.dual_attn(s, q, k, v, a_full=o["a_full"], a_loc_t=o["a_t"], delta_a_t=o["da_t"], ld_stat=ld,
                       lse_loc=o["lse_l"], lse_hist=o["lse_h"], workspace=ws_a, stream=st)
        ispa.gram_accum(o["a_t"], o["da_t"], sh.n_q, o["G"], o["C"], o["D"], stream=st)
        ispa.absorb_solve(o["G"], o["C"], W, 1e-3, True, o["dW"], o["info"], ws_s, D=o["D"], w_new=o["w_new"],
                          eps=o["eps"], refine=1, stream=st)
        ispa.local_attn_fused_proj(sl, q, k_loc, v_loc, o["w_new"], o["y16"], ws_l, stream=st)
        ispa.quantize_weight_fp8(o["w_new"], o["wq"], o["sw"], stream=st)
        ispa.local_attn_fused_proj_w8a8(sl, q, k_loc, v_loc, o["wq"], o["sw"], o["y8"], ws_8, stream=st)
        ispa.local_attn_fp8_proj_w8a8(sl, q, k_loc, v_loc, o["wq"], o["sw"], o["y8f"], ws_8f, stream=st)
        ispa.transpose_rows(v[n_old:], vt, n_old, stream=st)
        ispa.dual_attn_vt(s, q, k, vt, a_full=o["a_full_vt"], a_loc_t=o["a_t_vt"], delta_a_t=o["da_t_vt"],
                          ld_stat=ld, workspace=ws_vt, stream=st)

    with t.cuda.stream(st):
        step()
    t.cuda.synchronize()
    assert int(o["info"].item()) == 0
    # the kept V^T gives the per-call copy's outputs bit for bit
    for a, b in (("a_full", "a_full_vt"), ("a_t", "a_t_vt"), ("da_t", "da_t_vt")):
        assert t.equal(o[a].view(t.int16), o[b].view(t.int16)), a
    ref = {name: x.clone() for name, x in o.items()}
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph, stream=st):
        step()
    t.cuda.synchronize()
    for rep in range(3):
        for x in o.values():
            x.zero_()
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        for name, x in o.items():
            assert t.equal(x, ref[name]), (rep, name)
        with t.cuda.stream(st):
            step()           # eager work between replays
        t.cuda.synchronize()
        for name, x in o.items():
            assert t.equal(x, ref[name]), ("eager", rep, name)
