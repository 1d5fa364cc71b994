"""The pages' ablation variants as uses of the C ABI (technical summary, section 4 "Ablations"):
No Sink (n_sink = 0), No Absorb (the converted layer keeps W, i.e. dW = 0) and the warmup length
T_warm (how many chunks the statistics cover).  Each runs through the same calls as the method and
is checked against the oracle; the T_warm sweep also times the Gram over 1-4 warmup chunks at the
1.3B layer shape (the cost the ablation trades against quality)."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import dev, host, maxrel, relfro, torch, tdtype

pytestmark = pytest.mark.gpu


def _l_layer(shape, q, k, v, w, io):
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    s = ispa.AttnShape.of(shape)
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, s), dtype=t.uint8, device="cuda")
    out = t.empty((shape.n_q, shape.d), dtype=tdtype(io), device="cuda")
    ispa.local_attn_fused_proj(s, dev(q, io), dev(k, io), dev(v, io), dev(w, io), out, ws)
    t.cuda.synchronize()
    return out


def _rand(shape_rows, d, seed, io, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.round_to(rng.standard_normal((shape_rows, d)) * scale, io)


def test_no_sink_l_layer():
    """No Sink: the converted layer's local set is the current chunk alone."""
    io = "bf16"
    shape = wl.AttnShape(130, 0, 0, 130, 2, 128)
    q, k, v = _rand(shape.n_q, shape.d, 1, io), _rand(shape.n_k, shape.d, 2, io), _rand(shape.n_k, shape.d, 3, io)
    w = _rand(shape.d, shape.d, 4, io, 1 / math.sqrt(shape.d))
    out = _l_layer(shape, q, k, v, w, io)
    ref = oracle.local_layer_output(q, k, v, 0, shape.n_cur, shape.n_heads, w)
    assert maxrel(host(out), ref) <= 2e-2


def test_no_absorb_l_layer():
    """No Absorb: with nothing absorbed (C = 0) the solve returns dW = 0 and W_new = W bit for bit, so
    the converted layer computes local attention times the original W."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    io, d = "bf16", 256
    shape = wl.AttnShape(96, 32, 0, 96, 2, 128)
    rng = np.random.default_rng(5)
    a = rng.standard_normal((300, d)) * 0.05
    G = t.from_numpy(a.T @ a).float().cuda()
    C = t.zeros((d, d), device="cuda")
    W = dev(_rand(d, d, 6, io, 1 / math.sqrt(d)), io)
    dW = t.empty((d, d), device="cuda")
    W_new = t.empty((d, d), dtype=tdtype(io), device="cuda")
    info = t.zeros(1, dtype=t.int32, device="cuda")
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d), dtype=t.uint8, device="cuda")
    ispa.absorb_solve(G, C, W, 1e-3, True, dW, info, ws, w_new=W_new)
    t.cuda.synchronize()
    assert int(info.item()) == 0 and bool((dW == 0).all()) and t.equal(W_new, W)
    q, k, v = _rand(shape.n_q, d, 7, io), _rand(shape.n_k, d, 8, io), _rand(shape.n_k, d, 9, io)
    w_host = host(W)
    out = _l_layer(shape, q, k, v, w_host, io)
    ref = oracle.local_layer_output(q, k, v, shape.n_sink, shape.n_cur, shape.n_heads, w_host)
    assert maxrel(host(out), ref) <= 2e-2


@pytest.mark.parametrize("t_warm", [1, 2, 3])
def test_t_warm_sweep(t_warm):
    """T_warm chunks of statistics (small bf16 layer): dual attention per chunk, Gram accumulated call
    by call, then dW, against the oracle's solve over the same T_warm chunks."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    w = wl.Workload("tw_bf16", 78, wl.AttnShape(320, 96, 256, 320, 2, 128), "bf16", "f16", 1e-3, True)
    s = w.shape
    d = s.d
    G, C = t.empty((d, d), device="cuda"), t.empty((d, d), device="cuda")
    ld = ((s.n_q + 7) // 8) * 8
    sh = ispa.AttnShape.of(s)
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, sh), dtype=t.uint8, device="cuda")
    refs = []
    for c in range(t_warm):
        x = wl.layer_inputs(w, chunk=c, with_w=False)
        a_t = t.empty((d, ld), dtype=t.float16, device="cuda")
        da_t = t.empty((d, ld), dtype=t.float16, device="cuda")
        ispa.dual_attn(sh, dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), a_loc_t=a_t, delta_a_t=da_t,
                       ld_stat=ld, workspace=ws)
        ispa.gram_accum(a_t, da_t, s.n_q, G, C, None, accumulate=c > 0)
        r = oracle.dual_stream(x["q"], x["k"], x["v"], s.n_sink, s.n_hist, s.n_cur, s.n_heads)
        refs.append((r["a_loc"], r["delta_a"]))
    W = wl.layer_inputs(w, chunk=0)["w"]
    dW = t.empty((d, d), device="cuda")
    info = t.zeros(1, dtype=t.int32, device="cuda")
    wss = t.empty(ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d), dtype=t.uint8, device="cuda")
    ispa.absorb_solve(G, C, dev(W, "bf16"), w.lam, w.lam_relative, dW, info, wss)
    t.cuda.synchronize()
    Gr, Cr, _ = oracle.gram_stats(refs)
    dW_ref = oracle.solve_delta_w(Gr, Cr, W, oracle.ridge_lambda(Gr, w.lam, w.lam_relative))
    assert int(info.item()) == 0
    assert maxrel(host(G), Gr) <= 2e-2
    assert relfro(host(dW), dW_ref) <= 1e-2


def test_t_warm_gram_cost():
    """Gram cost against warmup length at the 1.3B layer (d = 1536, 4680 tokens per chunk, fp16
    statistics with D): one accumulating call per chunk, T_warm = 1..4; the cost is linear in T_warm."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    d, n = 1536, 4680
    g = t.Generator(device="cpu").manual_seed(3)
    a_t = (t.randn((d, n), generator=g) * 0.02).half().cuda()
    da_t = (t.randn((d, n), generator=g) * 0.02).half().cuda()
    G, C, D = (t.empty((d, d), device="cuda") for _ in range(3))
    per = []
    for t_warm in (1, 2, 3, 4):
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        best = 1e9
        for _ in range(3):
            e0.record()
            for c in range(t_warm):
                ispa.gram_accum(a_t, da_t, n, G, C, D, accumulate=c > 0)
            e1.record()
            t.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3)
        per.append(best / t_warm)
        print(f"\nT_warm {t_warm}: Gram {best:.1f} us ({best / t_warm:.1f} us per chunk)")
    assert max(per) <= 1.25 * min(per)
