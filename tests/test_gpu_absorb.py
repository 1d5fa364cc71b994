"""GPU parity: ispa_gram_accum and ispa_absorb_solve against the CPU oracle.

Tolerances: Gram statistics against float64 products of the very same stored
inputs (max-rel 1e-4, fp32 accumulation); dW rel-Frobenius 1e-3 for fp32
workloads and 1e-2 for bf16 workloads; epsilon relative 1e-2.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import dev, host, maxrel, relfro, run_dual, torch, tdtype

pytestmark = pytest.mark.gpu


def _stat_dev(x_tokens_major: np.ndarray, dtype: str, ld: int, pad=1234.0):
    """Feature-major [d, ld] device buffer whose first n columns hold x^T (extra columns hold `pad`)."""
    t = torch()
    n, d = x_tokens_major.shape
    buf = t.full((d, ld), pad, dtype=tdtype(dtype), device="cuda")
    buf[:, :n] = dev(x_tokens_major.T.copy(), dtype)
    return buf


def _gram_gpu(chunks, dtype, d, with_d=True, pad=1234.0):
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    G = t.full((d, d), float("nan"), device="cuda")
    C = t.full((d, d), float("nan"), device="cuda")
    D = t.full((d, d), float("nan"), device="cuda") if with_d else None
    for i, (a, da) in enumerate(chunks):
        n = a.shape[0]
        ld = ((n + 7) // 8) * 8 + 8
        ispa.gram_accum(_stat_dev(a, dtype, ld, pad), _stat_dev(da, dtype, ld, pad), n, G, C, D, accumulate=i > 0)
    t.cuda.synchronize()
    return host(G), host(C), (host(D) if with_d else None)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d,ns", [(256, [300]), (160, [77, 5, 130]), (128, [1]), (384, [1000, 24])])
def test_gram_matches_float64_of_same_inputs(dtype, d, ns):
    rng = np.random.default_rng(d + len(ns))
    chunks = [(wl.round_to(rng.standard_normal((n, d)) * 0.05, dtype), wl.round_to(rng.standard_normal((n, d)) * 0.03, dtype))
              for n in ns]
    G, C, D = _gram_gpu(chunks, dtype, d)
    Gr, Cr, Dr = oracle.gram_stats(chunks)
    assert maxrel(G, Gr) <= 1e-4 and maxrel(C, Cr) <= 1e-4 and maxrel(D, Dr) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,n", [(384, 517), (640, 64), (96, 33)])
def test_gram_without_d(dtype, d, n):
    """D = NULL: only G (lower tiles, mirrored) and C are computed."""
    rng = np.random.default_rng(d + n)
    chunks = [(wl.round_to(rng.standard_normal((n, d)) * 0.05, dtype), wl.round_to(rng.standard_normal((n, d)) * 0.03, dtype))]
    G, C, _ = _gram_gpu(chunks, dtype, d, with_d=False)
    Gr, Cr, _ = oracle.gram_stats(chunks)
    assert maxrel(G, Gr) <= 1e-4 and maxrel(C, Cr) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,n", [(384, 33), (640, 77), (256, 517), (160, 1)])
def test_gram_nan_padding(dtype, d, n):
    """Token columns past n hold NaN (e.g. an uninitialised buffer): they are never read as data, even
    in the chunk of 8 tokens that straddles n, for every row of X and of Y."""
    rng = np.random.default_rng(7 * d + n)
    chunks = [(wl.round_to(rng.standard_normal((n, d)) * 0.05, dtype), wl.round_to(rng.standard_normal((n, d)) * 0.03, dtype))]
    G, C, D = _gram_gpu(chunks, dtype, d, pad=float("nan"))
    Gr, Cr, Dr = oracle.gram_stats(chunks)
    assert np.isfinite(G).all() and np.isfinite(C).all() and np.isfinite(D).all()
    assert maxrel(G, Gr) <= 1e-4 and maxrel(C, Cr) <= 1e-4 and maxrel(D, Dr) <= 1e-4


def _spd_problem(d, n, seed, w_dtype="f32"):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, d)) * 0.05
    da = rng.standard_normal((n, d)) * 0.03 + 0.3 * a @ rng.standard_normal((d, d)) / math.sqrt(d)
    G, C, D = oracle.gram_stats([(a, da)])
    G, C, D = (x.astype(np.float32).astype(np.float64) for x in (G, C, D))
    W = wl.round_to(rng.standard_normal((d, d)) / math.sqrt(d), w_dtype)
    return G, C, D, W


def _solve_gpu(G, C, D, W, lam, relative, w_dtype="f32", refine=False):
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    d = G.shape[0]
    Gd, Cd = dev(G, "f32"), dev(C, "f32")
    Dd = dev(D, "f32") if D is not None else None
    Wd = dev(W, w_dtype)
    dW = t.full((d, d), float("nan"), device="cuda")
    w_new = t.empty((d, d), dtype=tdtype(w_dtype), device="cuda")
    eps = t.full((1,), float("nan"), device="cuda")
    lam_out = t.full((1,), float("nan"), device="cuda")
    info = t.full((1,), -7, dtype=t.int32, device="cuda")
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d), dtype=t.uint8, device="cuda")
    ispa.absorb_solve(Gd, Cd, Wd, lam, relative, dW, info, ws, D=Dd, w_new=w_new, eps=eps if D is not None else None,
                      lambda_out=lam_out, refine=refine)
    t.cuda.synchronize()
    return {"dW": host(dW), "w_new": host(w_new), "eps": float(eps.item()), "lambda": float(lam_out.item()),
            "info": int(info.item())}


@pytest.mark.parametrize("d,n", [(32, 50), (96, 70), (128, 400), (160, 500), (256, 200), (320, 2000), (2112, 2500)])
@pytest.mark.parametrize("refine", [False, True])
def test_solve_matches_oracle(d, n, refine):
    """d <= 2048: one launch factorises; 2112 (33 panels): per-panel launches, R and P on the NT kernel."""
    G, C, D, W = _spd_problem(d, n, d + n)
    lam = oracle.ridge_lambda(G, 1e-3, True)
    got = _solve_gpu(G, C, D, W, 1e-3, True, refine=refine)
    assert got["info"] == 0
    assert abs(got["lambda"] - lam) <= 1e-6 * lam
    dW = oracle.solve_delta_w(G, C, W, lam)
    assert relfro(got["dW"], dW) <= 1e-3
    # the fold W_new = W + dW, checked against the kernel's own dW (fp32 storage)
    assert maxrel(got["w_new"], W + got["dW"]) <= 1e-6
    eps = oracle.recon_error_traces(G, C, D, W, dW, lam)
    assert abs(got["eps"] - eps) <= 1e-2 * eps


@pytest.mark.parametrize("d", [192, 2112])
@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_solve_16bit_weights(w_dtype, d):
    G, C, D, W = _spd_problem(d, 300 if d < 1024 else 2500, 5, w_dtype)
    got = _solve_gpu(G, C, D, W, 0.05, False, w_dtype=w_dtype)
    dW = oracle.solve_delta_w(G, C, W, 0.05)
    assert got["info"] == 0 and abs(got["lambda"] - 0.05) < 1e-9
    assert relfro(got["dW"], dW) <= 1e-3
    # W_new = W + dW rounded to the weight type
    assert maxrel(got["w_new"], wl.round_to(W + got["dW"], w_dtype)) <= 1e-2


def test_solve_large_lambda_limit():
    """lambda -> infinity: dW = (G + lambda I)^-1 C W -> C W / lambda, and ||dW|| <= ||C W|| / lambda
    (G is positive semi-definite), against the oracle at lambda = 1e6 tr(G) / d."""
    d = 256
    G, C, D, W = _spd_problem(d, 400, 21)
    lam = oracle.ridge_lambda(G, 1e6, True)
    got = _solve_gpu(G, C, D, W, 1e6, True)
    assert got["info"] == 0 and abs(got["lambda"] - lam) <= 1e-6 * lam
    cw = C @ W
    assert np.linalg.norm(got["dW"]) <= np.linalg.norm(cw) / lam * (1 + 1e-5)
    assert relfro(got["dW"], oracle.solve_delta_w(G, C, W, lam)) <= 1e-3
    assert relfro(got["dW"], cw / lam) <= 1e-3    # first order in 1 / lambda: ||G|| / lambda ~ 1e-6 d


@pytest.mark.parametrize("d,n", [(256, 100), (640, 300)])
@pytest.mark.parametrize("refine", [False, True])
def test_solve_fewer_tokens_than_features(d, n, refine):
    """n < d (as at the 14B layer): G has rank n, so lambda = 1e-3 tr(G) / d alone lifts its null space
    and cond(G + lambda I) is about 1e3 d / n.  dW within 1e-3 of the float64 solve.

    epsilon is small here (the few tokens are fitted almost exactly), and the library evaluates it
    by the trace formula that holds at the optimum, num^2 = <D,P> - <dW,R> - lambda ||dW||^2
    (P = W W^T, R = C W).  An error e in dW moves that by -<e, R + 2 lambda dW> - lambda ||e||^2,
    to first order, where the exact formula would move to second order; so num^2 is held to that
    bound, computed from the measured e, plus 1e-6 of the traces for their fp32 inputs.  The
    formula itself, evaluated in float64 on the kernel's own dW, must match the kernel's num^2 to
    5e-7 of its traces (fp32 R and P; measured 1e-8 to 1e-7).  Here num^2 is itself only about 3e-7
    of the traces, so a small epsilon is known to a few percent at best from fp32 statistics."""
    G, C, D, W = _spd_problem(d, n, d + 3 * n)
    lam = oracle.ridge_lambda(G, 1e-3, True)
    got = _solve_gpu(G, C, D, W, 1e-3, True, refine=refine)
    assert got["info"] == 0
    dW = oracle.solve_delta_w(G, C, W, lam)
    err = relfro(got["dW"], dW)
    eps = oracle.recon_error_traces(G, C, D, W, dW, lam)
    Rm = C @ W
    den2 = np.sum(W * ((G + C + C.T + D) @ W))
    e = np.linalg.norm(got["dW"] - dW)
    slack = (e * np.linalg.norm(Rm + 2.0 * lam * dW) + lam * e * e
             + 1e-6 * (abs(np.sum(W * (D @ W))) + abs(np.sum(dW * Rm))))
    print(f"d={d} n={n} refine={refine}: dW rel-Frobenius {err:.2e}; eps {got['eps']:.4e} vs {eps:.4e}, "
          f"num^2 off by {abs(got['eps'] ** 2 - eps ** 2) * den2:.2e} of a {slack:.2e} bound")
    assert err <= 1e-3
    assert abs(got["eps"] ** 2 - eps ** 2) * den2 <= slack
    g = got["dW"]
    dp, gr, gg = np.sum(W * (D @ W)), np.sum(g * Rm), lam * np.sum(g * g)
    dev_rel = abs(got["eps"] ** 2 * den2 - (dp - gr - gg)) / (abs(dp) + abs(gr) + gg)
    print(f"  kernel num^2 against the formula on its own dW: {dev_rel:.2e} of the traces")
    assert dev_rel <= 5e-7


@pytest.mark.parametrize("bad", [1, 70, 129])
def test_solve_reports_first_nonpositive_pivot(bad):
    """info = k (1-based) when the leading minor of order k of G + lambda I is not positive definite."""
    d = 160
    G = np.eye(d)
    G[bad - 1, bad - 1] = -1.0
    C = np.zeros((d, d))
    W = np.eye(d)
    got = _solve_gpu(G, C, None, W, 0.0, False)
    assert got["info"] == bad


def test_absorb_nothing_to_absorb():
    """A_loc = A_full: C = 0, so dW = 0 exactly."""
    G, _, D, W = _spd_problem(128, 300, 9)
    got = _solve_gpu(G, np.zeros_like(G), np.zeros_like(G), W, 1e-2, False)
    assert got["info"] == 0 and np.all(got["dW"] == 0.0) and got["eps"] == 0.0


def _warmup_chain(w, chunks, layer=0, refine=False):
    """dual attention per chunk -> Gram accumulation -> solve, all through the C ABI."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    s = w.shape
    d = s.d
    G = t.empty((d, d), device="cuda")
    C = t.empty((d, d), device="cuda")
    D = t.empty((d, d), device="cuda")
    ref_chunks = []
    for i, c in enumerate(chunks):
        x = wl.layer_inputs(w, chunk=c, layer=layer, with_w=False)
        ld = ((s.n_q + 7) // 8) * 8
        a_t = t.empty((d, ld), dtype=tdtype(w.stat_dtype), device="cuda")
        da_t = t.empty((d, ld), dtype=tdtype(w.stat_dtype), device="cuda")
        sh = ispa.AttnShape.of(s)
        ws = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, sh), dtype=t.uint8, device="cuda")
        ispa.dual_attn(sh, dev(x["q"], w.dtype), dev(x["k"], w.dtype), dev(x["v"], w.dtype),
                       a_loc_t=a_t, delta_a_t=da_t, ld_stat=ld, workspace=ws)
        ispa.gram_accum(a_t, da_t, s.n_q, G, C, D, accumulate=i > 0)
        r = oracle.dual_stream(x["q"], x["k"], x["v"], s.n_sink, s.n_hist, s.n_cur, s.n_heads)
        ref_chunks.append((r["a_loc"], r["delta_a"], r["a_full"]))
    t.cuda.synchronize()
    W = wl.layer_inputs(w, chunk=0, layer=layer)["w"]
    got = _solve_gpu(host(G), host(C), host(D), W, w.lam, w.lam_relative, w_dtype=w.dtype, refine=refine)
    Gr, Cr, Dr = oracle.gram_stats([(a, da) for a, da, _ in ref_chunks])
    lam = oracle.ridge_lambda(Gr, w.lam, w.lam_relative)
    dW = oracle.solve_delta_w(Gr, Cr, W, lam)
    eps_direct = oracle.recon_error_direct(np.concatenate([a for a, _, _ in ref_chunks]),
                                           np.concatenate([f for _, _, f in ref_chunks]), W, dW)
    return got, dW, eps_direct, (host(G), Gr)


def test_tiny_workload_end_to_end():
    """Tiny fp32 workload: 4 warmup chunks -> G, C, D -> dW, eps; fp32 tolerances."""
    got, dW, eps, (G, Gr) = _warmup_chain(wl.TINY, range(4))
    assert maxrel(G, Gr) <= 1e-4
    assert got["info"] == 0
    assert relfro(got["dW"], dW) <= 1e-3
    assert abs(got["eps"] - eps) <= 1e-3 * eps


def test_bf16_small_end_to_end():
    """A scaled-down bf16 layer (2 heads x 128, ragged chunk) through the whole chain; bf16 tolerances."""
    w = wl.Workload("small_bf16", 77, wl.AttnShape(600, 150, 450, 600, 2, 128), "bf16", "f16", 1e-3, True)
    got, dW, eps, _ = _warmup_chain(w, range(2))
    assert got["info"] == 0
    assert relfro(got["dW"], dW) <= 1e-2
    assert abs(got["eps"] - eps) <= 1e-2 * eps


@pytest.mark.parametrize("d,layers,refine", [(96, 2, 0), (256, 3, 0), (1536, 4, 0), (320, 2, 1), (2048, 2, 0), (2112, 2, 1)])
def test_batched_solve_equals_per_layer_calls(d, layers, refine):
    """ispa_absorb_solve_batched: every layer's dW, W_new, eps, lambda and info equal those of a
    separate ispa_absorb_solve call, bit for bit; one layer is indefinite (info set, others intact);
    the per-layer results also match the oracle.  A batched call factorises panel by panel, a single
    call with d <= 2048 in one launch, so this also checks the two factorisations against each other
    (d = 96: two panels, the second partial; d = 2048: the largest one-launch size)."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    probs = [_spd_problem(d, 2 * d + 7 * l, 100 + l, "bf16") for l in range(layers)]
    G = t.stack([dev(p[0], "f32") for p in probs])
    C = t.stack([dev(p[1], "f32") for p in probs])
    D = t.stack([dev(p[2], "f32") for p in probs])
    W = t.stack([dev(p[3], "bf16") for p in probs])
    bad = layers - 1 if layers > 2 else None
    if bad is not None:
        G[bad, 5, 5] = -1e3                       # not positive definite: info = 6
    dW = t.full((layers, d, d), float("nan"), device="cuda")
    w_new = t.empty((layers, d, d), dtype=t.bfloat16, device="cuda")
    eps = t.full((layers,), float("nan"), device="cuda")
    lam = t.full((layers,), float("nan"), device="cuda")
    info = t.full((layers,), -7, dtype=t.int32, device="cuda")
    ws_one = ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d)
    ws = t.empty(layers * ws_one, dtype=t.uint8, device="cuda")
    ispa.absorb_solve_batched(G, C, W, 1e-3, True, dW, info, ws, D=D, w_new=w_new, eps=eps, lambda_out=lam,
                              refine=refine)
    t.cuda.synchronize()
    for l in range(layers):
        dW1 = t.empty((d, d), device="cuda")
        wn1 = t.empty((d, d), dtype=t.bfloat16, device="cuda")
        e1, l1 = t.empty((1,), device="cuda"), t.empty((1,), device="cuda")
        i1 = t.empty((1,), dtype=t.int32, device="cuda")
        ispa.absorb_solve(G[l].contiguous(), C[l].contiguous(), W[l].contiguous(), 1e-3, True, dW1, i1,
                          ws[:ws_one], D=D[l].contiguous(), w_new=wn1, eps=e1, lambda_out=l1, refine=refine)
        t.cuda.synchronize()
        assert int(info[l].item()) == int(i1.item())
        if l == bad:
            assert int(i1.item()) == 6
            continue
        assert int(i1.item()) == 0
        assert t.equal(dW[l], dW1) and t.equal(w_new[l], wn1)
        assert t.equal(eps[l:l + 1], e1) and t.equal(lam[l:l + 1], l1)
        Gp, Cp, Dp, Wp = probs[l]
        lam_ref = oracle.ridge_lambda(Gp, 1e-3, True)
        assert relfro(host(dW1), oracle.solve_delta_w(Gp, Cp, Wp, lam_ref)) <= 1e-3
