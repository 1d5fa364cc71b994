"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes an implementation namespace (the real ``oracle`` package,
or a copy with a planted mistake) and raises AssertionError when the pin fails.
The pins come from the ISPA pages and from mathematics:

* brute-force attention in pure Python on tiny inputs (definition of softmax);
* hand-computed worked examples under tests/golden/ (each cites its passage);
* closed forms and special cases (Q = 0, one key, duplicated or empty history);
* the decomposable-attention identity: merging the local and history branches
  through their log-sum-exp equals the separate full pass;
* ridge facts: normal-equation residual, an independent SVD least-squares route
  on the augmented system, lambda limits, linearity in W, optimality and
  convexity, row-space property when tokens < features;
* accounting closed forms for FLOPs and KV bytes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def brute_attention(q, k, v, rows, n_heads, scale):
    """Softmax written as its definition, exp(s_j) / sum_k exp(s_k), in pure Python floats."""
    n_q, d = len(q), len(q[0])
    dh = d // n_heads
    out = [[0.0] * d for _ in range(n_q)]
    lse = [[-math.inf] * n_q for _ in range(n_heads)]
    if not rows:
        return out, lse
    for h in range(n_heads):
        for i in range(n_q):
            e = []
            for j in rows:
                s = sum(q[i][h * dh + c] * k[j][h * dh + c] for c in range(dh)) * scale
                e.append(math.exp(s))
            z = sum(e)
            lse[h][i] = math.log(z)
            for c in range(dh):
                out[i][h * dh + c] = sum(e[t] * v[rows[t]][h * dh + c] for t in range(len(rows))) / z
    return out, lse


def check_brute_force(impl, seed=0):
    rng = _rng(seed)
    for (n_sink, n_hist, n_cur, n_heads, dh, n_q) in [(1, 2, 3, 2, 3, 3), (2, 3, 1, 1, 4, 2), (1, 0, 2, 2, 2, 1)]:
        n_k = n_sink + n_hist + n_cur
        d = n_heads * dh
        q = rng.standard_normal((n_q, d))
        k = rng.standard_normal((n_k, d))
        v = rng.standard_normal((n_k, d))
        scale = 1.0 / math.sqrt(dh)
        r = impl.dual_stream(q, k, v, n_sink, n_hist, n_cur, n_heads)
        local = list(range(n_sink)) + list(range(n_sink + n_hist, n_k))
        hist = list(range(n_sink, n_sink + n_hist))
        for name, rows in (("loc", local), ("full", list(range(n_k))), ("hist", hist)):
            o_ref, l_ref = brute_attention(q.tolist(), k.tolist(), v.tolist(), rows, n_heads, scale)
            o_key = {"loc": "a_loc", "full": "a_full", "hist": "o_hist"}[name]
            assert np.allclose(r[o_key], np.array(o_ref), rtol=0, atol=1e-13), name
            l_ref = np.array(l_ref)
            got = r["lse_" + name]
            fin = np.isfinite(l_ref)
            assert np.array_equal(np.isfinite(got), fin), name
            assert np.allclose(got[fin], l_ref[fin], rtol=0, atol=1e-13), name


def check_golden_attention(impl):
    g = _golden("attention_hand.json")
    r = impl.dual_stream(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["n_sink"], g["n_hist"],
                         g["n_cur"], g["n_heads"], scale=g["scale"])
    for key in ("a_loc", "lse_loc", "o_hist", "lse_hist", "a_full", "lse_full", "delta_a"):
        assert np.allclose(r[key], np.array(g["expect"][key]), rtol=1e-14, atol=1e-14), key
    merged, lse = impl.lse_merge(r["a_loc"], r["lse_loc"], r["o_hist"], r["lse_hist"], g["n_heads"])
    assert np.allclose(merged, np.array(g["expect"]["a_full"]), rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, np.array(g["expect"]["lse_full"]), rtol=1e-14, atol=1e-14)


def check_q_zero(impl, seed=1):
    rng = _rng(seed)
    n_sink, n_hist, n_cur, H, dh = 5, 7, 4, 3, 8
    n_k = n_sink + n_hist + n_cur
    k = rng.standard_normal((n_k, H * dh))
    v = rng.standard_normal((n_k, H * dh))
    q = np.zeros((6, H * dh))
    r = impl.dual_stream(q, k, v, n_sink, n_hist, n_cur, H)
    loc = np.r_[0:n_sink, n_sink + n_hist:n_k]
    assert np.allclose(r["a_loc"], v[loc].mean(0), atol=1e-14)
    assert np.allclose(r["a_full"], v.mean(0), atol=1e-14)
    assert np.allclose(r["lse_loc"], math.log(n_sink + n_cur), atol=1e-14)
    assert np.allclose(r["lse_full"], math.log(n_k), atol=1e-14)
    assert np.allclose(r["lse_hist"], math.log(n_hist), atol=1e-14)


def check_single_row(impl, seed=2):
    rng = _rng(seed)
    H, dh = 2, 4
    q = rng.standard_normal((3, H * dh))
    k = rng.standard_normal((1, H * dh))
    v = rng.standard_normal((1, H * dh))
    o, lse = impl.softmax_attention(q, k, v, np.array([0]), H)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-15)
    for h in range(H):
        s = q[:, h * dh:(h + 1) * dh] @ k[0, h * dh:(h + 1) * dh] / math.sqrt(dh)
        assert np.allclose(lse[h], s, atol=1e-14)


def check_merge_identity(impl, seed=3):
    rng = _rng(seed)
    for (n_sink, n_hist, n_cur, H, dh, n_q) in [(64, 256, 64, 2, 64, 48), (17, 93, 31, 3, 16, 29), (1, 1, 1, 1, 8, 5)]:
        n_k = n_sink + n_hist + n_cur
        q = rng.standard_normal((n_q, H * dh)) * 2.0
        k = rng.standard_normal((n_k, H * dh))
        v = rng.standard_normal((n_k, H * dh))
        r = impl.dual_stream(q, k, v, n_sink, n_hist, n_cur, H)
        merged, lse = impl.lse_merge(r["a_loc"], r["lse_loc"], r["o_hist"], r["lse_hist"], H)
        assert np.max(np.abs(merged - r["a_full"])) <= 1e-12 * np.max(np.abs(r["a_full"]))
        assert np.max(np.abs(lse - r["lse_full"])) <= 1e-12 * np.max(np.abs(r["lse_full"]))
        assert np.allclose(r["delta_a"], merged - r["a_loc"], atol=1e-12)


def check_duplicate_history(impl, seed=4):
    """History rows an exact copy of the local rows: A_full = A_loc, LSE_full = LSE_loc + ln 2."""
    rng = _rng(seed)
    n_sink, n_cur, H, dh = 6, 10, 2, 8
    ks = rng.standard_normal((n_sink, H * dh))
    kc = rng.standard_normal((n_cur, H * dh))
    vs = rng.standard_normal((n_sink, H * dh))
    vc = rng.standard_normal((n_cur, H * dh))
    k = np.concatenate([ks, kc, ks, kc])
    v = np.concatenate([vs, vc, vs, vc])
    q = rng.standard_normal((7, H * dh))
    r = impl.dual_stream(q, k, v, n_sink, n_sink + n_cur, n_cur, H)
    # history = rows [n_sink, 2 n_sink + n_cur) = kc, ks (a permutation of the local rows)
    assert np.allclose(r["a_full"], r["a_loc"], atol=1e-14)
    assert np.allclose(r["lse_full"], r["lse_loc"] + math.log(2.0), atol=1e-13)
    assert np.max(np.abs(r["delta_a"])) < 1e-14


def check_empty_history(impl, seed=5):
    rng = _rng(seed)
    n_sink, n_cur, H, dh = 4, 9, 2, 8
    q = rng.standard_normal((5, H * dh))
    k = rng.standard_normal((n_sink + n_cur, H * dh))
    v = rng.standard_normal((n_sink + n_cur, H * dh))
    r = impl.dual_stream(q, k, v, n_sink, 0, n_cur, H)
    assert np.array_equal(r["a_full"], r["a_loc"])
    assert np.all(r["delta_a"] == 0.0)
    assert np.all(np.isneginf(r["lse_hist"]))
    merged, lse = impl.lse_merge(r["a_loc"], r["lse_loc"], r["o_hist"], r["lse_hist"], H)
    assert np.array_equal(merged, r["a_loc"]) and np.array_equal(lse, r["lse_loc"])


def check_split_invariance(impl, seed=6):
    """Splitting a key set into ranges and LSE-merging the range passes = one pass over the set."""
    rng = _rng(seed)
    H, dh, n_k = 2, 8, 50
    q = rng.standard_normal((9, H * dh))
    k = rng.standard_normal((n_k, H * dh))
    v = rng.standard_normal((n_k, H * dh))
    ref_o, ref_l = impl.softmax_attention(q, k, v, np.arange(n_k), H)
    cuts = [0, 7, 8, 33, n_k]
    o, l = impl.softmax_attention(q, k, v, np.arange(cuts[0], cuts[1]), H)
    for a, b in zip(cuts[1:-1], cuts[2:]):
        o2, l2 = impl.softmax_attention(q, k, v, np.arange(a, b), H)
        o, l = impl.lse_merge(o, l, o2, l2, H)
    assert np.allclose(o, ref_o, atol=1e-13) and np.allclose(l, ref_l, atol=1e-13)


def check_permutations(impl, seed=7):
    rng = _rng(seed)
    n_sink, n_hist, n_cur, H, dh = 4, 11, 6, 2, 8
    n_k = n_sink + n_hist + n_cur
    q = rng.standard_normal((8, H * dh))
    k = rng.standard_normal((n_k, H * dh))
    v = rng.standard_normal((n_k, H * dh))
    r = impl.dual_stream(q, k, v, n_sink, n_hist, n_cur, H)
    perm = np.concatenate([rng.permutation(n_sink), n_sink + rng.permutation(n_hist),
                           n_sink + n_hist + rng.permutation(n_cur)])
    pq = rng.permutation(8)
    r2 = impl.dual_stream(q[pq], k[perm], v[perm], n_sink, n_hist, n_cur, H)
    for key in ("a_loc", "a_full", "delta_a"):
        assert np.allclose(r2[key], r[key][pq], atol=1e-13), key
    G, C, D = impl.gram_stats([(r["a_loc"], r["delta_a"])])
    G2, C2, D2 = impl.gram_stats([(r2["a_loc"], r2["delta_a"])])
    assert np.allclose(G, G2, atol=1e-13) and np.allclose(C, C2, atol=1e-13) and np.allclose(D, D2, atol=1e-13)


# ----------------------------------------------------------------------------
# absorption
# ----------------------------------------------------------------------------
def _objective(a_loc, a_full, W, dW, lam):
    return float(np.sum((a_loc @ (W + dW) - a_full @ W) ** 2) + lam * np.sum(dW ** 2))


def check_golden_ridge(impl):
    for name in ("ridge_hand_d1.json", "ridge_hand_d2.json"):
        g = _golden(name)
        a_loc, a_full, W = (np.array(g[x]) for x in ("a_loc", "a_full", "w"))
        G, C, D = impl.gram_stats([(a_loc, a_full - a_loc)])
        e = g["expect"]
        assert np.allclose(G, e["G"], atol=1e-14) and np.allclose(C, e["C"], atol=1e-14), name
        assert np.allclose(D, e["D"], atol=1e-14), name
        lam = impl.ridge_lambda(G, g["lambda"], False)
        dW = impl.solve_delta_w(G, C, W, lam)
        assert np.allclose(dW, e["delta_w"], atol=1e-14), name
        if "objective" in e:
            assert abs(_objective(a_loc, a_full, W, dW, lam) - e["objective"]) < 1e-12
        assert abs(impl.recon_error_direct(a_loc, a_full, W, dW) - e["eps"]) < 1e-14, name
        assert abs(impl.recon_error_traces(G, C, D, W, dW, lam) - e["eps"]) < 1e-12, name


def _ridge_problem(seed, n, d, dout=None, lam=0.3):
    rng = _rng(seed)
    a_loc = rng.standard_normal((n, d)) * 0.05
    da = rng.standard_normal((n, d)) * 0.03 + 0.2 * a_loc @ rng.standard_normal((d, d)) / math.sqrt(d)
    W = rng.standard_normal((d, dout or d)) / math.sqrt(d)
    return a_loc, da, W, lam


def check_residual(impl):
    for (n, d) in [(300, 96), (64, 128), (1000, 64)]:
        a_loc, da, W, lam = _ridge_problem(10 + d, n, d, lam=1e-3)
        G, C, D = impl.gram_stats([(a_loc, da)])
        lam = impl.ridge_lambda(G, lam, True)
        dW = impl.solve_delta_w(G, C, W, lam)
        assert impl.normal_equation_residual(G, C, W, dW, lam) <= 1e-10


def check_augmented_lstsq(impl):
    """Ridge = ordinary least squares on [A_loc; sqrt(lam) I] X ~ [dA W; 0], solved by SVD."""
    for (n, d) in [(200, 40), (30, 60)]:
        a_loc, da, W, lam = _ridge_problem(20 + d, n, d)
        G, C, D = impl.gram_stats([(a_loc, da)])
        dW = impl.solve_delta_w(G, C, W, lam)
        A_aug = np.concatenate([a_loc, math.sqrt(lam) * np.eye(d)])
        B_aug = np.concatenate([da @ W, np.zeros((d, W.shape[1]))])
        X, *_ = np.linalg.lstsq(A_aug, B_aug, rcond=None)
        assert np.linalg.norm(dW - X) <= 1e-9 * np.linalg.norm(X)


def check_lambda_limits(impl):
    a_loc, da, W, _ = _ridge_problem(30, 400, 32)
    G, C, D = impl.gram_stats([(a_loc, da)])
    R = C @ W
    big = 1e12
    dW = impl.solve_delta_w(G, C, W, big)
    assert np.linalg.norm(big * dW - R) <= 1e-8 * np.linalg.norm(R)
    assert np.linalg.norm(dW) <= 1e-9 * np.linalg.norm(W)
    dW0 = impl.solve_delta_w(G, C, W, 1e-13)
    X = np.linalg.solve(G, R)
    assert np.linalg.norm(dW0 - X) <= 1e-8 * np.linalg.norm(X)


def check_relative_lambda(impl):
    """Orthonormal A_loc columns give G = I, so the relative rule yields lambda = lam_rel exactly."""
    rng = _rng(31)
    n, d = 50, 12
    Q, _ = np.linalg.qr(rng.standard_normal((n, d)))
    da = rng.standard_normal((n, d))
    W = rng.standard_normal((d, d))
    G, C, D = impl.gram_stats([(Q, da)])
    lam = impl.ridge_lambda(G, 0.25, True)
    assert abs(lam - 0.25) < 1e-13
    dW = impl.solve_delta_w(G, C, W, lam)
    assert np.allclose(dW, (Q.T @ da @ W) / 1.25, atol=1e-12)


def check_linearity_in_w(impl):
    a_loc, da, W1, lam = _ridge_problem(40, 120, 24)
    W2 = _rng(41).standard_normal(W1.shape)
    G, C, D = impl.gram_stats([(a_loc, da)])
    lhs = impl.solve_delta_w(G, C, 2.0 * W1 - 3.0 * W2, lam)
    rhs = 2.0 * impl.solve_delta_w(G, C, W1, lam) - 3.0 * impl.solve_delta_w(G, C, W2, lam)
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


def check_optimality(impl):
    a_loc, da, W, lam = _ridge_problem(50, 150, 20)
    a_full = a_loc + da
    G, C, D = impl.gram_stats([(a_loc, da)])
    dW = impl.solve_delta_w(G, C, W, lam)
    grad = 2.0 * (a_loc.T @ (a_loc @ (W + dW) - a_full @ W)) + 2.0 * lam * dW
    assert np.linalg.norm(grad) <= 1e-10 * np.linalg.norm(a_loc.T @ a_full @ W)
    f0 = _objective(a_loc, a_full, W, dW, lam)
    rng = _rng(51)
    for t in (1e-3, 1e-1, 1.0):
        E = rng.standard_normal(dW.shape)
        assert _objective(a_loc, a_full, W, dW + t * E, lam) > f0


def check_rowspace(impl):
    """Fewer tokens than features: dW lies in the row space of A_loc."""
    a_loc, da, W, lam = _ridge_problem(60, 20, 48)
    G, C, D = impl.gram_stats([(a_loc, da)])
    dW = impl.solve_delta_w(G, C, W, lam)
    Qr, _ = np.linalg.qr(a_loc.T)           # basis of the row space
    off = dW - Qr @ (Qr.T @ dW)
    assert np.linalg.norm(off) <= 1e-10 * np.linalg.norm(dW)


def check_eps_two_ways(impl):
    a_loc, da, W, lam = _ridge_problem(70, 200, 30)
    a_full = a_loc + da
    G, C, D = impl.gram_stats([(a_loc, da)])
    dW = impl.solve_delta_w(G, C, W, lam)
    for X in (dW, 0.7 * dW, np.zeros_like(dW)):
        e1 = impl.recon_error_direct(a_loc, a_full, W, X)
        e2 = impl.recon_error_traces(G, C, D, W, X, lam)
        assert abs(e1 - e2) <= 1e-8 * e1
    # no absorption: epsilon = ||dA W|| / ||A_full W||
    e0 = impl.recon_error_direct(a_loc, a_full, W, np.zeros_like(dW))
    assert abs(e0 - np.linalg.norm(da @ W) / np.linalg.norm(a_full @ W)) < 1e-13
    assert impl.recon_error_direct(a_loc, a_full, W, dW) < e0


def check_zero_absorb(impl):
    """A_loc = A_full (nothing to absorb) gives dW = 0 and epsilon = 0."""
    rng = _rng(80)
    a = rng.standard_normal((40, 16))
    W = rng.standard_normal((16, 16))
    G, C, D = impl.gram_stats([(a, a - a)])
    dW = impl.solve_delta_w(G, C, W, 0.1)
    assert np.all(dW == 0.0)
    assert impl.recon_error_direct(a, a, W, dW) == 0.0


def check_gram_associativity(impl):
    rng = _rng(90)
    chunks = [(rng.standard_normal((n, 24)), rng.standard_normal((n, 24))) for n in (13, 40, 7, 29)]
    G, C, D = impl.gram_stats(chunks)
    A = np.concatenate([c[0] for c in chunks])
    B = np.concatenate([c[1] for c in chunks])
    G1, C1, D1 = impl.gram_stats([(A, B)])
    assert np.allclose(G, G1, atol=1e-12) and np.allclose(C, C1, atol=1e-12) and np.allclose(D, D1, atol=1e-12)


def check_selection(impl):
    eps = [0.5, 0.1, 0.3, 0.1, 0.9, 0.3]
    assert list(impl.select_local_layers(eps, 3)) == [1, 2, 3]
    assert list(impl.select_local_layers(eps, 2)) == [1, 3]
    assert list(impl.select_local_layers(eps, 4)) == [1, 2, 3, 5]
    assert list(impl.select_local_layers(eps, 0)) == []
    # a NaN error (a failed absorption) ranks last and is never converted: two numbers for k = 3
    assert list(impl.select_local_layers([0.5, float("nan"), 0.3, float("nan")], 3)) == [0, 2]


def check_golden_l_layer(impl):
    """Hand-worked converted-layer step: local attention over sink + current rows, then A @ W_new."""
    g = _golden("l_layer_hand.json")
    q, k, v, w = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v", "w_new"))
    out = impl.local_layer_output(q, k, v, g["n_sink"], g["n_cur"], g["n_heads"], w)
    assert np.allclose(out, np.array(g["expect"]["out"]), rtol=0, atol=1e-13)
    # the identity projection leaves the attention output itself
    att = impl.local_layer_output(q, k, v, g["n_sink"], g["n_cur"], g["n_heads"], np.eye(w.shape[0]))
    assert np.allclose(att, np.array(g["expect"]["attention"]), rtol=0, atol=1e-13)


def check_golden_residual_and_fold(impl):
    g = _golden("residual_fold_hand.json")
    r = g["residual"]
    got = impl.normal_equation_residual(*(np.array(r[x]) for x in ("G", "C", "w", "delta_w")), r["lambda"])
    assert abs(got - r["expect"]) <= 1e-15
    f = g["fold"]
    assert np.array_equal(impl.fold_weights(np.array(f["w"]), np.array(f["delta_w"])), np.array(f["expect"]))


def check_golden_w8a8_l_layer(impl):
    """W8A8 converted-layer step where the bf16 storage of the attention output decides an E4M3 code."""
    g = _golden("w8a8_l_layer_hand.json")
    q, k, v, w = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v", "w"))
    out = impl.local_layer_output_w8a8(q, k, v, g["n_sink"], g["n_cur"], g["n_heads"], w)
    assert np.array_equal(out, np.array(g["expect"]["out"]))


def check_golden_w8a8_fp8attn_l_layer(impl):
    """W8A8 converted-layer step with FP8 attention: exact FP8 attention (Q = 0, four local rows), bf16
    storage that decides an activation code, a non-symmetric W; then the W8A8 fixture's inputs, where the
    FP8 coding of V decides a code; and the weight codes of a non-square W."""
    g = _golden("w8a8_fp8attn_l_layer_hand.json")
    q, k, v, w = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v", "w"))
    out = impl.local_layer_output_w8a8_fp8attn(q, k, v, g["n_sink"], g["n_cur"], g["n_heads"], w)
    assert np.array_equal(out, np.array(g["expect"]["out"]))
    h = _golden("w8a8_l_layer_hand.json")
    q, k, v, w = (np.array(h[x], dtype=np.float64) for x in ("q", "k", "v", "w"))
    out = impl.local_layer_output_w8a8_fp8attn(q, k, v, h["n_sink"], h["n_cur"], h["n_heads"], w)
    assert np.array_equal(out, np.array(g["expect"]["case2_out"]))
    qw = g["quantize_weight"]
    codes, scales = impl.quantize_weight(np.array(qw["w"]))
    assert np.array_equal(np.asarray(codes), np.array(qw["codes"])) and np.array_equal(np.asarray(scales), np.array(qw["scales"]))


def check_golden_fp8_attention(impl):
    """Hand-worked FP8 attention of a converted layer: dominant key, rounding against the integer
    reference, Q = 0."""
    g = _golden("fp8_attention_hand.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v"))
    out = impl.local_attention_fp8(q, k, v, g["n_sink"], g["n_cur"], g["n_heads"], scale=g["scale"])
    assert np.allclose(out, np.array(g["expect"]["out"]), rtol=1e-13, atol=1e-12)
    c = g["case2"]
    q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
    out = impl.local_attention_fp8(q, k, v, c["n_sink"], c["n_cur"], c["n_heads"], scale=c["scale"])
    assert np.allclose(out, np.array(c["expect"]["out"]), rtol=1e-13, atol=1e-12)


def check_fp8_attention_structure(impl, seed=11):
    """Without rounding the FP8 attention is plain softmax attention over the layer's rows; with it the
    error is quantisation-sized; V scaled by a power of two scales the output exactly (codes and
    probabilities unchanged); the order of the key rows within each segment does not matter."""
    rng = _rng(seed)
    n_sink, n_cur, H, dh = 7, 25, 2, 16
    q = rng.standard_normal((9, H * dh))
    k = rng.standard_normal((n_sink + n_cur, H * dh))
    v = rng.standard_normal((n_sink + n_cur, H * dh))
    exact, _ = impl.softmax_attention(q, k, v, np.arange(n_sink + n_cur), H)
    plain = impl.local_attention_fp8(q, k, v, n_sink, n_cur, H, quantize=False)
    assert np.allclose(plain, exact, atol=1e-13)
    got = impl.local_attention_fp8(q, k, v, n_sink, n_cur, H)
    err = np.max(np.abs(got - exact)) / np.max(np.abs(exact))
    assert 1e-3 < err < 0.25, err
    assert np.array_equal(impl.local_attention_fp8(q, k, 4.0 * v, n_sink, n_cur, H), 4.0 * got)
    perm = np.concatenate([rng.permutation(n_sink), n_sink + rng.permutation(n_cur)])
    assert np.allclose(impl.local_attention_fp8(q, k[perm], v[perm], n_sink, n_cur, H), got, atol=1e-12)


# ----------------------------------------------------------------------------
# accounting
# ----------------------------------------------------------------------------
def check_kv_bytes(impl):
    frame, cf, d, L = 1560, 3, 1536, 30
    for chunk in (0, 1, 7, 39):
        n_local = 15
        count = 0
        for layer in range(L):
            rows = list(range(frame))                                  # sink frame
            if layer >= n_local:                                       # F-layer keeps history
                rows += list(range(frame, frame * (1 + cf * chunk)))
            rows += list(range(frame * (1 + cf * chunk), frame * (1 + cf * chunk + cf)))  # current chunk
            count += 2 * len(rows) * d * 2
        assert impl.kv_cache_bytes(chunk, L, n_local, frame, cf, d) == count
    f39 = impl.kv_removed_fraction(39, L, 15, frame, cf, d)
    assert abs(f39 - (1.0 - 125.0 / 242.0)) < 1e-12       # 1 - (121 + 4) / (2 * 121) = 48.3%
    # "up to 50%": converting half the layers approaches one half as history grows
    assert impl.kv_removed_fraction(10_000, L, 15, frame, cf, d) < 0.5
    assert impl.kv_removed_fraction(10_000, L, 15, frame, cf, d) > 0.4999
    assert impl.kv_removed_fraction(0, L, 15, frame, cf, d) == 0.0


def check_flops(impl):
    # the dual-stream call does the work of exactly one full attention
    f_loc = impl.attn_flops(4680, 1560 + 4680, 128, 12)
    f_hist = impl.attn_flops(4680, 14040, 128, 12)
    assert f_loc + f_hist == impl.attn_flops(4680, 20280, 128, 12) == 583_129_497_600


ATTENTION_PINS = [check_brute_force, check_golden_attention, check_q_zero, check_single_row,
                  check_merge_identity, check_duplicate_history, check_empty_history,
                  check_split_invariance, check_permutations]
ABSORB_PINS = [check_golden_ridge, check_residual, check_augmented_lstsq, check_lambda_limits,
               check_relative_lambda, check_linearity_in_w, check_optimality, check_rowspace,
               check_eps_two_ways, check_zero_absorb, check_gram_associativity, check_selection,
               check_golden_l_layer, check_golden_residual_and_fold, check_golden_w8a8_l_layer,
               check_golden_fp8_attention, check_fp8_attention_structure, check_golden_w8a8_fp8attn_l_layer]
ACCOUNTING_PINS = [check_kv_bytes, check_flops]
ALL_PINS = ATTENTION_PINS + ABSORB_PINS + ACCOUNTING_PINS
