"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows the pins are strong enough: a dropped term, a wrong sign or index,
a transposed operand or a missing regulariser anywhere in the oracle is caught.
The mistakes are planted on the CPU, in copies; the oracle itself is untouched.
"""
import math
import types

import numpy as np
import pytest

import oracle
from oracle import fp8
from oracle_pins import ALL_PINS

NAMES = ["branch_rows", "softmax_attention", "dual_stream", "lse_merge", "gram_stats", "ridge_lambda",
         "solve_delta_w", "normal_equation_residual", "recon_error_direct", "recon_error_traces",
         "select_local_layers", "fold_weights", "local_layer_output", "attn_flops", "kv_cache_bytes",
         "kv_removed_fraction", "default_scale", "local_layer_output_w8a8", "local_attention_fp8"]
FP8_NAMES = ["local_layer_output_w8a8_fp8attn", "quantize_weight"]


def _ns(**over):
    ns = types.SimpleNamespace(**{n: getattr(oracle, n) for n in NAMES}, **{n: getattr(fp8, n) for n in FP8_NAMES})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _dual_with(softmax_fn=None, rows_fn=None, delta_sign=1.0):
    softmax_fn = softmax_fn or oracle.softmax_attention
    rows_fn = rows_fn or oracle.branch_rows

    def dual(q, k, v, n_sink, n_hist, n_cur, n_heads, scale=None, threads=1):
        rows = rows_fn(n_sink, n_hist, n_cur)
        a_loc, lse_loc = softmax_fn(q, k, v, rows["local"], n_heads, scale)
        a_full, lse_full = softmax_fn(q, k, v, rows["full"], n_heads, scale)
        o_hist, lse_hist = softmax_fn(q, k, v, rows["hist"], n_heads, scale)
        return {"a_loc": a_loc, "lse_loc": lse_loc, "a_full": a_full, "lse_full": lse_full,
                "o_hist": o_hist, "lse_hist": lse_hist, "delta_a": delta_sign * (a_full - a_loc)}
    return dual


def _softmax_variant(scale_fn=None, drop_max_in_lse=False):
    def attn(q, k, v, rows, n_heads, scale=None, q_block=512, threads=1):
        q = np.asarray(q, dtype=np.float64)
        n_q, d = q.shape
        dh = d // n_heads
        if scale is None:
            scale = scale_fn(dh) if scale_fn else 1.0 / math.sqrt(dh)
        out = np.zeros((n_q, d))
        lse = np.full((n_heads, n_q), -np.inf)
        rows = np.asarray(rows, dtype=np.int64)
        if rows.size == 0:
            return out, lse
        for h in range(n_heads):
            c = slice(h * dh, (h + 1) * dh)
            s = q[:, c] @ k[rows, c].T * scale
            m = s.max(1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(1, keepdims=True)
            out[:, c] = p @ v[rows, c] / l
            lse[h] = np.log(l)[:, 0] if drop_max_in_lse else (m + np.log(l))[:, 0]
        return out, lse
    return attn


def _rows_no_sink(n_sink, n_hist, n_cur):
    r = oracle.branch_rows(n_sink, n_hist, n_cur)
    r["local"] = np.arange(n_sink + n_hist, n_sink + n_hist + n_cur)
    return r


def _rows_off_by_one(n_sink, n_hist, n_cur):
    r = oracle.branch_rows(n_sink, n_hist, n_cur)
    if n_hist > 0:
        r["local"] = np.concatenate([np.arange(0, n_sink + 1), np.arange(n_sink + n_hist, n_sink + n_hist + n_cur)])
        r["hist"] = np.arange(n_sink + 1, n_sink + n_hist)
    return r


def _merge_wrong_weight(o_a, lse_a, o_b, lse_b, n_heads):
    dh = o_a.shape[1] // n_heads
    lse = np.logaddexp(lse_a, lse_b)
    w_a = np.exp(lse_a - lse)
    return o_a + np.repeat(w_a.T, dh, axis=1) * (np.nan_to_num(o_b) - o_a), lse


def _gram_transposed_c(chunks):
    G, C, D = oracle.gram_stats(chunks)
    return G, C.T, D


def _gram_swapped_c(chunks):
    chunks = list(chunks)
    G, _, D = oracle.gram_stats(chunks)
    _, C, _ = oracle.gram_stats([(b, a) for a, b in chunks])
    return G, C, D


def _gram_no_d(chunks):
    G, C, D = oracle.gram_stats(chunks)
    return G, C, G


def _solve_no_lambda(G, C, W, lam):
    return oracle.solve_delta_w(G, C, W, 0.0)


def _solve_w_transposed(G, C, W, lam):
    return oracle.solve_delta_w(G, C, np.asarray(W).T, lam)


def _solve_wc_order(G, C, W, lam):
    M = G + lam * np.eye(G.shape[0])
    return np.linalg.solve(M, (W @ C) if W.shape[0] == C.shape[0] else C @ W)


def _lambda_no_d(G, lam, relative):
    return float(lam) * float(np.trace(G)) if relative else float(lam)


def _traces_sign(G, C, D, W, dW, lam=None):
    R = C @ W
    num2 = np.sum(dW * (G @ dW)) + 2.0 * np.sum(dW * R) + np.sum(W * (D @ W))
    den2 = np.sum(W * ((G + C + C.T + D) @ W))
    return float(np.sqrt(max(num2, 0.0) / den2))


def _select_converts_nan(eps, k):
    return np.sort(np.argsort(np.asarray(eps, dtype=np.float64), kind="stable")[:k])


def _select_highest(eps, k):
    order = np.argsort(-np.asarray(eps, dtype=np.float64), kind="stable")
    return np.sort(order[:k])


def _kv_off_by_one(chunk, n_layers, n_local, frame, chunk_frames, d, elem_bytes=2):
    f_rows = frame * (chunk_frames * chunk + chunk_frames)          # sink frame dropped
    l_rows = frame * (1 + chunk_frames)
    return 2 * d * elem_bytes * ((n_layers - n_local) * f_rows + n_local * l_rows)


def _flops_half(n_q, n_k, head_dim, n_heads):
    return 2 * n_q * n_k * head_dim * n_heads


def _l_layer_w_transposed(q, k, v, n_sink, n_cur, n_heads, W_new, scale=None, threads=1):
    return oracle.local_layer_output(q, k, v, n_sink, n_cur, n_heads, np.asarray(W_new).T, scale, threads)


def _fold_subtracts(W, dW):
    return np.asarray(W, dtype=np.float64) - np.asarray(dW, dtype=np.float64)


def _residual_zero(G, C, W, dW, lam):
    return 0.0


def _residual_no_lambda(G, C, W, dW, lam):
    return oracle.normal_equation_residual(G, C, W, dW, 0.0)


def _w8a8_no_bf16_rounding(q, k, v, n_sink, n_cur, n_heads, W, scale=None, threads=1):
    rows = oracle.branch_rows(n_sink, 0, n_cur)["local"]
    a, _ = oracle.softmax_attention(q, k, v, rows, n_heads, scale, threads=threads)
    return fp8.w8a8_matmul(a.astype(np.float32), W)


def _fp8attn_layer_no_bf16(q, k, v, n_sink, n_cur, n_heads, W, scale=None):
    a = fp8.local_attention_fp8(q, k, v, n_sink, n_cur, n_heads, scale)
    return fp8.w8a8_matmul(a.astype(np.float32), W)


def _fp8attn_layer_float_attention(q, k, v, n_sink, n_cur, n_heads, W, scale=None):
    return fp8.local_layer_output_w8a8(q, k, v, n_sink, n_cur, n_heads, W, scale)


def _fp8attn_layer_w_transposed(q, k, v, n_sink, n_cur, n_heads, W, scale=None):
    return fp8.local_layer_output_w8a8_fp8attn(q, k, v, n_sink, n_cur, n_heads, np.asarray(W).T, scale)


def _quantize_weight_untransposed(W):
    return fp8.quantize_rows(np.asarray(W, dtype=np.float32))


def _fp8_attention_variant(reference="ceil", p_scale=256.0, l_from="codes", k_scale="head"):
    def attn(q, k, v, n_sink, n_cur, n_heads, scale=None, quantize=True):
        if not quantize:   # the planted mistakes are in the rounding only
            return oracle.local_attention_fp8(q, k, v, n_sink, n_cur, n_heads, scale, quantize=False)
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        n_q, d = q.shape
        dh = d // n_heads
        scale = 1.0 / math.sqrt(dh) if scale is None else scale
        rows = oracle.branch_rows(n_sink, 0, n_cur)["local"]
        out = np.zeros((n_q, d))

        def codes(x, s):
            y = np.clip((np.asarray(x, dtype=np.float32) / np.float32(s)).astype(np.float32), -448.0, 448.0)
            return fp8.e4m3_decode(fp8.e4m3_encode(y))

        def sc(a):
            m = np.float32(np.max(np.abs(a)))
            return np.float32(m / np.float32(448.0)) if m > 0 else np.float32(1.0)
        for h in range(n_heads):
            c = slice(h * dh, (h + 1) * dh)
            qh, kh, vh = q[:, c], k[rows, c], v[rows, c]
            sq = [sc(qh[i]) for i in range(n_q)]
            qd = np.stack([codes(qh[i], sq[i]) for i in range(n_q)])
            if k_scale == "head":
                sk = [sc(kh)] * len(rows)
            else:
                sk = [sc(kh[j]) for j in range(len(rows))]
            kd = np.stack([codes(kh[j], sk[j]) for j in range(len(rows))])
            sv = sc(vh)
            vd = codes(vh, sv)
            S = (qd @ kd.T) * np.array(sq, dtype=np.float64)[:, None] * np.array(sk, dtype=np.float64)[None, :]
            x = S * scale / math.log(2.0)
            m = np.max(x, axis=1, keepdims=True)
            M = np.ceil(m) if reference == "ceil" else m
            P = np.exp2(x - M)
            Pq = fp8.e4m3_decode(fp8.e4m3_encode(np.minimum(p_scale * P, 448.0).astype(np.float32))) / p_scale
            l = (Pq if l_from == "codes" else P).sum(axis=1, keepdims=True)
            out[:, c] = float(sv) * (Pq @ vd) / l
        return out
    return attn


MUTANTS = {
    "scale_1_over_d": dict(softmax_attention=_softmax_variant(scale_fn=lambda dh: 1.0 / dh),
                           dual_stream=_dual_with(_softmax_variant(scale_fn=lambda dh: 1.0 / dh))),
    "lse_drops_max": dict(softmax_attention=_softmax_variant(drop_max_in_lse=True),
                          dual_stream=_dual_with(_softmax_variant(drop_max_in_lse=True))),
    "local_set_without_sink": dict(dual_stream=_dual_with(rows_fn=_rows_no_sink)),
    "branch_boundary_off_by_one": dict(dual_stream=_dual_with(rows_fn=_rows_off_by_one)),
    "delta_a_sign": dict(dual_stream=_dual_with(delta_sign=-1.0)),
    "merge_weights_wrong_branch": dict(lse_merge=_merge_wrong_weight),
    "cross_term_transposed": dict(gram_stats=_gram_transposed_c),
    "cross_term_operands_swapped": dict(gram_stats=_gram_swapped_c),
    "d_term_dropped": dict(gram_stats=_gram_no_d),
    "solve_without_lambda": dict(solve_delta_w=_solve_no_lambda),
    "solve_with_w_transposed": dict(solve_delta_w=_solve_w_transposed),
    "solve_rhs_order": dict(solve_delta_w=_solve_wc_order),
    "relative_lambda_not_over_d": dict(ridge_lambda=_lambda_no_d),
    "eps_cross_sign": dict(recon_error_traces=_traces_sign),
    "select_highest": dict(select_local_layers=_select_highest),
    "select_converts_nan_layers": dict(select_local_layers=_select_converts_nan),
    "kv_rows_drop_sink": dict(kv_cache_bytes=_kv_off_by_one),
    "flops_half": dict(attn_flops=_flops_half),
    "l_layer_projects_by_w_transposed": dict(local_layer_output=_l_layer_w_transposed),
    "fold_subtracts_delta_w": dict(fold_weights=_fold_subtracts),
    "residual_returns_zero": dict(normal_equation_residual=_residual_zero),
    "residual_drops_lambda": dict(normal_equation_residual=_residual_no_lambda),
    "w8a8_skips_bf16_storage": dict(local_layer_output_w8a8=_w8a8_no_bf16_rounding),
    "fp8attn_layer_skips_bf16_storage": dict(local_layer_output_w8a8_fp8attn=_fp8attn_layer_no_bf16),
    "fp8attn_layer_float_attention": dict(local_layer_output_w8a8_fp8attn=_fp8attn_layer_float_attention),
    "fp8attn_layer_w_transposed": dict(local_layer_output_w8a8_fp8attn=_fp8attn_layer_w_transposed),
    "weight_codes_per_input_channel": dict(quantize_weight=_quantize_weight_untransposed),
    "fp8_reference_not_integer": dict(local_attention_fp8=_fp8_attention_variant(reference="max")),
    "fp8_probabilities_scaled_448": dict(local_attention_fp8=_fp8_attention_variant(p_scale=448.0)),
    "fp8_row_sum_unquantised": dict(local_attention_fp8=_fp8_attention_variant(l_from="exact")),
    "fp8_key_scales_per_token": dict(local_attention_fp8=_fp8_attention_variant(k_scale="token")),
}


def test_real_oracle_passes_all_pins():
    for pin in ALL_PINS:
        pin(_ns())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    ns = _ns(**MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns)
        except Exception as e:  # AssertionError, or a crash on nonsense (e.g. singular matrix)
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
