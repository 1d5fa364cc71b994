"""Oracle: attention over the local and full key sets (float64, CPU).

TEST INFRASTRUCTURE ONLY -- never imported by the GPU library.

Follows the ISPA technical summary (gist.science, nl/pt), section 2, stage 1
"Dual-Stream Warmup": during warmup an F-layer produces A_full, the attention
output over the whole cached history (the ground truth), and A_loc, the output
over local context only -- the current frame(s) and the sink tokens.  The
summary says the two are obtained in one pass by splitting attention into a
local and a historical branch and merging them afterwards through their
log-sum-exp states.  That merge is exact, so this oracle does NOT use it to
produce A_full: A_full comes from a separate plain pass over all rows, and the
merge (``lse_merge``) exists only so the tests can pin the identity.

Readings of points the pages leave open:
  * cache rows are ordered [sink | history | current chunk]; the local set is
    sink + current chunk, the history set is the rows in between;
  * no mask: every query sees every row of its set (chunk-level causality comes
    from which rows are cached);
  * scale = 1/sqrt(head_dim); log-sum-exp in natural log;
  * heads are contiguous column blocks of width head_dim in [tokens, d] tensors.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def branch_rows(n_sink: int, n_hist: int, n_cur: int) -> Dict[str, np.ndarray]:
    """Row indices of the local (sink + current), history and full sets of one cache."""
    n_k = n_sink + n_hist + n_cur
    local = np.concatenate([np.arange(0, n_sink), np.arange(n_sink + n_hist, n_k)])
    hist = np.arange(n_sink, n_sink + n_hist)
    return {"local": local, "hist": hist, "full": np.arange(n_k)}


def _head_pass(q_h, k_h, v_h, scale, q_block):
    """Two-pass softmax for one head: pass 1 takes the row max, pass 2 exponentiates and sums."""
    n_q = q_h.shape[0]
    out = np.empty((n_q, v_h.shape[1]))
    lse = np.empty(n_q)
    for i0 in range(0, n_q, q_block):
        s = (q_h[i0:i0 + q_block] @ k_h.T) * scale          # scores [bq, n_rows]
        m = s.max(axis=1, keepdims=True)                     # pass 1: row maximum
        p = np.exp(s - m)                                    # pass 2: shifted exponentials
        l = p.sum(axis=1, keepdims=True)
        out[i0:i0 + q_block] = (p @ v_h) / l
        lse[i0:i0 + q_block] = (m + np.log(l))[:, 0]
    return out, lse


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray, n_heads: int,
                      scale: Optional[float] = None, q_block: int = 512,
                      threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(q k_R^T * scale) v_R per head over the key rows R; returns (O [n_q,d], LSE [H,n_q]).

    An empty row set gives O = 0 and LSE = -inf (a branch with no keys has zero weight).
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, d = q.shape
    dh = d // n_heads
    scale = default_scale(dh) if scale is None else scale
    out = np.zeros((n_q, d))
    lse = np.full((n_heads, n_q), -np.inf)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return out, lse
    kr = np.asarray(k, dtype=np.float64)[rows]
    vr = np.asarray(v, dtype=np.float64)[rows]

    def one(h):
        c = slice(h * dh, (h + 1) * dh)
        return h, _head_pass(q[:, c], kr[:, c], vr[:, c], scale, q_block)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(one, range(n_heads)))
    else:
        results = [one(h) for h in range(n_heads)]
    for h, (o, l) in results:
        out[:, h * dh:(h + 1) * dh] = o
        lse[h] = l
    return out, lse


def dual_stream(q, k, v, n_sink: int, n_hist: int, n_cur: int, n_heads: int,
                scale: Optional[float] = None, threads: int = 1) -> Dict[str, np.ndarray]:
    """Everything one dual-stream call yields, each from its own plain pass.

    a_loc / lse_loc   : attention over the local set (sink + current chunk)
    a_full / lse_full : attention over all cached rows (separate pass)
    o_hist / lse_hist : attention over the history rows alone (LSE -inf if none)
    delta_a           : a_full - a_loc (exact in float64)
    """
    rows = branch_rows(n_sink, n_hist, n_cur)
    a_loc, lse_loc = softmax_attention(q, k, v, rows["local"], n_heads, scale, threads=threads)
    a_full, lse_full = softmax_attention(q, k, v, rows["full"], n_heads, scale, threads=threads)
    o_hist, lse_hist = softmax_attention(q, k, v, rows["hist"], n_heads, scale, threads=threads)
    return {"a_loc": a_loc, "lse_loc": lse_loc, "a_full": a_full, "lse_full": lse_full,
            "o_hist": o_hist, "lse_hist": lse_hist, "delta_a": a_full - a_loc}


def lse_merge(o_a, lse_a, o_b, lse_b, n_heads: int) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two branch outputs through their log-sum-exp states (decomposable attention).

    Each branch is a softmax over disjoint key sets; the softmax over the union
    weights branch b by exp(lse_b - lse) with lse = log(exp(lse_a) + exp(lse_b)).
    A branch with lse = -inf gets weight 0.
    """
    n_q, d = o_a.shape
    dh = d // n_heads
    lse = np.logaddexp(lse_a, lse_b)                         # [H, n_q]
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse))
    w_cols = np.repeat(w_b.T, dh, axis=1)                     # [n_q, d]
    o_b_safe = np.where(np.repeat(np.isneginf(lse_b).T, dh, axis=1), 0.0, o_b)
    return o_a + w_cols * (o_b_safe - o_a), lse
