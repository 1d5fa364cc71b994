"""Oracle: ridge absorption, reconstruction error and layer selection (float64, CPU).

TEST INFRASTRUCTURE ONLY -- never imported by the GPU library.

Follows the ISPA technical summary (gist.science, nl/pt), section 2:

* stage 2 "Layer Absorb": find the weight modulation dW minimising
  ||A_loc (W + dW) - A_full W||^2 + lambda ||dW||^2 (first displayed equation);
  its analytic minimiser is dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W
  (second displayed equation), computed without iteration or gradients;
* stage 3 "Memory-Efficient Inference": selected layers run on local context
  with W_new = W + dW;
* "Dynamic layer selection": after warmup, rank layers by reconstruction error
  epsilon and convert the lowest-error ones.

The closed form is the unique minimiser for lambda > 0, so the oracle is that
definition: accumulate G = A_loc^T A_loc and C = A_loc^T (A_full - A_loc)
(plus D = dA^T dA for epsilon) over the warmup rows, form R = C W and solve
(G + lambda I) dW = R with a float64 Cholesky factorisation (a library routine
used as one step).

Readings of points the pages leave open: the norm on matrices is Frobenius; A is
[tokens, d] and the projection is A @ W with W [d_in, d_out]; lambda is either
absolute or relative, lambda_rel * tr(G) / d; epsilon is the relative Frobenius
residual of the data term on the warmup rows; selection is a stable ascending
sort (ties -> lower layer index).
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np
import scipy.linalg

from .attention import branch_rows, softmax_attention


def gram_stats(chunks: Iterable[Tuple[np.ndarray, np.ndarray]]):
    """Sum over warmup chunks of G = A_loc^T A_loc, C = A_loc^T dA, D = dA^T dA (each [d, d]).

    ``chunks`` yields (A_loc [n, d], dA [n, d]) with dA = A_full - A_loc.
    """
    G = C = D = None
    for a_loc, da in chunks:
        a_loc = np.asarray(a_loc, dtype=np.float64)
        da = np.asarray(da, dtype=np.float64)
        g, c, dd = a_loc.T @ a_loc, a_loc.T @ da, da.T @ da
        if G is None:
            G, C, D = g, c, dd
        else:
            G, C, D = G + g, C + c, D + dd
    return G, C, D


def ridge_lambda(G: np.ndarray, lam: float, relative: bool) -> float:
    """lambda itself, or lambda * tr(G) / d for the relative rule."""
    if relative:
        return float(lam) * float(np.trace(G)) / G.shape[0]
    return float(lam)


def solve_delta_w(G: np.ndarray, C: np.ndarray, W: np.ndarray, lam: float) -> np.ndarray:
    """dW solving (G + lambda I) dW = C W, by float64 Cholesky (lower factor)."""
    d = G.shape[0]
    M = np.asarray(G, dtype=np.float64) + lam * np.eye(d)
    R = np.asarray(C, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    factor = scipy.linalg.cho_factor(M, lower=True, check_finite=True)
    return scipy.linalg.cho_solve(factor, R)


def normal_equation_residual(G, C, W, dW, lam) -> float:
    """||(G + lambda I) dW - C W||_F / ||C W||_F."""
    R = C @ W
    r = G @ dW + lam * dW - R
    return float(np.linalg.norm(r) / max(np.linalg.norm(R), 1e-300))


def recon_error_direct(a_loc, a_full, W, dW) -> float:
    """epsilon = ||A_loc (W + dW) - A_full W||_F / ||A_full W||_F over the stacked warmup rows."""
    ref = a_full @ W
    return float(np.linalg.norm(a_loc @ (W + dW) - ref) / np.linalg.norm(ref))


def recon_error_traces(G, C, D, W, dW, lam: Optional[float] = None) -> float:
    """The same epsilon from the statistics alone, valid for any dW.

    With E = A_loc dW - dA W:  ||E||^2 = <dW, G dW> - 2 <dW, C W> + <W, D W>,
    and ||A_full W||^2 = <W, (G + C + C^T + D) W> since A_full = A_loc + dA.
    ``lam`` is accepted for call symmetry and not used.
    """
    R = C @ W
    num2 = np.sum(dW * (G @ dW)) - 2.0 * np.sum(dW * R) + np.sum(W * (D @ W))
    den2 = np.sum(W * ((G + C + C.T + D) @ W))
    return float(np.sqrt(max(num2, 0.0) / den2))


def select_local_layers(eps, k: int) -> np.ndarray:
    """Indices of the k layers with the lowest epsilon (stable: ties keep the lower index).

    Technical summary section 2, "Dynamic layer selection": the layers are ranked by epsilon and the
    lowest-error ones converted.  A NaN epsilon (an undefined error: the layer's absorption failed)
    ranks last and is never converted, so fewer than k come back when fewer than k are numbers."""
    e = np.asarray(eps, dtype=np.float64)
    order = np.argsort(e, kind="stable")[:k]
    return np.sort(order[~np.isnan(e[order])])


def fold_weights(W, dW) -> np.ndarray:
    """W_new = W + dW for a layer that becomes a local-attention layer."""
    return np.asarray(W, dtype=np.float64) + np.asarray(dW, dtype=np.float64)


def local_layer_output(q, k, v, n_sink: int, n_cur: int, n_heads: int, W_new,
                       scale: Optional[float] = None, threads: int = 1) -> np.ndarray:
    """An L-layer step: attention over sink + current rows only, projected by W_new.

    The L-layer cache holds only [sink | current chunk] (its history was dropped).
    """
    rows = branch_rows(n_sink, 0, n_cur)["local"]
    a, _ = softmax_attention(q, k, v, rows, n_heads, scale, threads=threads)
    return a @ np.asarray(W_new, dtype=np.float64)
