"""Oracle: the W8A8 (8-bit weights and activations) variant of the L-layer projection.

TEST INFRASTRUCTURE ONLY -- never imported by the GPU library.

The ISPA pages pair the method with W8A8 post-training quantisation (technical
summary, section 4 "Results": ISPA combined with W8A8 gives the largest overall
speed-up) without saying which scheme.  The plainest reading, used here and on
the GPU, is symmetric absmax scaling per channel into the FP8 E4M3 format of the
OCP 8-bit floating point specification (1 sign, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, the all-ones code is NaN, largest finite value
448):

* weights: one scale per output channel j, s_w[j] = max_i |W[i, j]| / 448;
* activations: one scale per token i, s_a[i] = max_k |A[i, k]| / 448;
* a value x of a channel with scale s becomes the E4M3 code of x / s, rounded to
  nearest with ties to even (after clamping to [-448, 448]);
* the product is out[i, j] = s_a[i] s_w[j] sum_k dec(Aq[i, k]) dec(Wq[k, j]).

The scales and x / s are float32 operations (IEEE division), so every code is a
decision taken in float32 on both sides; a channel whose values are all zero
gets the scale 1.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes, from the format definition; the NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of float values with |x| <= 448, rounded to nearest, ties to even.

    Every finite E4M3 value is a multiple of 2^-9; the spacing in the binade of x is
    2^(e - 3) for normal values (e = floor(log2 |x|) >= -6) and 2^-9 below 2^-6, so x is
    rounded to that grid with ties to the even multiple, which is the code with the even
    mantissa (the code order follows the value order)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode takes finite values with |x| <= 448")
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    q = a / step                      # exact: step is a power of two
    n = np.floor(q)
    frac = q - n
    n = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(n, 2) == 1)), n + 1, n)
    v = n * step                      # the rounded magnitude (may reach the next binade)
    # code of v: exponent field and mantissa from the value itself
    ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    sub = v < 2.0 ** -6
    ef = np.where(sub, 0, ev + 7).astype(np.int64)
    mf = np.where(sub, np.round(v / 2.0 ** -9), np.round((v / np.exp2(ev) - 1.0) * 8.0)).astype(np.int64)
    code = (ef << 3) | mf
    code = np.where(v == 0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def round_bf16(x) -> np.ndarray:
    """float32 values rounded to bfloat16 (nearest, ties to even), as float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def quantize_rows(X) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row absmax E4M3 quantisation of a float32 matrix: (codes [r, c] uint8, scales [r] float32)."""
    X = np.asarray(X, dtype=np.float32)
    amax = np.max(np.abs(X), axis=1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (X / s[:, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(y), s


def quantize_weight(W) -> Tuple[np.ndarray, np.ndarray]:
    """W [d_in, d_out] -> (codes of W^T [d_out, d_in], per-output-channel scales [d_out])."""
    return quantize_rows(np.asarray(W, dtype=np.float32).T)


def w8a8_matmul(A, W) -> np.ndarray:
    """out = A W with A quantised per row and W per column as above; float64 sums of the decoded codes."""
    aq, sa = quantize_rows(A)
    wq, sw = quantize_weight(W)
    prod = e4m3_decode(aq) @ e4m3_decode(wq).T
    return prod * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]


def local_attention_fp8(q, k, v, n_sink: int, n_cur: int, n_heads: int, scale: Optional[float] = None,
                        quantize: bool = True) -> np.ndarray:
    """Attention of a converted layer with its operands in FP8 E4M3 (the W8A8 reading of the attention).

    The layer's key rows are its whole (local) cache: sink rows + current chunk.  Per head h:
      * Q per query token: s_q[i] = max_c |Q[i, c]| / 448, codes E4M3(Q / s_q);
      * K and V with one scale each over all key rows: s_k = max |K| / 448, s_v = max |V| / 448;
      * scores S = s_q s_k (dec(Qq) dec(Kq)^T), in log2 units x = S * scale * log2(e);
      * row reference M = ceil(max_j x) (an integer, so the largest probability is in (1/2, 1]);
        P = 2^(x - M) and its codes E4M3(256 P) (a fixed power-of-two scale: 256 P <= 256 < 448);
      * l = sum_j dec(Pq) / 256, O = s_v (dec(Pq) / 256) dec(Vq) / l.
    Scales and quotients are float32 operations, so every code is a float32 decision (as for the
    projection); S and the sums are exact (float64).  quantize=False skips every rounding (the codes
    become the values themselves), which is plain softmax attention over the same rows.
    """
    from .attention import branch_rows, default_scale
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    dh = d // n_heads
    scale = default_scale(dh) if scale is None else scale
    rows = branch_rows(n_sink, 0, n_cur)["local"]
    out = np.zeros((n_q, d))
    log2e = 1.0 / np.log(2.0)

    def codes(x, s):
        y = np.clip((np.asarray(x, dtype=np.float32) / np.float32(s)).astype(np.float32), -E4M3_MAX, E4M3_MAX)
        return e4m3_decode(e4m3_encode(y))

    def tensor_scale(x):
        a = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
        return np.float32(a / np.float32(E4M3_MAX)) if a > 0 else np.float32(1.0)

    for h in range(n_heads):
        c = slice(h * dh, (h + 1) * dh)
        qh, kh, vh = q[:, c], k[rows, c], v[rows, c]
        if quantize:
            amax = np.max(np.abs(qh.astype(np.float32)), axis=1)
            sq = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            sk, sv = tensor_scale(kh.astype(np.float32)), tensor_scale(vh.astype(np.float32))
            qd = np.stack([codes(qh[i], sq[i]) for i in range(n_q)]) if n_q else qh
            kd, vd = codes(kh, sk), codes(vh, sv)
            S = (qd @ kd.T) * sq.astype(np.float64)[:, None] * float(sk)
        else:
            S, vd, sv = qh @ kh.T, vh, 1.0
        x = S * scale * log2e
        M = np.ceil(np.max(x, axis=1, keepdims=True))
        P = np.exp2(x - M)
        if quantize:
            Pq = e4m3_decode(e4m3_encode((256.0 * P).astype(np.float32))) / 256.0
        else:
            Pq = P
        l = Pq.sum(axis=1, keepdims=True)
        out[:, c] = float(sv) * (Pq @ vd) / l
    return out


def local_layer_output_w8a8_fp8attn(q, k, v, n_sink: int, n_cur: int, n_heads: int, W,
                                    scale: Optional[float] = None) -> np.ndarray:
    """The converted layer in W8A8 end to end: FP8 attention (local_attention_fp8), its output stored in
    bfloat16, then the W8A8 projection by W."""
    a = local_attention_fp8(q, k, v, n_sink, n_cur, n_heads, scale)
    return w8a8_matmul(round_bf16(a.astype(np.float32)), W)


def local_layer_output_w8a8(q, k, v, n_sink: int, n_cur: int, n_heads: int, W,
                            scale: Optional[float] = None, threads: int = 1) -> np.ndarray:
    """An L-layer step with the W8A8 projection: local attention (float64), its output stored in
    bfloat16 (the io type of the call, rounded to nearest even), then w8a8_matmul with W."""
    from .attention import branch_rows, softmax_attention
    rows = branch_rows(n_sink, 0, n_cur)["local"]
    a, _ = softmax_attention(q, k, v, rows, n_heads, scale, threads=threads)
    return w8a8_matmul(round_bf16(a.astype(np.float32)), W)
