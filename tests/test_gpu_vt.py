"""GPU: attention over a V^T the caller keeps (ispa_transpose_rows + ispa_dual_attn_vt).

* ispa_transpose_rows against a host transpose, exactly (bf16 -> fp16 is exact for the magnitudes
  used here), with the zero columns it leaves after its rows and the columns it must not touch
  (the buffer starts as NaN).
* ispa_dual_attn_vt runs the kernel of ispa_dual_attn on the same values, so every output must be
  bit-identical to ispa_dual_attn's (whose oracle parity the other attention tests check).  The
  V^T is built by three appends (sink, history, current chunk) into a NaN-filled buffer, so the
  finite columns past n_k that the call requires come only from the appends' zero tails.
* One shape of the V^T path against the oracle directly, and the 1.3B-shaped layer bit-identical
  to ispa_dual_attn.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import dev, host, maxrel, torch, tdtype

pytestmark = pytest.mark.gpu


def _away_from_zero(x):
    """Values below 2^-14 in magnitude are moved to 0.5 so that bf16 -> fp16 is exact."""
    x = np.array(x, dtype=np.float64)
    x[np.abs(x) < 2.0 ** -14] = 0.5
    return x


@pytest.mark.parametrize("vd,td", [("bf16", "f16"), ("bf16", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("rows,col0,ldv", [(100, 8, 256), (200, 40, 248), (64, 0, 64), (1, 16, 24), (0, 8, 200),
                                           (1560, 1560, 4096)])
def test_transpose_rows_exact(vd, td, rows, col0, ldv):
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    d = 192
    rng = np.random.default_rng(rows + col0)
    v = wl.round_to(_away_from_zero(rng.standard_normal((rows, d))), vd)
    vt = t.full((d, ldv), float("nan"), dtype=tdtype(td), device="cuda")
    ispa.transpose_rows(dev(v, vd).reshape(rows, d), vt, col0)
    t.cuda.synchronize()
    got = host(vt)
    assert np.array_equal(got[:, col0:col0 + rows], v.T.astype(np.float64))
    # zeros after the rows: to the end of the 64-column block the rows end in, plus one more block
    z_end = min(ldv, col0 + (rows + 63) // 64 * 64 + 64)
    assert np.all(got[:, col0 + rows:z_end] == 0.0)
    assert np.all(np.isnan(got[:, z_end:])) and np.all(np.isnan(got[:, :col0]))


VT_SHAPES = [
    wl.AttnShape(200, 72, 152, 100, 2, 128),    # ragged tiles in every segment, 2 query blocks
    wl.AttnShape(77, 40, 0, 50, 3, 128),        # empty history
    wl.AttnShape(65, 0, 136, 65, 1, 128),       # no sink
    wl.AttnShape(40, 64, 96, 0, 1, 128),        # local set = sink only (the last append writes no rows)
    wl.AttnShape(300, 8, 1000, 7, 2, 128),      # long history, tiny local set
]


def _vt_of(shape, v, vt_dtype, ldv):
    """V^T built the way a cache keeps it: sink, history and current rows appended one call each."""
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    vt = t.full((shape.d, ldv), float("nan"), dtype=vt_dtype, device="cuda")
    r0 = 0
    for n in (shape.n_sink, shape.n_hist, shape.n_cur):
        ispa.transpose_rows(v[r0:r0 + n], vt, r0)
        r0 += n
    return vt


def _outputs(shape, io, stat, mode):
    t = torch()
    d = shape.d
    ld = (shape.n_q + 5 + 7) // 8 * 8
    nan = float("nan")
    o = {"a_full": t.full((shape.n_q, d), nan, dtype=tdtype(io), device="cuda")}
    if mode in ("stats", "lse"):
        o["lse_loc"] = t.full((shape.n_heads, shape.n_q), nan, device="cuda")
        o["lse_hist"] = t.full((shape.n_heads, shape.n_q), nan, device="cuda")
    if mode == "stats":
        o["a_loc_t"] = t.full((d, ld), nan, dtype=tdtype(stat), device="cuda")
        o["delta_a_t"] = t.full((d, ld), nan, dtype=tdtype(stat), device="cuda")
    return o


def _bits(x):
    t = torch()
    return x.view(t.int16) if x.element_size() == 2 else x.view(t.int32)


def _run_both(shape, q, k, v, io, stat, mode, ldv_extra):
    import kv_cache_attention_ispa_amd as ispa
    t = torch()
    s = ispa.AttnShape.of(shape)
    qd, kd, vd = dev(q, io), dev(k, io), dev(v, io)
    dual = mode != "single"
    vt_dtype = t.float16 if dual else tdtype(io)
    ldv = (shape.n_k + 7) // 8 * 8 + ldv_extra
    vt = _vt_of(shape, vd, vt_dtype, ldv)
    ref, got = _outputs(shape, io, stat, mode), _outputs(shape, io, stat, mode)
    ws = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, s), dtype=t.uint8, device="cuda")
    ispa.dual_attn(s, qd, kd, vd, workspace=ws, **ref)
    ws_vt = t.empty(ispa.workspace_bytes(ispa.CALL_DUAL_ATTN_VT, s), dtype=t.uint8, device="cuda") if dual else None
    ispa.dual_attn_vt(s, qd, kd, vt, workspace=ws_vt, **got)
    t.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("mode,io,stat", [("stats", "bf16", "f16"), ("stats", "bf16", "f32"), ("stats", "f16", "bf16"),
                                          ("lse", "bf16", "f16"), ("single", "bf16", "f16"),
                                          ("single", "f16", "f16")])
@pytest.mark.parametrize("si", range(len(VT_SHAPES)))
def test_dual_attn_vt_bit_identical(si, mode, io, stat):
    shape = VT_SHAPES[si]
    rng = np.random.default_rng(100 + si)
    q = wl.round_to(rng.standard_normal((shape.n_q, shape.d)), io)
    k = wl.round_to(rng.standard_normal((shape.n_k, shape.d)), io)
    v = wl.round_to(_away_from_zero(rng.standard_normal((shape.n_k, shape.d))), io)
    # V^T exactly as long as the rows (tails clipped, reads past it wrap) or with room to spare
    for extra in (0, 72):
        ref, got = _run_both(shape, q, k, v, io, stat, mode, extra)
        for name in ref:
            assert torch().equal(_bits(ref[name]), _bits(got[name])), (name, shape, extra)


def test_dual_attn_vt_against_oracle():
    shape = VT_SHAPES[0]
    rng = np.random.default_rng(7)
    q = wl.round_to(rng.standard_normal((shape.n_q, shape.d)), "bf16")
    k = wl.round_to(rng.standard_normal((shape.n_k, shape.d)), "bf16")
    v = wl.round_to(_away_from_zero(rng.standard_normal((shape.n_k, shape.d))), "bf16")
    _, got = _run_both(shape, q, k, v, "bf16", "f16", "stats", 16)
    ref = oracle.dual_stream(q, k, v, shape.n_sink, shape.n_hist, shape.n_cur, shape.n_heads)
    n = shape.n_q
    assert maxrel(host(got["a_full"]), ref["a_full"]) <= 2e-2
    assert maxrel(host(got["a_loc_t"])[:, :n].T, ref["a_loc"]) <= 2e-2
    assert maxrel(host(got["delta_a_t"])[:, :n].T, ref["delta_a"]) <= 2e-2
    assert maxrel(host(got["lse_loc"]), ref["lse_loc"]) <= 2e-2
    assert maxrel(host(got["lse_hist"]), ref["lse_hist"]) <= 2e-2


def test_dual_attn_vt_1p3b_bit_identical():
    """The bench's layer (4680 queries, 1560 sink, 14040 history, 4680 current rows, 12 heads): the
    V^T path gives ispa_dual_attn's outputs bit for bit."""
    w = wl.LAYER_1P3B
    shape = w.shape
    x = wl.layer_inputs(w)
    ref, got = _run_both(shape, x["q"], x["k"], x["v"], "bf16", "f16", "stats", 0)
    for name in ref:
        assert torch().equal(_bits(ref[name]), _bits(got[name])), name
