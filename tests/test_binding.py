"""The Python binding rejects mismatched tensors before anything reaches the C ABI (no GPU needed:
every check here fails on dtype, shape or layout, or on the device check that runs last)."""
import pytest

torch = pytest.importorskip("torch")
import kv_cache_attention_ispa_amd as ispa  # noqa: E402

H, DH, NQ, NS, NH, NC = 2, 128, 40, 16, 24, 40
D, NK = H * DH, NS + NH + NC


def _shape():
    return ispa.AttnShape(NQ, NS, NH, NC, H, DH, 0.0)


def _attn(**over):
    a = dict(q=torch.zeros(NQ, D, dtype=torch.bfloat16), k=torch.zeros(NK, D, dtype=torch.bfloat16),
             v=torch.zeros(NK, D, dtype=torch.bfloat16), a_full=torch.zeros(NQ, D, dtype=torch.bfloat16),
             a_loc_t=torch.zeros(D, 48, dtype=torch.float16), delta_a_t=torch.zeros(D, 48, dtype=torch.float16),
             lse_loc=torch.zeros(H, NQ), lse_hist=torch.zeros(H, NQ), workspace=torch.zeros(16, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(k=torch.zeros(NK, D, dtype=torch.float16)), "k must have dtype"),
    (dict(v=torch.zeros(NK - 1, D, dtype=torch.bfloat16)), "v must have shape"),
    (dict(q=torch.zeros(NQ, D, dtype=torch.float64)), "q must have dtype"),
    (dict(a_full=torch.zeros(NQ, D, dtype=torch.float32)), "a_full must have dtype"),
    (dict(a_loc_t=torch.zeros(D, 48, dtype=torch.float32)), "share a dtype"),
    (dict(delta_a_t=torch.zeros(D, 32, dtype=torch.float16)), "delta_a_t must be a"),
    (dict(a_loc_t=torch.zeros(D, 56, dtype=torch.float16)), "same leading dimension"),
    (dict(lse_hist=torch.zeros(H, NQ, dtype=torch.float16)), "lse_hist must have dtype"),
    (dict(lse_loc=torch.zeros(H + 1, NQ)), "lse_loc must have shape"),
    (dict(q=torch.zeros(D, NQ, dtype=torch.bfloat16).t()), "q must be contiguous"),
    ({}, "on the GPU"),
])
def test_dual_attn_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        ispa.dual_attn(_shape(), **_attn(**over))


def test_dual_attn_rejects_ld_stat_mismatch():
    with pytest.raises(ValueError, match="ld_stat"):
        ispa.dual_attn(_shape(), ld_stat=56, **_attn())


def _gram(**over):
    a = dict(a_loc_t=torch.zeros(D, 48, dtype=torch.float16), delta_a_t=torch.zeros(D, 48, dtype=torch.float16),
             n=40, G=torch.zeros(D, D), C=torch.zeros(D, D), D=torch.zeros(D, D))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(G=torch.zeros(D, D, dtype=torch.bfloat16)), "G must have dtype"),
    (dict(C=torch.zeros(D, D - 32)), "C must have shape"),
    (dict(D=torch.zeros(D, D, dtype=torch.float64)), "D must have dtype"),
    (dict(delta_a_t=torch.zeros(D, 48, dtype=torch.bfloat16)), "share a dtype"),
    (dict(n=49), "a_loc_t must be a"),
    (dict(a_loc_t=torch.zeros(D - 32, 48, dtype=torch.float16)), "a_loc_t must be a"),
    ({}, "on the GPU"),
])
def test_gram_accum_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        ispa.gram_accum(**_gram(**over))


def _solve(**over):
    a = dict(G=torch.zeros(D, D), C=torch.zeros(D, D), W=torch.zeros(D, D, dtype=torch.bfloat16), lam=1e-3,
             relative=True, delta_w=torch.zeros(D, D), info=torch.zeros(1, dtype=torch.int32),
             workspace=torch.zeros(16, dtype=torch.uint8), D=torch.zeros(D, D),
             w_new=torch.zeros(D, D, dtype=torch.bfloat16), eps=torch.zeros(1), lambda_out=torch.zeros(1))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(delta_w=torch.zeros(D, D, dtype=torch.bfloat16)), "delta_w must have dtype"),
    (dict(w_new=torch.zeros(D, D, dtype=torch.float32)), "w_new must have dtype"),
    (dict(info=torch.zeros(1, dtype=torch.int64)), "info must have dtype"),
    (dict(eps=torch.zeros(1, dtype=torch.float64)), "eps must have dtype"),
    (dict(lambda_out=torch.zeros(0)), "lambda_out needs at least 1"),
    (dict(W=torch.zeros(D, D + 8, dtype=torch.bfloat16)), "W must have shape"),
    (dict(workspace=torch.zeros(4, dtype=torch.float32)), "on the GPU|workspace must be"),
    ({}, "on the GPU"),
])
def test_absorb_solve_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        ispa.absorb_solve(**_solve(**over))


def test_local_layer_rejects():
    s = ispa.AttnShape(NQ, NS, 0, NC, H, DH, 0.0)
    q = torch.zeros(NQ, D, dtype=torch.bfloat16)
    kv = torch.zeros(NS + NC, D, dtype=torch.bfloat16)
    w = torch.zeros(D, D, dtype=torch.bfloat16)
    out = torch.zeros(NQ, D, dtype=torch.bfloat16)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="w_new must have dtype"):
        ispa.local_attn_fused_proj(s, q, kv, kv, w.half(), out, ws)
    with pytest.raises(ValueError, match="q must have dtype"):
        ispa.local_attn_fused_proj(s, q.float(), kv.float(), kv.float(), w.float(), out.float(), ws)
    with pytest.raises(ValueError, match="out must have shape"):
        ispa.local_attn_fused_proj(s, q, kv, kv, w, out[:-1], ws)
    with pytest.raises(ValueError, match="wq_t must have dtype"):
        ispa.local_attn_fused_proj_w8a8(s, q, kv, kv, w, torch.zeros(D), out, ws)
    with pytest.raises(ValueError, match="w_scales must have shape"):
        ispa.local_attn_fused_proj_w8a8(s, q, kv, kv, w.view(torch.uint8)[:, :D].contiguous(), torch.zeros(D + 1),
                                        out, ws)
    with pytest.raises(ValueError, match="on the GPU"):
        ispa.local_attn_fused_proj(s, q, kv, kv, w, out, ws)


def test_fp8_quantisers_reject():
    w = torch.zeros(128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="wq_t must have shape"):
        ispa.quantize_weight_fp8(w, torch.zeros(128, 64, dtype=torch.uint8), torch.zeros(64))
    with pytest.raises(ValueError, match="w_scales must have dtype"):
        ispa.quantize_weight_fp8(w, torch.zeros(64, 128, dtype=torch.uint8), torch.zeros(64, dtype=torch.float16))
    x = torch.zeros(10, 64)
    with pytest.raises(ValueError, match="q must have shape"):
        ispa.quantize_rows_fp8(x, torch.zeros(10, 32, dtype=torch.uint8), torch.zeros(10))
    with pytest.raises(ValueError, match="scales must have shape"):
        ispa.quantize_rows_fp8(x, torch.zeros(10, 64, dtype=torch.uint8), torch.zeros(9))
