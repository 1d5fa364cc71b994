"""The C-ABI library: it loads, exports every function include/ispa.h declares, and its host-side
validation rejects bad arguments before any GPU work (no GPU needed for these calls)."""
import ctypes
import os
import re

import pytest

import kv_cache_attention_ispa_amd as ispa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ispa.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s+(ispa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ispa.library_path()):
        pytest.fail("libispa.so is not built: run python -m kv_cache_attention_ispa_amd.build")
    return ispa.lib()


def test_header_declares_the_four_hot_path_calls():
    fns = declared_functions()
    for f in ("ispa_dual_attn", "ispa_gram_accum", "ispa_absorb_solve", "ispa_local_attn_fused_proj"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    for f in declared_functions():
        assert hasattr(L, f), f"libispa.so does not export {f}"


def test_status_strings_and_version(L):
    assert L.ispa_version() >= 100
    assert L.ispa_status_string(0) == b"ok"
    for s in (1, 2, 3, 4):
        assert L.ispa_status_string(s) not in (b"ok", b"unknown status")
    assert L.ispa_status_string(99) == b"unknown status"


def test_workspace_queries(L):
    s = ispa.AttnShape(4680, 1560, 14040, 4680, 12, 128, 0.0)
    assert ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, s) >= 20280 * 1536 * 2
    assert ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, s) >= 4680 * 1536 * 2
    assert ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, 1536) >= 6 * 1536 * 1536 * 4
    assert L.ispa_workspace_bytes(42, None, 0) == ctypes.c_size_t(-1).value


FAKE = 1 << 20  # a non-NULL, 16-byte aligned address; never dereferenced because validation fails first


def _dual(L, shape, io=1, stat=2, ld=None, q=FAKE, a_full=FAKE, a_loc=FAKE, lse=FAKE):
    ld = shape.n_q if ld is None else ld
    return L.ispa_dual_attn(ctypes.byref(shape), io, q, FAKE, FAKE, a_full, stat, a_loc, a_loc, ld, lse, lse,
                            None, 0, None)


@pytest.mark.parametrize("field,value,status", [
    ("n_q", 0, EINVAL), ("n_sink", -1, EINVAL), ("n_hist", -2, EINVAL), ("n_heads", 0, EINVAL),
    ("head_dim", 96, EUNSUPPORTED), ("head_dim", 256, EUNSUPPORTED)])
def test_dual_attn_rejects_bad_shapes(L, field, value, status):
    s = ispa.AttnShape(64, 8, 16, 64, 2, 128, 0.0)
    setattr(s, field, value)
    assert _dual(L, s) == status


def test_dual_attn_rejects_empty_local_set(L):
    assert _dual(L, ispa.AttnShape(64, 0, 100, 0, 2, 128, 0.0)) == EINVAL


def test_dual_attn_rejects_bad_arguments(L):
    s = ispa.AttnShape(64, 8, 16, 64, 2, 128, 0.0)
    assert _dual(L, s, io=1, stat=2) == EWORKSPACE        # bf16 inputs + fp16 statistics need the V copy
    assert _dual(L, s, q=0) == EINVAL                       # NULL q
    assert _dual(L, s, q=FAKE + 4) == EINVAL                # misaligned
    assert _dual(L, s, ld=60) == EINVAL                     # ld_stat < n_q
    assert _dual(L, s, ld=68) == EINVAL                     # ld_stat not a multiple of 8
    assert _dual(L, s, io=7) == EUNSUPPORTED                # unknown dtype
    assert _dual(L, s, io=0, stat=2) == EUNSUPPORTED        # fp32 inputs need fp32 statistics
    s64 = ispa.AttnShape(64, 8, 16, 64, 2, 64, 0.0)
    assert _dual(L, s64, io=1) == EUNSUPPORTED              # 16-bit path is head_dim 128
    # one head's rows of the V^T copy are addressed with 32-bit offsets: n_k < 8,388,544; K and V
    # themselves may pass 2^31 bytes (d = 5120 with 216,840 cached rows)
    big = ispa.AttnShape(64, 8, 8388544 - 8 - 64, 64, 2, 128, 0.0)
    assert _dual(L, big, io=1) == EWORKSPACE               # size accepted (workspace missing)
    big.n_hist += 1
    assert _dual(L, big, io=1) == EUNSUPPORTED
    long14b = ispa.AttnShape(64, 1560, 216840 - 1560 - 4680, 4680, 40, 128, 0.0)
    assert _dual(L, long14b, io=1) == EWORKSPACE
    # full-only mode needs a_full
    assert L.ispa_dual_attn(ctypes.byref(s), 1, FAKE, FAKE, FAKE, None, 2, None, None, 0, None, None, None, 0,
                            None) == EINVAL


def test_gram_rejects_bad_arguments(L):
    g = lambda d=256, n=100, st=2, ld=104, acc=0, G=FAKE: L.ispa_gram_accum(d, n, st, FAKE, FAKE, ld, acc, G, FAKE,
                                                                               None, None)
    assert g(d=100) == EINVAL
    assert g(d=0) == EINVAL
    assert g(n=0) == EINVAL
    assert g(ld=96) == EINVAL
    assert g(ld=105) == EINVAL
    assert g(st=9) == EUNSUPPORTED
    assert g(acc=2) == EINVAL
    assert g(G=0) == EINVAL


def test_solve_rejects_bad_arguments(L):
    def s(d=256, D=FAKE, eps=FAKE, info=FAKE, ws=FAKE, wsb=None, lam=1e-3, rel=1, wdt=1):
        wsb = ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, d) if wsb is None else wsb
        return L.ispa_absorb_solve(d, FAKE, FAKE, D, wdt, FAKE, lam, rel, 0, FAKE, None, eps, None, info, ws, wsb,
                                   None)
    assert s(d=250) == EINVAL
    assert s(info=0) == EINVAL
    assert s(D=0) == EINVAL                     # eps needs D
    assert s(lam=float("nan")) == EINVAL
    assert s(rel=3) == EINVAL
    assert s(wdt=5) == EUNSUPPORTED
    assert s(ws=0) == EWORKSPACE
    assert s(wsb=1000) == EWORKSPACE


def test_local_proj_rejects_bad_arguments(L):
    sh = ispa.AttnShape(64, 8, 0, 64, 2, 128, 0.0)
    need = ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, sh)
    f = lambda io=1, ws=FAKE, wsb=need, w=FAKE: L.ispa_local_attn_fused_proj(ctypes.byref(sh), io, FAKE, FAKE, FAKE,
                                                                             w, FAKE, ws, wsb, None)
    assert f(io=0) == EUNSUPPORTED
    assert f(w=0) == EINVAL
    assert f(ws=0) == EWORKSPACE
    assert f(wsb=need - 1) == EWORKSPACE
    # the same checks with W_new given transposed
    g = lambda io=1, ws=FAKE, wsb=need, w=FAKE: L.ispa_local_attn_fused_proj_wt(ctypes.byref(sh), io, FAKE, FAKE,
                                                                                FAKE, w, FAKE, ws, wsb, None)
    assert g(io=0) == EUNSUPPORTED
    assert g(w=0) == EINVAL
    assert g(w=FAKE + 8) == EINVAL            # 16-byte alignment
    assert g(ws=0) == EWORKSPACE
    assert g(wsb=need - 1) == EWORKSPACE


def test_transpose16_validation(L):
    t = lambda r=64, c=128, dt=1, src=FAKE, dst=FAKE + 4096: L.ispa_transpose16(r, c, dt, src, dst, None)
    assert t(dt=0) == EUNSUPPORTED                 # fp32 is not a 16-bit type
    assert t(dt=7) == EUNSUPPORTED
    for r, c in ((8, 128), (64, 120), (0, 64), (65552, 16), (64, -16)):
        assert t(r=r, c=c) == EINVAL, (r, c)
    assert t(src=0) == EINVAL
    assert t(dst=0) == EINVAL
    assert t(dst=FAKE) == EINVAL                   # in place
    assert t(src=FAKE + 2) == EINVAL               # alignment


def _dual_vt(L, shape, io=1, vt_dtype=2, vt=FAKE, ldv=None, a_loc=FAKE, ws=None, wsb=0):
    ldv = shape.n_sink + shape.n_hist + shape.n_cur if ldv is None else ldv
    return L.ispa_dual_attn_vt(ctypes.byref(shape), io, FAKE, FAKE, vt_dtype, vt, ldv, FAKE, 2, a_loc, a_loc,
                               shape.n_q, FAKE if a_loc else None, FAKE if a_loc else None, ws, wsb, None)


def test_dual_attn_vt_validation(L):
    s = ispa.AttnShape(64, 8, 16, 64, 2, 128, 0.0)
    need = ispa.workspace_bytes(ispa.CALL_DUAL_ATTN_VT, s)
    # only the parked local outputs: no room for a V^T copy
    assert 0 < need < ispa.workspace_bytes(ispa.CALL_DUAL_ATTN, s)
    assert need == 256 * 128 * 4 * 2                 # one 256-query block per head
    assert _dual_vt(L, s) == EWORKSPACE              # every other argument accepted
    assert _dual_vt(L, s, ws=FAKE, wsb=need - 16) == EWORKSPACE
    assert _dual_vt(L, s, vt=0) == EINVAL            # NULL V^T
    assert _dual_vt(L, s, vt=FAKE + 8) == EINVAL     # misaligned V^T
    assert _dual_vt(L, s, vt_dtype=1) == EINVAL      # the dual stream's PV product is fp16
    assert _dual_vt(L, s, ldv=87) == EINVAL          # ldv < n_k
    assert _dual_vt(L, s, ldv=92) == EINVAL          # ldv not a multiple of 8
    assert _dual_vt(L, s, ldv=96) == EWORKSPACE      # ldv > n_k is fine
    assert _dual_vt(L, s, ldv=8388600) == EWORKSPACE
    assert _dual_vt(L, s, ldv=8388608) == EUNSUPPORTED   # 128 rows of V^T reach 2^31 bytes
    assert _dual_vt(L, s, io=0, vt_dtype=0) == EUNSUPPORTED   # no fp32 variant
    # single stream: V^T in the input type (bf16 here); fp16 is rejected before any launch
    assert _dual_vt(L, s, vt_dtype=2, a_loc=0) == EINVAL
    s64 = ispa.AttnShape(64, 8, 16, 64, 2, 64, 0.0)
    assert _dual_vt(L, s64) == EUNSUPPORTED


def test_transpose_rows_validation(L):
    t = lambda rows=100, d=128, vd=1, v=FAKE, td=2, vt=FAKE + 65536, ldv=256, col0=8: L.ispa_transpose_rows(
        rows, d, vd, v, td, vt, ldv, col0, None)
    assert t(vd=0) == EUNSUPPORTED                  # fp32 rows
    assert t(vd=2, td=1) == EUNSUPPORTED            # fp16 -> bf16 is not offered
    for kw in (dict(d=96), dict(d=0), dict(rows=-1), dict(col0=4), dict(ldv=252), dict(col0=160),
               dict(v=0), dict(vt=0), dict(v=FAKE + 2), dict(col0=-8)):
        assert t(**kw) == EINVAL, kw


def test_kv_cache_rejects_bad_arguments_without_allocating(L):
    """ispa_kv_*: invalid sizes, dtypes and NULL handles fail on the host before any HIP call."""
    h = ctypes.c_void_p(FAKE)
    for args in ((0, 64, 1, 8, 16, 2), (2, 60, 1, 8, 16, 2), (2, 64, 7, 8, 16, 2), (2, 64, 1, -1, 16, 2),
                 (2, 64, 1, 8, 0, 2), (2, 64, 1, 8, 16, 0), (2, 64, 1, 8, 1 << 30, 4)):
        assert L.ispa_kv_create(*args, ctypes.byref(h)) == EINVAL, args
        assert h.value is None
    assert L.ispa_kv_create(2, 64, 1, 8, 16, 2, None) == EINVAL
    assert L.ispa_kv_destroy(None) == OK
    p, r = ctypes.c_void_p(), (ctypes.c_int32 * 3)()
    assert L.ispa_kv_layer(None, 0, ctypes.byref(p), ctypes.byref(p), r) == EINVAL
    held, res = ctypes.c_int64(), ctypes.c_int64()
    assert L.ispa_kv_bytes(None, ctypes.byref(held), ctypes.byref(res)) == EINVAL
    assert L.ispa_kv_append_chunk(None, 0, FAKE, FAKE, None) == EINVAL
    assert L.ispa_kv_write_sink(None, 0, FAKE, FAKE, None) == EINVAL
    assert L.ispa_kv_release_history(None, 0, None) == EINVAL


def test_w8a8_calls_reject_bad_arguments(L):
    """ispa_quantize_weight_fp8, ispa_quantize_rows_fp8 and ispa_local_attn_fused_proj_w8a8: sizes,
    strides, dtypes, NULL pointers and short workspaces fail on the host."""
    qw = lambda d_in=128, d_out=64, dt=1, w=FAKE, wq=FAKE, sc=FAKE: L.ispa_quantize_weight_fp8(d_in, d_out, dt, w, wq,
                                                                                                  sc, None)
    assert qw(d_in=96) == EINVAL                 # d_in % 64
    assert qw(d_out=66) == EINVAL                # d_out % 4
    assert qw(dt=7) == EINVAL
    assert qw(wq=0) == EINVAL
    assert qw(w=FAKE + 4) == EINVAL              # misaligned
    qr = lambda rows=4, cols=64, dt=1, ldx=64, ldq=64, q=FAKE: L.ispa_quantize_rows_fp8(rows, cols, dt, FAKE, ldx, q,
                                                                                       ldq, FAKE, None)
    assert qr(cols=60) == EINVAL                 # cols % 8
    assert qr(ldx=60) == EINVAL                  # ldx < cols
    assert qr(ldx=68) == EINVAL                  # ldx % 8 (16-byte row loads)
    assert qr(ldq=68) == EINVAL                  # ldq % 8
    assert qr(rows=0) == EINVAL
    assert qr(q=0) == EINVAL
    sh = ispa.AttnShape(64, 8, 0, 64, 2, 128, 0.0)
    need = ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ_W8A8, sh)
    f = lambda io=1, wq=FAKE, ws=FAKE, wsb=need: L.ispa_local_attn_fused_proj_w8a8(
        ctypes.byref(sh), io, FAKE, FAKE, FAKE, wq, FAKE, FAKE, ws, wsb, None)
    assert f(io=0) == EUNSUPPORTED               # fp32 io
    assert f(wq=0) == EINVAL
    assert f(ws=0) == EWORKSPACE
    assert f(wsb=need - 1) == EWORKSPACE


def test_select_layers_validation(L):
    f = lambda n=30, eps=FAKE, k=15, role=FAKE, order=None, info=None: L.ispa_select_layers(n, eps, info, k, role,
                                                                                          order, None)
    assert f(n=0) == EINVAL
    assert f(n=4097) == EINVAL
    assert f(k=-1) == EINVAL
    assert f(k=31) == EINVAL
    assert f(eps=None) == EINVAL
    assert f(role=None) == EINVAL
    assert f(eps=FAKE + 2) == EINVAL
    assert f(order=FAKE + 1) == EINVAL
    assert f(info=FAKE + 2) == EINVAL


def test_noalloc_validation(L):
    """The no-allocation L-layer step rejects what does not fit its fixed scratch, and bad arguments,
    before any device work."""
    assert L.ispa_noalloc_scratch_bytes() == 64 << 20
    big = ispa.AttnShape(4680, 1560, 0, 4680, 40, 128, 0.0)
    ok = ispa.AttnShape(4680, 1560, 0, 4680, 12, 128, 0.0)
    assert ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_PROJ, ok) <= L.ispa_noalloc_scratch_bytes()
    f = lambda s, io=1, q=FAKE, w=FAKE: L.ispa_local_attn_fused_proj_noalloc(ctypes.byref(s), io, q, FAKE, FAKE, w,
                                                                              FAKE, None)
    assert f(big) == EWORKSPACE
    assert f(ok, io=0) == EUNSUPPORTED
    assert f(ok, q=None) == EINVAL
    assert f(ok, w=FAKE + 8) == EINVAL


def test_batched_solve_validation(L):
    need = ispa.workspace_bytes(ispa.CALL_ABSORB_SOLVE, None, 256)

    def f(n=3, d=256, ws=FAKE, wsb=None, eps=FAKE, D=FAKE, refine=0):
        return L.ispa_absorb_solve_batched(n, d, FAKE, FAKE, D, 1, FAKE, 1e-3, 1, refine, FAKE, None, eps, None,
                                           FAKE, ws, 3 * need if wsb is None else wsb, None)
    assert f(n=0) == EINVAL
    assert f(d=100) == EINVAL
    assert f(eps=FAKE, D=None) == EINVAL
    assert f(refine=9) == EINVAL
    assert f(wsb=3 * need - 1) == EWORKSPACE
    assert f(ws=None) == EWORKSPACE


def test_fp8_attention_validation(L):
    s = ispa.AttnShape(300, 100, 0, 333, 2, 128, 0.0)
    need = ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_FP8, s)
    need2 = ispa.workspace_bytes(ispa.CALL_LOCAL_ATTN_FP8_PROJ_W8A8, s)
    assert 433 * 256 <= need < need2      # K codes, transposed V codes and scales; then the projection's
    f = lambda io=1, q=FAKE, ws=FAKE, wsb=need: L.ispa_local_attn_fp8(ctypes.byref(s), io, q, FAKE, FAKE, FAKE,
                                                                       ws, wsb, None)
    assert f(io=0) == EUNSUPPORTED
    assert f(q=None) == EINVAL
    assert f(q=FAKE + 8) == EINVAL
    assert f(ws=None) == EWORKSPACE
    assert f(wsb=need - 1) == EWORKSPACE
    g = lambda wq=FAKE, wsb=need2: L.ispa_local_attn_fp8_proj_w8a8(ctypes.byref(s), 1, FAKE, FAKE, FAKE, wq, FAKE,
                                                                   FAKE, FAKE, wsb, None)
    assert g(wq=None) == EINVAL
    assert g(wsb=need2 - 1) == EWORKSPACE
    s64 = ispa.AttnShape(300, 100, 0, 333, 2, 64, 0.0)
    assert L.ispa_local_attn_fp8(ctypes.byref(s64), 1, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == EUNSUPPORTED
