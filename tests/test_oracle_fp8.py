"""Pins for oracle/fp8.py (the W8A8 reading) against things other than itself: the E4M3 values the
OCP 8-bit floating point specification fixes, an exhaustive nearest-value search, PyTorch's own
float8_e4m3fn conversion, and products that must come out exact."""
import numpy as np
import pytest

from oracle import fp8


def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def test_decode_fixed_points_of_the_format():
    # largest finite 448 = 1.75 * 2^8, smallest normal 2^-6, smallest subnormal 2^-9, 1.0 at exponent 7
    assert fp8.e4m3_decode([0x7E, 0x08, 0x01, 0x38, 0x00])[:5].tolist() == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, 0.0]
    assert np.isnan(fp8.e4m3_decode([0x7F, 0xFF])).all()
    assert fp8.e4m3_decode([0xB8])[0] == -1.0


def test_encode_decode_round_trip_on_every_finite_code():
    c = _finite_codes()
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(c)), c)


def test_encode_known_roundings():
    # ties go to the even mantissa: 1.0625 lies between 1.0 (m=0) and 1.125 (m=1), 1.1875 between
    # 1.125 (m=1) and 1.25 (m=2); 0.1 = 1.6 * 2^-4 -> mantissa 4.8 -> 5; 2^-10 is half the smallest
    # subnormal (tie to the even code 0)
    x = [448.0, 1.0625, 1.1875, float(np.float32(0.1)), 240.0, 2.0 ** -10, 3 * 2.0 ** -10, -1.0625]
    assert fp8.e4m3_encode(x).tolist() == [0x7E, 0x38, 0x3A, 0x1D, 0x77, 0x00, 0x02, 0xB8]


def test_encode_matches_exhaustive_nearest_search():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 2000), rng.standard_normal(2000), rng.uniform(-0.02, 0.02, 2000)])
    codes = _finite_codes()
    vals = fp8.e4m3_decode(codes)
    got = fp8.e4m3_encode(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = codes[d == d.min()]
        best = best[(best & 0x80) == (0x80 if np.signbit(xi) else 0)] if len(best) > 1 else best
        if len(best) > 1:                       # a tie: the even mantissa
            best = best[(best & 1) == 0]
        assert gi == best[0], (xi, gi, best)


def test_encode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("this PyTorch has no float8_e4m3fn")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 5000), rng.standard_normal(5000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_quantize_rows_scale_and_error_bound():
    rng = np.random.default_rng(2)
    X = (rng.standard_normal((40, 300)) * rng.uniform(0.01, 10, (40, 1))).astype(np.float32)
    X[3] = 0.0
    codes, s = fp8.quantize_rows(X)
    assert s[3] == 1.0 and not codes[3].any()
    mags = codes & 0x7F
    assert np.all(mags[np.arange(40) != 3].max(axis=1) == 0x7E)      # each row's absmax maps to 448
    back = fp8.e4m3_decode(codes) * s[:, None]
    # half a unit in the last place: 2^-4 relative for normal codes, 2^-10 * s below 2^-6 * s
    err = np.abs(back - X)
    bound = np.maximum(np.abs(X) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_w8a8_product_is_exact_on_representable_inputs():
    """Rows of A and columns of W that are already E4M3 values with absmax 448 get scale 1 and exact
    codes, so the W8A8 product equals the float64 product exactly."""
    rng = np.random.default_rng(3)
    vals = fp8.e4m3_decode(_finite_codes())
    A = rng.choice(vals, (16, 64))
    W = rng.choice(vals, (64, 24))
    A[:, 0] = 448.0
    W[0, :] = -448.0
    assert np.array_equal(fp8.w8a8_matmul(A, W), A @ W)


def test_w8a8_product_error_is_quantisation_sized():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((64, 512)).astype(np.float32)
    W = (rng.standard_normal((512, 96)) / np.sqrt(512)).astype(np.float32)
    ref = A.astype(np.float64) @ W
    got = fp8.w8a8_matmul(A, W)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.06


def test_round_bf16():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1 (even); 1 + 3*2^-8 ties to 1 + 2^-6 (even);
    # just above the tie rounds up
    assert fp8.round_bf16(x).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -3.0, 1.0 + 2.0 ** -7]
