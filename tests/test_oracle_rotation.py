"""Pins of the oracle's key/query rotation (KV4-RL Section 5.1 and Appendix A.3
"Encoding and allocation": a fixed normalized Hadamard transform of keys after
RoPE and of queries before attention, values unrotated; eq. 3.4: with HH^T = I
the unquantized scores are unchanged).

Independent routes used here:
  * the Sylvester matrix built by Kronecker products in numpy (no butterflies):
    the transform of each unit vector is that matrix's row times the scale,
    which pins the ordering and every sign;
  * integer inputs, where every butterfly sum is exact in binary32, against the
    exact integer product x H;
  * the scale against exact decimal arithmetic (nearest binary32 to 1/sqrt(d));
  * the binary32 error bound of the butterfly stages against x H / sqrt(d) in
    binary64, orthogonality (applying the transform twice gives x back), and
    score invariance (q H)(k H)^T = q k^T;
  * the quantizers on rotated (non-bf16) inputs, brute force with exact
    rational arithmetic, and the rotated cache equals the quantizers applied to
    the rotated keys with values untouched.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact as X


def _sylvester(d):
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def _bf16(a):
    from int8_mixed_precision_amd.workloads import to_bf16_values
    return to_bf16_values(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("d", [2, 8, 128, 256])
def test_unit_vectors_give_sylvester_rows(d):
    H = _sylvester(d)
    s = np.float32(oracle.wht_scale(d))
    y = oracle.wht(np.eye(d, dtype=np.float32))
    want = (H.astype(np.float32) * s).astype(np.float32)
    assert np.array_equal(y, want)


def test_scale_is_nearest_binary32():
    getcontext().prec = 60
    for d in (2, 8, 32, 128, 512):
        exact = Decimal(1) / Decimal(d).sqrt()
        s = oracle.wht_scale(d)
        assert X.round_to_format(Fraction(str(exact)), X.BINARY32) == Fraction(s)
    assert np.float32(oracle.wht_scale(128)).view(np.uint32) == 0x3DB504F3


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(31)
    d = 128
    H = _sylvester(d)
    x = rng.integers(-200, 201, size=(64, d)).astype(np.float32)
    z = (x.astype(np.float64) @ H).astype(np.float32)       # exact integers, |z| < 2^24
    want = z * np.float32(oracle.wht_scale(d))
    assert np.array_equal(oracle.wht(x), want)


def test_error_bound_orthogonality_and_scores():
    rng = np.random.default_rng(32)
    d = 128
    H = _sylvester(d) / np.sqrt(d)
    x = _bf16(rng.standard_normal((256, d)) * np.where(rng.random((256, d)) < 0.03, 30.0, 1.0))
    y = oracle.wht(x).astype(np.float64)
    ref = x.astype(np.float64) @ H
    u = 2.0 ** -24
    # seven stages of one rounding each on partial sums bounded by sum |x|, then the scale
    bound = (np.log2(d) + 2) * u * np.abs(x).astype(np.float64).sum(1, keepdims=True) / np.sqrt(d) * 2
    assert np.all(np.abs(y - ref) <= bound)
    # H H^T = I: twice the transform is the identity up to the same bound, twice
    xx = oracle.wht(oracle.wht(x)).astype(np.float64)
    assert np.all(np.abs(xx - x) <= 3 * bound)
    assert np.allclose(H @ H.T, np.eye(d), atol=1e-15)
    # (qH)(kH)^T = qk^T, exactly in binary64 and within the binary32 bound
    q = _bf16(rng.standard_normal((8, d)))
    s_ref = q.astype(np.float64) @ x.astype(np.float64).T
    s64 = (q.astype(np.float64) @ H) @ (x.astype(np.float64) @ H).T
    assert np.allclose(s64, s_ref, rtol=0, atol=1e-10)
    s32 = oracle.wht(q).astype(np.float64) @ y.T
    tol = 4 * (np.log2(d) + 2) * u * np.abs(q).sum(1)[:, None] * np.abs(x).sum(1)[None, :]
    assert np.all(np.abs(s32 - s_ref) <= tol)


def test_quantizers_on_rotated_inputs_brute_force():
    rng = np.random.default_rng(33)
    d, G = 128, 32
    x = oracle.wht(_bf16(rng.standard_normal((12, d)) * 3))
    assert not np.array_equal(x, _bf16(x))                   # genuinely not bf16 values
    codes, delta, offs = oracle.quant_int4(x, G)
    for v in range(x.shape[0]):
        for g in range(d // G):
            xg = x[v, g * G:(g + 1) * G]
            m = X.round_to_format(Fraction(float(xg.min())), X.BINARY16)
            r = X.round_to_format(Fraction(float(xg.max())) - m, X.BINARY32)
            D = X.round_to_format(X.round_to_format(r / 15, X.BINARY32), X.BINARY16) if r > 0 else 0
            assert X.f16_bits_value(int(offs[v, g])) == m
            assert X.f16_bits_value(int(delta[v, g])) == D
            grid = [m + c * D for c in range(16)]
            for i in range(G):
                want = 0 if D == 0 else X.nearest_code(Fraction(float(xg[i])), grid)
                assert codes[v, g * G + i] == want
    c8, s8 = oracle.quant_int8(x)
    for v in range(x.shape[0]):
        s = X.round_to_format(X.round_to_format(Fraction(float(np.abs(x[v]).max())) / 127, X.BINARY32),
                              X.BINARY16)
        assert X.f16_bits_value(int(s8[v])) == s
        for i in range(0, d, 7):
            xv = Fraction(float(x[v, i]))
            best = min(range(-127, 128), key=lambda c: (abs(xv - c * s), c % 2))
            assert c8[v, i] == best


def test_rotated_cache_rotates_keys_only():
    rng = np.random.default_rng(34)
    k = [_bf16(rng.standard_normal((n, 2, 128))) for n in (5, 40)]
    v = [_bf16(rng.standard_normal((n, 2, 128))) for n in (5, 40)]
    plain = oracle.MixedCache(k, v, 32)
    rot = oracle.MixedCache(k, v, 32, rotate=True)
    K = np.concatenate(k, 0)
    c, dd, mm = oracle.quant_int4(oracle.wht(K), 32)
    assert np.array_equal(rot.k4, c) and np.array_equal(rot.k4d, dd) and np.array_equal(rot.k4m, mm)
    c8, s8 = oracle.quant_int8(oracle.wht(K))
    assert np.array_equal(rot.k8, c8) and np.array_equal(rot.k8s, s8)
    for name in ("v4", "v4d", "v4m", "v8", "v8s"):
        assert np.array_equal(getattr(rot, name), getattr(plain, name))
    assert not np.array_equal(rot.k4, plain.k4)


def test_rotation_spreads_outlier_channels():
    """What the rotation is for (KV4-RL Section 5.1): with a few outlier key
    channels, INT4 keys stored in the rotated basis give smaller score errors
    (q H) . k^_rot - q . k than keys stored as they are."""
    rng = np.random.default_rng(35)
    n, d = 512, 128
    k = rng.standard_normal((n, 1, d))
    k[:, :, [3, 40, 77, 110]] *= 10.0
    k = _bf16(k)
    q = _bf16(rng.standard_normal((16, d)))
    exact = q.astype(np.float64) @ k[:, 0].astype(np.float64).T
    plain = oracle.MixedCache([k], [k], 32)
    rot = oracle.MixedCache([k], [k], 32, rotate=True)
    kp = oracle.dequant_int4(plain.k4, plain.k4d, plain.k4m, 32)[:, 0]
    kr = oracle.dequant_int4(rot.k4, rot.k4d, rot.k4m, 32)[:, 0]
    err_plain = np.abs(q.astype(np.float64) @ kp.T - exact).mean()
    err_rot = np.abs(oracle.wht(q).astype(np.float64) @ kr.T - exact).mean()
    assert err_rot < 0.8 * err_plain, (err_rot, err_plain)      # 0.67 at this seed
