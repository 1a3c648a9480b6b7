"""Pins of the oracle's quantizers (KV4-RL, eq. 3.3 affine INT4; Appendix A.3
symmetric INT8 side entries).

Independent routes used here:
  * exact rational arithmetic (fractions.Fraction) for the nearest-code
    choice, by brute force over all 16 (INT4) or 255 (INT8) codes, ties to the
    even code;
  * exact rational rounding onto the binary32 / binary16 grids for Delta, m
    and the INT8 scale (tests/exact.py), not the oracle's conversion code;
  * closed forms: grid-exact groups round-trip with zero error, constructed
    ties land on the even code, constant groups give Delta = 0, power-of-two
    scalings scale Delta exactly;
  * the round-trip bounds |x - x^| <= Delta/2 (INT4, interior) and <= s/2
    (INT8, normal s).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact as X


def _bf16(a):
    from int8_mixed_precision_amd.workloads import to_bf16_values
    return to_bf16_values(np.asarray(a, dtype=np.float32))


def _groups(rng, G, count):
    """A mix of group value distributions (all bf16 values, |x| <= 65504)."""
    out = []
    for i in range(count):
        kind = i % 8
        if kind == 0:
            g = rng.standard_normal(G)
        elif kind == 1:
            g = rng.standard_normal(G) * 10.0 ** rng.integers(-6, 4)
        elif kind == 2:                       # one outlier
            g = rng.standard_normal(G); g[rng.integers(G)] *= 40
        elif kind == 3:                       # positive offset, narrow range
            g = 300 + rng.random(G)
        elif kind == 4:                       # tiny values near fp16 subnormals
            g = rng.standard_normal(G) * 1e-6
        elif kind == 5:                       # two values only
            g = rng.choice([-1.5, 2.25], size=G)
        elif kind == 6:                       # integers 0..15 shuffled (exact grid)
            g = rng.integers(0, 16, size=G).astype(np.float64)
        else:                                 # very small bf16 (f32 subnormal) mixed with normal
            g = rng.standard_normal(G); g[: G // 2] = 1e-39
        out.append(g)
    return _bf16(np.stack(out))


def _expected_int4_params(xg):
    """m and Delta per reading Q-1, computed with exact rational rounding."""
    lo, hi = Fraction(float(xg.min())), Fraction(float(xg.max()))
    m = X.round_to_format(lo, X.BINARY16)
    r = X.round_to_format(hi - m, X.BINARY32)
    if r <= 0:
        return m, Fraction(0)
    q = X.round_to_format(r / 15, X.BINARY32)
    return m, X.round_to_format(q, X.BINARY16)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_int4_params_and_codes_brute_force(G):
    rng = np.random.default_rng(100 + G)
    d = 128
    ngroups = 48 if G == 32 else 24
    x = _groups(rng, G, ngroups * (d // G)).reshape(-1, d)
    codes, delta, offs = oracle.quant_int4(x, G)
    for v in range(x.shape[0]):
        for g in range(d // G):
            xg = x[v, g * G:(g + 1) * G]
            m_bits, d_bits = int(offs[v, g]), int(delta[v, g])
            m, D = _expected_int4_params(xg)
            assert X.f16_bits_value(m_bits) == m
            assert X.f16_bits_value(d_bits) == D
            assert m_bits != 0x8000 and d_bits != 0x8000     # stored zeros are +0
            grid = [m + c * D for c in range(16)]
            for i in range(G):
                want = 0 if D == 0 else X.nearest_code(Fraction(float(xg[i])), grid)
                assert codes[v, g * G + i] == want, (v, g, i, float(xg[i]))


def test_int4_constructed_ties_and_closed_forms():
    # group spanning 0..15 exactly: m = 0, Delta = 1 (r = 15, 15/15 = 1)
    base = np.arange(16, dtype=np.float32)
    x = np.concatenate([base, np.array([2.5, 3.5, 4.5, 0.5, 14.5, 7.5, 8.5, 1.5,
                                        0.25, 0.75, 13.49, 9.0, 10.0, 11.0, 12.0, 5.5],
                                       dtype=np.float32)])
    x = _bf16(x)[None, :]
    codes, delta, offs = oracle.quant_int4(x, 32)
    assert offs[0, 0] == 0x0000 and delta[0, 0] == 0x3C00
    assert list(codes[0, :16]) == list(range(16))                 # grid-exact round trip
    # ties go to the even code: 2.5->2, 3.5->4, 4.5->4, 0.5->0, 14.5->14, 7.5->8,
    # 8.5->8, 1.5->2, 5.5->6
    assert list(codes[0, 16:24]) == [2, 4, 4, 0, 14, 8, 8, 2]
    assert codes[0, 31] == 6
    assert codes[0, 24] == 0 and codes[0, 25] == 1                 # 0.25 -> 0, 0.75 -> 1
    # bf16(13.49) = 13.5 -> tie -> 14
    assert codes[0, 26] == 14


def test_int4_negative_offset_and_power_of_two_scaling():
    # -8..7 : m = -8, r = 15, Delta = 1, codes = x + 8
    x = np.tile(np.arange(-8, 8, dtype=np.float32), 2)
    for e in (-10, -3, 0, 5, 10):
        xs = _bf16(x * np.float32(2.0 ** e))[None, :]
        codes, delta, offs = oracle.quant_int4(xs, 32)
        assert X.f16_bits_value(int(delta[0, 0])) == Fraction(2) ** e
        assert X.f16_bits_value(int(offs[0, 0])) == -8 * Fraction(2) ** e
        assert list(codes[0]) == list(np.tile(np.arange(16), 2))


def test_int4_constant_group():
    for val in (0.0, -0.0, 3.140625, -1e-30, 65280.0, -2.0 ** -20):
        x = _bf16(np.full((1, 32), val, dtype=np.float32))
        codes, delta, offs = oracle.quant_int4(x, 32)
        assert delta[0, 0] == 0
        assert np.all(codes == 0)
        m = X.round_to_format(Fraction(float(x[0, 0])), X.BINARY16)
        assert X.f16_bits_value(int(offs[0, 0])) == m
        assert offs[0, 0] != 0x8000


def test_int4_round_trip_bound():
    rng = np.random.default_rng(5)
    x = _groups(rng, 32, 4000).reshape(-1, 128)
    codes, delta, offs = oracle.quant_int4(x, 32)
    xh = oracle.dequant_int4(codes, delta, offs, 32)
    D = np.repeat(oracle.f16_bits_to_f64(delta), 32, axis=-1)
    M = np.repeat(oracle.f16_bits_to_f64(offs), 32, axis=-1)
    err = np.abs(x.astype(np.float64) - xh)
    q = (x.astype(np.float64) - M) / np.where(D > 0, D, 1)
    interior = (D > 0) & (q >= -0.5) & (q <= 15.5)
    assert np.all(err[interior] <= D[interior] / 2 * (1 + 1e-12))
    # clamped extremes: bounded by Delta/2 plus the fp16 rounding slack of m and Delta
    lo = x.reshape(-1, 4, 32).min(-1).repeat(32, -1).reshape(x.shape).astype(np.float64)
    hi = x.reshape(-1, 4, 32).max(-1).repeat(32, -1).reshape(x.shape).astype(np.float64)
    slack = D / 2 + np.abs(lo - M) + 15 * np.abs((hi - M) / 15 - D) + 1e-300
    ok = (D == 0) | (err <= slack * (1 + 1e-9))
    assert np.all(ok)
    # Delta is within the rounding of fp32 then fp16 of the exact (hi - m)/15
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.abs(D - (hi - M) / 15) / ((hi - M) / 15)
    sel = (D > 2.0 ** -14) & (hi > M)
    assert np.all(rel[sel] <= 2.0 ** -11 + 2.0 ** -23)


def test_int4_bits_per_element():
    # Appendix D.4: 4.25 bits per element at G=128, 5.00 at G=32, 6.00 at G=16
    x = _bf16(np.random.default_rng(0).standard_normal((2, 128)))
    for G, bits in ((128, 4.25), (32, 5.00), (16, 6.00)):
        codes, delta, offs = oracle.quant_int4(x, G)
        assert codes.max() <= 15
        per_elem = (4 * codes.shape[-1] + 16 * (delta.shape[-1] + offs.shape[-1])) / codes.shape[-1]
        assert per_elem == bits


def _expected_int8_scale(x):
    amax = Fraction(float(np.abs(x).max()))
    q = X.round_to_format(amax / 127, X.BINARY32)
    return X.round_to_format(q, X.BINARY16)


def test_int8_brute_force():
    rng = np.random.default_rng(9)
    x = _groups(rng, 128, 64)
    codes, scale = oracle.quant_int8(x)
    for v in range(x.shape[0]):
        s = _expected_int8_scale(x[v])
        assert X.f16_bits_value(int(scale[v])) == s
        assert scale[v] != 0x8000
        grid = [c * s for c in range(-127, 128)]
        for i in range(x.shape[1]):
            xv = Fraction(float(x[v, i]))
            if s == 0:
                want = 0
            else:
                # nearest of -127..127; index parity equals code parity (offset 127 is odd)
                idx = None
                bestd = None
                for c in range(-127, 128):
                    dd = abs(xv - c * s)
                    if bestd is None or dd < bestd or (dd == bestd and c % 2 == 0):
                        idx, bestd = c, dd
                want = idx
            assert codes[v, i] == want, (v, i, float(x[v, i]))


def test_int8_constructed_ties_and_bound():
    # amax = 127 -> s = 1 exactly; x = k + 1/2 must go to the even neighbour
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0] = 127.0
    halves = np.array([0.5, 1.5, 2.5, -2.5, -3.5, 100.5, 101.5, -126.5], dtype=np.float32)
    x[0, 1:1 + halves.size] = halves
    x = _bf16(x)
    codes, scale = oracle.quant_int8(x)
    assert scale[0] == 0x3C00
    assert codes[0, 0] == 127
    assert list(codes[0, 1:1 + halves.size]) == [0, 2, 2, -2, -4, 100, 102, -126]
    # round-trip bound whenever s is a normal binary16 value
    rng = np.random.default_rng(2)
    y = _groups(rng, 128, 3000)
    c, s = oracle.quant_int8(y)
    sv = oracle.f16_bits_to_f64(s)
    err = np.abs(y.astype(np.float64) - sv[:, None] * c)
    normal = sv >= 2.0 ** -14
    assert np.all(err[normal] <= sv[normal, None] / 2 * (1 + 1e-12))
    assert np.all(np.abs(c) <= 127)
    # all-zero vector -> s = +0, codes 0
    c0, s0 = oracle.quant_int8(np.zeros((1, 128), np.float32))
    assert s0[0] == 0 and np.all(c0 == 0)
