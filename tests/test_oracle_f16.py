"""Pins of the oracle's binary16 conversion (used for Delta, m and the INT8 scale).

The oracle converts binary32 -> binary16 with its own code (round to nearest,
ties to even).  It is checked against numpy's independent float16 cast:
  * every (sign, exponent) of binary32, every binary16-visible mantissa value,
    crossed with the low-bit patterns that decide the rounding (0, 1, just
    under / at / just over the half-way point, all ones, and random ones);
  * every one of the 65,536 bfloat16 bit patterns (the offsets m are fp16
    roundings of bf16 group minima);
  * a large random sample.
Decoding (binary16 -> binary64) is checked for all 65,536 patterns.
"""
import numpy as np

import oracle


def _compare(x32: np.ndarray):
    got = oracle.f32_to_f16_bits(x32)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x32.astype(np.float16).view(np.uint16)
    nan = np.isnan(x32)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN (payload is not part of the contract)
    g = got[nan]
    assert np.all(((g & 0x7C00) == 0x7C00) & ((g & 0x03FF) != 0))


def test_f16_structured_sweep():
    signexp = np.arange(512, dtype=np.uint32) << 23              # all signs and exponents
    hi10 = np.arange(1024, dtype=np.uint32) << 13                # every fp16-visible mantissa
    rng = np.random.default_rng(7)
    low = np.array([0, 1, 2, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0800, 0x17FF],
                   dtype=np.uint32)
    low = np.concatenate([low, rng.integers(0, 1 << 13, size=23, dtype=np.uint32)])
    # subnormal binary16 outputs depend on more low bits: add patterns around
    # every power-of-two split point of the 23-bit mantissa.
    extra = np.array([(1 << k) + o for k in range(23) for o in (-1, 0, 1) if (1 << k) + o >= 0],
                     dtype=np.uint32) & 0x1FFF
    low = np.unique(np.concatenate([low, extra]))
    bits = (signexp[:, None, None] | hi10[None, :, None] | low[None, None, :]).ravel()
    _compare(bits.view(np.float32))


def test_f16_subnormal_region_dense():
    # binary32 exponents that land in binary16's subnormal range or just above:
    # check every one of their mantissas on a stride that hits all residues mod 8.
    rng = np.random.default_rng(11)
    out = []
    for e in range(127 - 26, 127 - 13):
        m = np.arange(0, 1 << 23, 97, dtype=np.uint32)
        for s in (0, 1):
            out.append((np.uint32(s << 31) | np.uint32(e << 23) | m))
    bits = np.concatenate(out)
    bits = np.concatenate([bits, rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    _compare(bits.view(np.float32))


def test_f16_all_bf16_patterns():
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    _compare(b.view(np.float32))


def test_f16_random_sample():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
    _compare(bits.view(np.float32))


def test_f16_decode_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.f16_bits_to_f64(h)
    want = h.view(np.float16).astype(np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_f16_known_values():
    # textbook binary16 facts
    assert oracle.f32_to_f16_bits(np.float32(1.0)) == 0x3C00
    assert oracle.f32_to_f16_bits(np.float32(65504.0)) == 0x7BFF
    assert oracle.f32_to_f16_bits(np.float32(65519.99)) == 0x7BFF
    assert oracle.f32_to_f16_bits(np.float32(65520.0)) == 0x7C00
    assert oracle.f32_to_f16_bits(np.float32(2.0 ** -24)) == 0x0001
    assert oracle.f32_to_f16_bits(np.float32(2.0 ** -25)) == 0x0000      # tie -> even (0)
    assert oracle.f32_to_f16_bits(np.float32(3 * 2.0 ** -25)) == 0x0002  # tie -> even (2)
    assert oracle.f32_to_f16_bits(np.float32(1.0 + 2.0 ** -11)) == 0x3C00  # tie -> even
    assert oracle.f32_to_f16_bits(np.float32(1.0 + 3 * 2.0 ** -11)) == 0x3C02
    assert oracle.f32_to_f16_bits(np.float32(-0.0)) == 0x8000
