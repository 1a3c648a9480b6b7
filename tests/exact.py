"""Exact-rational helpers for the oracle pins (test code only).

Rounding to a binary floating-point format is done here by exact rational
arithmetic on the format's grid -- an independent route from the oracle's C
code (frexp/nearbyint) and from numpy's conversion routines.
"""
from fractions import Fraction
import math
import struct

import numpy as np

# (significand bits incl. the implicit one, minimum normal exponent, maximum exponent)
BINARY16 = (11, -14, 15)
BINARY32 = (24, -126, 127)


def floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) after at most one correction step either way
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_format(x: Fraction, fmt) -> Fraction:
    """Nearest value of the format to the exact rational x, ties to even.
    Returns +-inf (as float) on overflow."""
    p, emin, emax = fmt
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    N = a / quantum
    N0 = N.numerator // N.denominator
    rem = N - N0
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and N0 % 2 == 1):
        N0 += 1
    v = N0 * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if v > max_finite:
        return math.inf * sign
    return sign * v


def f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def f16_bits_value(bits: int) -> Fraction:
    """Exact value of a binary16 bit pattern (finite only)."""
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def nearest_code(x: Fraction, grid) -> int:
    """Index of the grid value nearest to x; at a tie the even index wins."""
    best, bestd = None, None
    for c, g in enumerate(grid):
        dd = abs(x - g)
        if bestd is None or dd < bestd or (dd == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, dd
    return best


def bf16_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0]
