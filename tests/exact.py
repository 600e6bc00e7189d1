"""Exact rational arithmetic used to pin the oracle (no numpy rounding involved).

IEEE binary32 / binary16 round-to-nearest-even are implemented here from their
definition on python Fractions, so a check written with them does not depend on
the same library conversions the oracle uses.
"""
from __future__ import annotations

import math
from fractions import Fraction


def _round_to_grid(mag: Fraction, ulp: Fraction) -> Fraction:
    q, r = divmod(mag, ulp)          # q integer, 0 <= r < ulp
    half = ulp / 2
    if r > half or (r == half and q % 2 == 1):
        q += 1
    return q * ulp


def _rn(x: Fraction, mant_bits: int, emin: int, emax: int) -> float:
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    mag = abs(x)
    e = math.floor(math.log2(mag.numerator) - math.log2(mag.denominator))
    # fix the floor(log2) estimate exactly
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    e = max(e, emin)                       # subnormals share the emin grid
    ulp = Fraction(2) ** (e - mant_bits)
    r = _round_to_grid(mag, ulp)
    max_finite = (2 - Fraction(2) ** -mant_bits) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * float(r)


def rn32(x: Fraction) -> float:
    """Nearest binary32 value (ties to even), returned as an exact python float."""
    return _rn(Fraction(x), 23, -126, 127)


def rn16(x: Fraction) -> float:
    """Nearest binary16 value (ties to even, subnormals kept)."""
    return _rn(Fraction(x), 10, -14, 15)


def round_half_away(x: Fraction) -> int:
    x = Fraction(x)
    s = -1 if x < 0 else 1
    return s * math.floor(abs(x) + Fraction(1, 2))


def q8_0_block_exact(xs):
    """Q8_0 of one 32-value block of f32 numbers, step by step on exact rationals.

    Returns (codes list[int], d16 float).
    """
    fx = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fx)
    d = Fraction(rn32(amax / 127))
    inv = Fraction(rn32(1 / d)) if d != 0 else Fraction(0)
    codes = [max(-127, min(127, round_half_away(Fraction(rn32(v * inv))))) for v in fx]
    return codes, rn16(d)
