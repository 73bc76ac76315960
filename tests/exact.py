"""Exact rational helpers for pinning the oracle (no dependence on the oracle).

round_f32 rounds an exact rational to the nearest IEEE binary32 value, ties to
even, with subnormals, by integer arithmetic only, so a pin built on it does
not inherit any rounding of the code it checks.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def frac(x) -> Fraction:
    """Exact value of a finite float / numpy float."""
    return Fraction(float(x))


def round_f32(q: Fraction) -> np.float32:
    """Nearest binary32 to the rational q (ties to even)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    # spacing of binary32 numbers around a: 2^(e-23) for normals, 2^-149 below 2^-126
    q_exp = max(e, -126) - 23
    scaled = a / (Fraction(2) ** q_exp)          # want the nearest integer, ties to even
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * Fraction(2) ** q_exp
    if val >= Fraction(2) ** 128:   # rounded past the largest finite binary32
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))   # val has <= 24 significant bits: exact in float64


def f32_add(a, b) -> np.float32:
    return round_f32(frac(a) + frac(b))


def f32_sub(a, b) -> np.float32:
    return round_f32(frac(a) - frac(b))


def f32_mul(a, b) -> np.float32:
    return round_f32(frac(a) * frac(b))


def f32_div(a, b) -> np.float32:
    return round_f32(frac(a) / frac(b))


def f32_sqrt(a) -> np.float32:
    """Correctly rounded binary32 square root of a binary32 value, by integer search."""
    q = frac(a)
    if q < 0:
        return np.float32(np.nan)
    if q == 0:
        return np.float32(0.0)
    r = np.float32(np.sqrt(np.float64(a)))       # candidate, then verify with exact midpoints
    for _ in range(4):
        lo = np.nextafter(r, np.float32(0.0))
        hi = np.nextafter(r, np.float32(np.inf))
        mid_lo = (frac(lo) + frac(r)) / 2
        mid_hi = (frac(r) + frac(hi)) / 2
        if mid_lo * mid_lo > q:
            r = lo
        elif mid_hi * mid_hi < q:
            r = hi
        else:
            # on an exact midpoint the even significand wins
            if mid_hi * mid_hi == q and (int(np.float32(hi).view(np.uint32)) % 2 == 0):
                r = hi
            if mid_lo * mid_lo == q and (int(np.float32(lo).view(np.uint32)) % 2 == 0):
                r = lo
            return np.float32(r)
    raise AssertionError("sqrt search did not converge")
