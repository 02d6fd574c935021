"""Exact rational arithmetic used to pin the oracle (no floating-point division).

Everything here works on ``fractions.Fraction`` values of the binary32 inputs,
so it shares no rounding behaviour with the C oracle or the GPU.
"""
from __future__ import annotations

from fractions import Fraction
from math import floor

import numpy as np


def f32_fraction(v) -> Fraction:
    """Exact rational value of a binary32 number."""
    return Fraction(float(np.float32(v)))


def round_half_even(r: Fraction) -> int:
    """Nearest integer to an exact rational, ties to the even integer."""
    lo = floor(r)
    rem = r - lo
    if rem > Fraction(1, 2):
        return lo + 1
    if rem < Fraction(1, 2):
        return lo
    return lo if lo % 2 == 0 else lo + 1


def round_to_f32(r: Fraction) -> float:
    """Correctly rounded (nearest-even) binary32 value of an exact rational.

    Normal numbers carry 24 significant bits; below 2^-126 the spacing is a
    fixed 2^-149 (gradual underflow).  Overflow is not handled (not needed).
    """
    if r == 0:
        return 0.0
    sign = -1.0 if r < 0 else 1.0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    ulp_exp = max(e - 23, -149)
    units = a / (Fraction(2) ** ulp_exp)
    n = round_half_even(units)
    return sign * float(Fraction(n) * Fraction(2) ** ulp_exp)


def ulp_f32(v: float) -> Fraction:
    """Spacing of binary32 numbers at |v| (the gap above |v|)."""
    a = abs(Fraction(v))
    if a == 0:
        return Fraction(2) ** -149
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return Fraction(2) ** max(e - 23, -149)


def argmin_code(w: Fraction, s: Fraction, lo: int = -8, hi: int = 7) -> int:
    """Brute force: the code q in [lo, hi] minimising |w - q*s|, ties to even q."""
    best = None
    for q in range(lo, hi + 1):
        d = abs(w - q * s)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def round_to_16(r: Fraction, fmt: str) -> float:
    """Correctly rounded (nearest-even) value of an exact rational in the
    16-bit format ``fmt`` ("bf16": 8 significant bits, normal from 2^-126;
    "f16": 11 significant bits, normal from 2^-14).  Results whose magnitude
    reaches 2^(emax+1) after rounding are returned as +-inf."""
    p, emin, emax = (8, -126, 127) if fmt == "bf16" else (11, -14, 15)
    if r == 0:
        return 0.0
    sign = -1.0 if r < 0 else 1.0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp_exp = max(e, emin) - (p - 1)
    n = round_half_even(a / (Fraction(2) ** ulp_exp))
    v = Fraction(n) * Fraction(2) ** ulp_exp
    if v >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * float(v)
