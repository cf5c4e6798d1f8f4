"""Exact-arithmetic helpers for pinning the oracle (rationals, no NumPy math).

Independent of both the oracle and the GPU path: these routines use Python
``fractions.Fraction`` and integer arithmetic only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def frac(x) -> Fraction:
    """Exact rational value of a finite float."""
    return Fraction(float(x))


def round_to_f32(r: Fraction) -> np.float32:
    """Nearest IEEE binary32 value to the rational ``r`` (ties to even).

    Written from the binary32 format: 24-bit significand for normal numbers
    (exponent >= -126), fixed quantum 2**-149 below that, overflow to inf.
    """
    if r == 0:
        return np.float32(0.0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e, -126) - 23          # quantum exponent
    scaled = a / (Fraction(2) ** q_exp)  # value in units of the quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * (Fraction(2) ** q_exp)
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))


def round_half_even(r: Fraction) -> int:
    """Nearest integer to ``r``, ties to the even integer."""
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def round_to_f16(r: Fraction) -> np.float32:
    """Nearest IEEE binary16 value to the rational ``r`` (ties to even), as float32.

    Written from the binary16 format: 11-bit significand for normal numbers
    (exponent >= -14), fixed quantum 2**-24 below that, largest finite value
    65504, beyond which rounding goes to infinity.
    """
    if r == 0:
        return np.float32(0.0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e, -14) - 10
    scaled = a / (Fraction(2) ** q_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * (Fraction(2) ** q_exp)
    if val > 65504:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))
