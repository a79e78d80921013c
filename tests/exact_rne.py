"""Exact rational reference for the oracle's pins (pure Python, fractions only).

Independent of the oracle's C code: values are decoded with numpy's float16
view / the bfloat16 bit definition, summed exactly as Fractions, and rounded
with a round-half-to-even written here on rationals.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

F32, F16, BF16 = 0, 1, 2

# (fraction bits p, min normal exponent, max exponent, exponent-field width)
FORMATS = {
    F16: (10, -14, 15, 5),
    BF16: (7, -126, 127, 8),
    F32: (23, -126, 127, 8),
}


def value_of_bits16(bits: int, dtype: int) -> float:
    if dtype == F16:
        return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def value_of_out(x, dtype: int) -> float:
    if dtype == F32:
        return float(np.float32(x))
    return value_of_bits16(int(x), dtype)


def _floor_log2(a: Fraction) -> int:
    """Largest e with 2^e <= a, for a > 0 (exact)."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rne_bits(x, dtype: int) -> int:
    """Round an exact value (Fraction, or float inf/nan) to dtype; return bits."""
    p, emin, emax, ew = FORMATS[dtype]
    sign_shift = p + ew
    exp_ones = (1 << ew) - 1
    if isinstance(x, float):
        if math.isnan(x):
            return (exp_ones << p) | (1 << (p - 1))
        if math.isinf(x):
            return ((1 << sign_shift) if x < 0 else 0) | (exp_ones << p)
        x = Fraction(x)
    sign = (1 << sign_shift) if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign  # sign of an exact zero: callers compare zeros by value
    e = max(_floor_log2(a), emin)
    q = Fraction(2) ** (e - p)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl == 2 ** (p + 1):
        fl = 2 ** p
        e += 1
    if fl < 2 ** p:
        return sign | fl  # subnormal (e == emin)
    if e > emax:
        return sign | (exp_ones << p)
    return sign | ((e + emax) << p) | (fl - 2 ** p)


def max_norm_bits(dtype: int) -> int:
    return {F16: 0x7BFF, BF16: 0x7F7F, F32: 0x7F7FFFFF}[dtype]


def satf_bits(bits: int, dtype: int) -> int:
    """+Inf -> +MAX_NORM, -Inf -> -MAX_NORM, NaN -> +0, everything else unchanged."""
    p, _, _, ew = FORMATS[dtype]
    exp_ones = (1 << ew) - 1
    sign_bit = 1 << (p + ew)
    is_special = ((bits >> p) & exp_ones) == exp_ones
    if not is_special:
        return bits
    if bits & ((1 << p) - 1):
        return 0
    return (bits & sign_bit) | max_norm_bits(dtype)
