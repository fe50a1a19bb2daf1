"""Exact-arithmetic helpers for pinning the oracle (test code, not the oracle).

Values are Python ``fractions.Fraction``; rounding to IEEE binary32 is done
here from the definition (round to nearest, ties to even, gradual
underflow), independently of numpy's float32 arithmetic.
"""

from fractions import Fraction

import torch


def round_f32(v):
    """Round a Fraction to the nearest binary32 value (ties to even); returns a Fraction."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)  # below 2^-126 the quantum stays 2^-149 (subnormals)
    quantum = Fraction(2) ** (e - 23)
    n, rem = divmod(a, quantum)
    if rem * 2 > quantum or (rem * 2 == quantum and n % 2 == 1):
        n += 1
    r = n * quantum
    if r > (2 - Fraction(2) ** -23) * Fraction(2) ** 127:
        raise OverflowError("binary32 overflow")
    return sign * r


def e4m3_values_torch():
    """Value of each code 0..255 as decoded by torch's float8_e4m3fn (an independent decoder)."""
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
