"""Exact-arithmetic helpers for pinning the oracle (test code, independent of it).

Everything here uses Python integers / fractions.Fraction and torch's own
E4M3 decoding, never the oracle's arithmetic.
"""
import math
import struct
from fractions import Fraction

import torch

F32_MIN_EXP = -126
F32_MANT = 23


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def frac_of_f32(x):
    return Fraction(x)  # exact for any finite binary float


def _round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    d = q - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_f32(q: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) fp32 value of an exact rational;
    handles subnormals; overflow -> inf."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = math.floor(math.log2(a.numerator)) - math.floor(math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, F32_MIN_EXP)
    quantum = Fraction(2) ** (e - F32_MANT)
    k = _round_half_even(a / quantum)
    v = k * quantum
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def torch_e4m3_values():
    """Values of all 256 E4M3FN codes as decoded by torch (NaN as None)."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    out = []
    for v in codes.tolist():
        out.append(None if math.isnan(v) else Fraction(v))
    return out


_POS = None


def _positive_codes():
    global _POS
    if _POS is None:
        vals = torch_e4m3_values()
        _POS = [(c, vals[c]) for c in range(0, 0x7F) if vals[c] is not None]
    return _POS


def brute_force_e4m3(x: Fraction, negative_zero=False) -> int:
    """Nearest E4M3 code by exhaustive search over torch's code table;
    ties go to the code with an even mantissa (LSB 0); |x| >= 448 saturates.
    negative_zero: the sign to give a zero input (the sign bit of an fp32 zero)."""
    neg = x < 0 or (x == 0 and negative_zero)
    a = abs(x)
    if a >= 448:
        return (0x80 if neg else 0) | 0x7E
    best = None
    for c, v in _positive_codes():
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return (0x80 if neg else 0) | best[1]
