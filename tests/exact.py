"""Exact rational arithmetic for pinning the oracle.

Everything here works on ``fractions.Fraction`` values and rounds them with
IEEE-754 round-to-nearest-even written out from its definition (nearest
representable value; on a tie, the one with an even last significand bit).  It
never calls the oracle and never uses float arithmetic for a result, so a
value it produces is an independent statement of what the fp32/bf16 rounding of
an exact quantity is.
"""

from __future__ import annotations

import decimal
import math
import struct
from fractions import Fraction

import numpy as np


def _round_to_format(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round x to a binary format with ``mant_bits`` significand bits (including
    the implicit one), minimum normal exponent ``emin`` and maximum ``emax``.
    Returns +-inf (as a float) on overflow."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)  # subnormals share the minimum exponent's spacing
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    k = a / ulp
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    max_finite = (2 - Fraction(2) ** (1 - mant_bits)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * r


def rn32(x) -> Fraction:
    """Nearest fp32 value of an exact number (ties to even)."""
    return _round_to_format(Fraction(x), 24, -126, 127)


def rnbf16(x) -> Fraction:
    """Nearest bf16 value of an exact number (ties to even)."""
    return _round_to_format(Fraction(x), 8, -126, 127)


def f32_bits(x) -> int:
    """Bit pattern of an fp32-representable exact value."""
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bf16_bits_to_fraction(b: int) -> Fraction:
    return Fraction(bits_f32((b & 0xFFFF) << 16))


def rne_int(x: Fraction) -> int:
    """Nearest integer, ties to even, by brute force over the two neighbours."""
    lo = math.floor(x)
    hi = lo + 1
    dlo, dhi = x - lo, hi - x
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if lo % 2 == 0 else hi


_CTX = decimal.Context(prec=60, Emax=10**6, Emin=-(10**6))


def exp_exact(x: Fraction) -> Fraction:
    """exp(x) to 60 significant decimal digits (far beyond the 2^-24 needed to
    round it to fp32 except within ~1e-50 of a rounding midpoint)."""
    d = _CTX.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))
    return Fraction(_CTX.exp(d))


def sigmoid_exact(g: Fraction) -> Fraction:
    return 1 / (1 + exp_exact(-g))


def all_finite_bf16() -> np.ndarray:
    """All 65,280 finite bf16 bit patterns (both zeros included)."""
    b = np.arange(65536, dtype=np.uint32)
    exp_field = (b >> 7) & 0xFF
    return b[exp_field != 0xFF].astype(np.uint16)
