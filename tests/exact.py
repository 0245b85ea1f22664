"""Exact-arithmetic helpers for the oracle's pins (pure Python, Fraction).

Written from the format definitions (OCP E4M3FN, IEEE binary32, bfloat16),
independently of the oracle's C code: rounding here is done on exact rationals
by locating the two neighbouring representable values.
"""
from __future__ import annotations

import bisect
import struct
from fractions import Fraction


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(b) & 0xFFFFFFFF))[0]


def bf16_value(h: int) -> float:
    return f32_from_bits(int(h) << 16)


# ---- E4M3FN from the OCP 8-bit floating point definition -------------------

def e4m3_spec_value(code: int):
    """Value of an E4M3FN byte straight from the format definition, as a
    Fraction; None for the NaN codes."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return None
    if e == 0:
        v = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        v = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
    return s * v


# non-negative finite codes 0x00..0x7E, sorted by value (they are monotone)
_POS_CODES = list(range(0x00, 0x7F))
_POS_VALS = [e4m3_spec_value(c) for c in _POS_CODES]
assert all(a < b for a, b in zip(_POS_VALS, _POS_VALS[1:]))


def e4m3_nearest(x: Fraction, negative: bool) -> int:
    """Nearest E4M3FN code to the exact value x (a Fraction, magnitude used),
    ties to the code with even mantissa, saturating at 448."""
    a = abs(x)
    sign = 0x80 if negative else 0
    if a >= _POS_VALS[-1]:
        return sign | _POS_CODES[-1]
    i = bisect.bisect_left(_POS_VALS, a)
    if _POS_VALS[i] == a:
        return sign | _POS_CODES[i]
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    if dlo < dhi:
        c = _POS_CODES[lo]
    elif dhi < dlo:
        c = _POS_CODES[hi]
    else:
        c = _POS_CODES[lo] if _POS_CODES[lo] % 2 == 0 else _POS_CODES[hi]
    return sign | c


# ---- rounding an exact rational to a binary format -------------------------

def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(x: Fraction, p: int, emin: int, emax: int):
    """Round x to a binary format with p significant bits, minimum normal
    exponent emin, largest finite exponent emax, nearest-even.  Returns a
    Fraction, or +-inf as a float on overflow."""
    if x == 0:
        return Fraction(0)
    neg = x < 0
    a = -x if neg else x
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    q = a / quantum
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    maxv = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if v > maxv:
        return float("-inf") if neg else float("inf")
    return -v if neg else v


def round_f32(x: Fraction):
    return round_binary(x, 24, -126, 127)


def round_bf16(x: Fraction):
    return round_binary(x, 8, -126, 127)


def bf16_bits_of(v) -> int:
    """BF16 bit pattern of an exactly representable value (Fraction or inf)."""
    if isinstance(v, float):
        return f32_bits(v) >> 16
    f = float(v)
    b = f32_bits(f)
    assert b & 0xFFFF == 0, "value not representable in bf16"
    return b >> 16


def bf16_neighbours_midpoint_distance(x: Fraction):
    """Distance from x to the nearest BF16 rounding midpoint, relative to |x|."""
    if x == 0:
        return Fraction(1)
    a = abs(x)
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 7)
    q = a / quantum
    n = q.numerator // q.denominator
    mid = (n + Fraction(1, 2)) * quantum
    d = abs(a - mid)
    # the midpoint below the current binade is also a candidate at exact powers
    d2 = abs(a - (n - Fraction(1, 2)) * quantum)
    return min(d, d2) / a


def all_finite_bf16():
    """Every finite BF16 bit pattern."""
    out = []
    for h in range(1 << 16):
        if (h >> 7) & 0xFF == 0xFF:
            continue
        out.append(h)
    return out
