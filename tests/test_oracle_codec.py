"""Pins for the oracle's number formats: OCP E4M3FN and BF16 rounding.

The oracle's codec is checked against (a) the OCP specification's own table of
E4M3 values (tests/golden/e4m3fn_ocp.txt), (b) an exhaustive nearest-code
search written from the format definition with exact rationals, and (c) the
closed form dec(enc(dec(c))) == c.
"""
import math
import os
import random
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_ocp.txt")


def test_ocp_table_values():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 10
    for code_s, val_s, _ in rows:
        code = int(code_s, 16)
        got = O.e4m3_decode(code)
        if val_s == "nan":
            assert math.isnan(got)
            continue
        want = float(val_s)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code_s, got, want)
        # and every finite table entry encodes back to its code
        assert O.e4m3_encode(want) == code


def test_decode_matches_spec_definition():
    for c in range(256):
        v = X.e4m3_spec_value(c)
        got = O.e4m3_decode(c)
        if v is None:
            assert math.isnan(got)
        else:
            assert Fraction(got) == v, hex(c)


def test_roundtrip_closed_form():
    for c in range(256):
        v = O.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert O.e4m3_encode(v) == c, hex(c)


def _check_encode(x: float):
    got = O.e4m3_encode(x)
    if math.isnan(x):
        want = 0xFF if math.copysign(1, x) < 0 else 0x7F
    elif math.isinf(x):
        want = 0xFE if x < 0 else 0x7E
    else:
        want = X.e4m3_nearest(Fraction(x), math.copysign(1, x) < 0)
    assert got == want, (x, hex(got), hex(want))


def test_encode_exhaustive_over_bf16_values():
    # Every BF16 bit pattern as an fp32 input: covers all binades, signs,
    # zeros, subnormals, saturation and NaN/inf.
    for h in range(1 << 16):
        _check_encode(X.bf16_value(h))


def test_encode_at_and_around_every_rounding_midpoint():
    vals = X._POS_VALS
    for lo, hi in zip(vals, vals[1:]):
        mid = (lo + hi) / 2
        m = float(np.float32(float(mid)))
        assert Fraction(m) == mid  # midpoints are exact in fp32
        for b in (-2, -1, 0, 1, 2):
            x = X.f32_from_bits(X.f32_bits(m) + b) if m > 0 else m
            _check_encode(x)
            _check_encode(-x)
    # just above the largest finite value and far beyond it
    for x in (448.0, 448.00003, 463.99997, 464.0, 480.0, 1e6, 3.4e38):
        _check_encode(x)
        _check_encode(-x)


def test_encode_random_fp32():
    rng = random.Random(7)
    for _ in range(20000):
        b = rng.getrandbits(32)
        x = X.f32_from_bits(b)
        # concentrate on the E4M3 range: scale exponent into [-12, 9]
        if not math.isfinite(x) or x == 0:
            continue
        m, e = math.frexp(x)
        x = float(np.float32(math.ldexp(m, rng.randint(-12, 9))))
        _check_encode(x)


def test_f32_to_bf16_against_exact_rounding():
    rng = random.Random(11)
    specials = [0.0, -0.0, 1.0, -1.0, 3.4028234663852886e38, 1.17549435e-38, 1e-45, -1e-45]
    xs = specials + [X.f32_from_bits(rng.getrandbits(32)) for _ in range(20000)]
    for x in xs:
        if math.isnan(x):
            assert (O.f32_to_bf16(x) & 0x7FFF) > 0x7F80
            continue
        if math.isinf(x):
            assert O.f32_to_bf16(x) == X.f32_bits(x) >> 16
            continue
        want = X.round_bf16(Fraction(x))
        wb = X.bf16_bits_of(want)
        if want == 0 and math.copysign(1, x) < 0:
            wb = 0x8000
        assert O.f32_to_bf16(x) == wb, x


def test_f64_to_bf16_against_exact_rounding():
    rng = random.Random(13)
    for _ in range(20000):
        x = struct.unpack("<d", struct.pack("<Q", rng.getrandbits(64)))[0]
        if not math.isfinite(x):
            continue
        m, e = math.frexp(x)
        x = math.ldexp(m, rng.randint(-140, 130))
        want = X.round_bf16(Fraction(x))
        wb = X.bf16_bits_of(want)
        if want == 0 and math.copysign(1, x) < 0:
            wb = 0x8000
        assert O.f64_to_bf16(x) == wb, x
    # ties: exact BF16 midpoints go to the even neighbour
    for h in (0x3F80, 0x3F81, 0x4000, 0x0001, 0x7F7E):
        lo = Fraction(X.bf16_value(h))
        hi = Fraction(X.bf16_value(h + 1))
        mid = (lo + hi) / 2
        assert O.f64_to_bf16(float(mid)) == (h if h % 2 == 0 else h + 1)
