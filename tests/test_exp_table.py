"""CPU checks of the generated exp(-g) table the kernels' SwiGLU uses for BF16
gates: the ranges it leaves out really round to 1, +0 or +inf in fp32, and its
entries are exp in double precision rounded once to fp32 (numpy's own
float64 -> float32 conversion as the independent rounding)."""
import math
import struct

import numpy as np

from block_fp8_mixture_route_amd import gen_exp_table as T


def _bf16(sign, field, mant):
    return struct.unpack("<f", struct.pack("<I", ((sign << 15) | (field << 7) | mant) << 16))[0]


def _f32_bits(x):
    return int(np.array([x], dtype=np.float64).astype(np.float32).view(np.uint32)[0])


def test_left_out_ranges():
    # below exponent field 96: |g| < 2^-31, exp(-g) rounds to exactly 1
    for s in (0, 1):
        g = _bf16(s, T.LO - 1, 127)
        assert np.float32(math.exp(-g)) == np.float32(1.0)
    # above field 134: |g| >= 256, +0 for positive gates, +inf for negative
    assert np.float32(math.exp(-_bf16(0, T.HI + 1, 0))) == 0.0
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(math.exp(256.0)))


def test_entries_match_rounded_double_exp():
    rng = np.random.default_rng(3)
    for _ in range(2000):
        s, f, m = int(rng.integers(2)), int(rng.integers(T.LO, T.HI + 1)), int(rng.integers(128))
        g = _bf16(s, f, m)
        with np.errstate(over="ignore"):
            want = _f32_bits(math.exp(-g)) if -g < 709 else 0x7F800000
        assert T.entry(s, f, m) == want, (s, f, m)
    # the boundary entries themselves
    assert T.entry(0, T.LO, 0) == _f32_bits(math.exp(-2.0 ** -31))
    assert T.entry(1, T.HI, 127) == 0x7F800000  # exp(255) overflows fp32


def test_table_layout():
    text = T.render()
    assert f"kExpNegBf16[{2 * (T.HI - T.LO + 1) * 128}]" in text
    words = [int(w, 16) for w in text.split("{", 1)[1].split("}")[0].replace("u", "").replace(",", " ").split()]
    assert words[(1 * 39 + 127 - 96) * 128 + 0] == T.entry(1, 127, 0)  # g = -1: exp(1)
    assert struct.unpack("<f", struct.pack("<I", words[(0 * 39 + 127 - 96) * 128]))[0] == np.float32(math.exp(-1.0))
