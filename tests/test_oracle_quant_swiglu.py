"""Pins for the oracle's group-128 quantisation, SwiGLU and fused act+quant.

* group quant: brute-force nearest-code search on each x/s, closed-form scale
  properties (fp32: s = amax/448 rounded; UE8M0: power of two, s/2 < v <= s),
  the all-zero group, per-group indexing;
* exp: exhaustive over every finite BF16 gate value against a 100-bit mpmath
  exp rounded exactly to fp32;
* SwiGLU: exhaustive over every finite BF16 gate value against the exact real
  silu(g)*u (mpmath), within the error bound of an fp32 pipeline followed by one
  BF16 rounding; clamp special cases;
* act+quant: row filtering leaves masked rows untouched.
"""
import math
import random
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import oracle as O
from tests import exact as X

mpmath.mp.prec = 100


def _bf16_row(vals):
    return np.array([X.f32_bits(float(np.float32(v))) >> 16 for v in vals], np.uint16)


def _rand_bf16(rng, n, scale=1.0):
    v = rng.standard_normal(n).astype(np.float32) * np.float32(scale)
    return (v.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern is a valid input


# ---------------------------------------------------------------- group quant

@pytest.mark.parametrize("fmt", [O.SCALE_FP32, O.SCALE_UE8M0])
def test_group_quant_bruteforce(fmt):
    rng = np.random.default_rng(3)
    for K in (128, 256, 512):
        x = np.concatenate([_rand_bf16(rng, K, 10.0 ** rng.integers(-3, 3)) for _ in range(4)]).reshape(4, K)
        q, s = O.quant_fp8(x, fmt)
        for r in range(4):
            for g in range(K // 128):
                grp = [X.bf16_value(h) for h in x[r, g * 128:(g + 1) * 128]]
                amax = max(abs(v) for v in grp)
                sc = float(s[r, g])
                v = Fraction(float(np.float32(max(amax, np.float32(1e-10))) / np.float32(448.0)))
                if fmt == O.SCALE_FP32:
                    assert Fraction(sc) == v
                else:
                    # power of two with s/2 < v <= s
                    m, e = math.frexp(sc)
                    assert m == 0.5
                    assert Fraction(sc) / 2 < v <= Fraction(sc)
                for i, xv in enumerate(grp):
                    t = float(np.float32(xv) / np.float32(sc))  # one IEEE fp32 division
                    want = X.e4m3_nearest(Fraction(t), math.copysign(1, t) < 0)
                    assert q[r, g * 128 + i] == want, (r, g, i, xv, sc)


def test_group_quant_closed_forms():
    rng = np.random.default_rng(5)
    x = _rand_bf16(rng, 8 * 384, 3.0).reshape(8, 384)
    q, s = O.quant_fp8(x, O.SCALE_FP32)
    for r in range(8):
        for g in range(3):
            xs = np.array([X.bf16_value(h) for h in x[r, g * 128:(g + 1) * 128]])
            i = int(np.argmax(np.abs(xs)))
            # the amax element lands on +-448
            assert q[r, g * 128 + i] & 0x7F == 0x7E
            # dequantised values within half a code spacing of the input
            for j in range(128):
                d = O.e4m3_decode(int(q[r, g * 128 + j])) * float(s[r, g])
                assert abs(d - xs[j]) <= abs(xs[j]) * 0.0625 + float(s[r, g]) * 2 ** -10 + 1e-30


def test_group_quant_zero_group_and_indexing():
    x = np.zeros((2, 384), np.uint16)
    # group 1 of row 0 holds a single 3.0, group 2 of row 1 a single -0.5
    x[0, 128 + 17] = _bf16_row([3.0])[0]
    x[1, 256 + 5] = _bf16_row([-0.5])[0]
    q, s = O.quant_fp8(x, O.SCALE_FP32)
    eps_scale = float(np.float32(1e-10) / np.float32(448.0))
    assert s[0, 0] == np.float32(eps_scale) and s[0, 2] == np.float32(eps_scale)
    assert s[0, 1] == np.float32(np.float32(3.0) / np.float32(448.0))
    assert s[1, 2] == np.float32(np.float32(0.5) / np.float32(448.0))
    assert np.count_nonzero(q[0]) == 1 and q[0, 128 + 17] == 0x7E
    assert np.count_nonzero(q[1]) == 1 and q[1, 256 + 5] == 0xFE
    qu, su = O.quant_fp8(x, O.SCALE_UE8M0)
    # 3/448 = 0.0067 -> 2^-7 ; 0.5/448 -> 2^-9 (0.00195 >= 0.001116)
    assert su[0, 1] == np.float32(2.0 ** -7) and su[1, 2] == np.float32(2.0 ** -9)
    # 3 / 2^-7 = 384 exactly -> code for 384 = 1.5 * 2^8
    assert qu[0, 128 + 17] == 0x7C and qu[1, 256 + 5] == X.e4m3_nearest(Fraction(-256), True)


# ---------------------------------------------------------------- exp and SwiGLU

def _exact_exp_f32(x: float):
    """exp(x) rounded exactly to fp32 from a 100-bit mpmath value (exp of a
    nonzero rational is never a rounding tie, and 100 bits leave a margin far
    beyond any fp32 decision)."""
    if x > 89.0:                      # exp(x) > 4e38 > largest finite fp32
        return float("inf")
    if x < -110.0:                    # exp(x) < 2^-158, below half the least subnormal
        return Fraction(0)
    return X.round_f32(_to_fraction(mpmath.exp(mpmath.mpf(x))))


def test_exp_rn_exhaustive_bf16():
    bad = []
    for h in X.all_finite_bf16():
        g = X.bf16_value(h)
        got = O.exp_rn(-g)
        want = _exact_exp_f32(-g)
        if isinstance(want, float):
            ok = got == want
        else:
            ok = Fraction(got) == want if math.isfinite(got) else False
        if not ok:
            bad.append((h, g, got, want))
    assert not bad, bad[:5]


def _silu_exact(g: float, u: float, limit: float):
    gg, uu = g, u
    if math.isfinite(limit):
        gg = min(gg, limit)
        uu = min(max(uu, -limit), limit)
    G = mpmath.mpf(gg)
    return G / (1 + mpmath.exp(-G)) * mpmath.mpf(uu), gg


def _to_fraction(v):
    if v == 0:
        return Fraction(0)
    m, e = mpmath.frexp(v)
    return Fraction(int(m * mpmath.mpf(2) ** 90)) * Fraction(2) ** (int(e) - 90)


def _check_swiglu(gh: int, uh: int, limit: float):
    g, u = X.bf16_value(gh), X.bf16_value(uh)
    got = O.swiglu_one(gh, uh, limit)
    val, gg = _silu_exact(g, u, limit)
    if -gg > 88.72:  # exp(-g) overflows fp32: the fp32 form of silu gives a signed zero
        assert got & 0x7FFF == 0, (g, u, hex(got))
        return
    x = _to_fraction(val)
    want = X.round_bf16(x)
    wb = X.bf16_bits_of(want) if want != 0 else None
    if wb is None:  # exact result rounds to zero in bf16
        assert got & 0x7FFF == 0 or abs(Fraction(X.bf16_value(got))) <= abs(x) * 2, (g, u)
        return
    if got == wb:
        return
    # an fp32 pipeline of 4 roundings (exp, 1+e, g/d, *u) carries a relative
    # error below 5*2^-24; only inputs that close to a BF16 midpoint may differ
    assert X.bf16_neighbours_midpoint_distance(x) < Fraction(5, 2 ** 24) * 2, (g, u, hex(got), hex(wb))
    assert abs(got - wb) == 1


def test_swiglu_exhaustive_gate_unit_up():
    one = 0x3F80
    for gh in X.all_finite_bf16():
        _check_swiglu(gh, one, math.inf)


def test_swiglu_random_pairs_and_clamp():
    rng = random.Random(17)
    finite = X.all_finite_bf16()
    for _ in range(20000):
        gh = rng.choice(finite)
        # keep up values in a moderate range so products stay normal
        uh = X.f32_bits(float(np.float32(rng.uniform(-20, 20)))) >> 16
        _check_swiglu(gh, uh, math.inf)
        _check_swiglu(gh, uh, 7.0)


def test_swiglu_special_cases():
    bf = lambda v: X.f32_bits(float(np.float32(v))) >> 16
    one = bf(1.0)
    assert O.swiglu_one(bf(0.0), one) == 0
    # large positive gate: sigmoid rounds to 1, silu(g) = g
    for g in (20.0, 64.0, 1000.0):
        assert O.swiglu_one(bf(g), bf(2.5)) == bf(g * 2.5)
    # clamp: gate above the limit behaves as the limit; up clipped both ways
    assert O.swiglu_one(bf(8.0), one, 7.0) == O.swiglu_one(bf(7.0), one, 7.0)
    assert O.swiglu_one(bf(3.0), bf(-9.0), 7.0) == O.swiglu_one(bf(3.0), bf(-7.0), 7.0)
    assert O.swiglu_one(bf(3.0), bf(9.0), 7.0) == O.swiglu_one(bf(3.0), bf(7.0), 7.0)
    # negative gates are not clamped from below
    assert O.swiglu_one(bf(-9.0), one, 7.0) == O.swiglu_one(bf(-9.0), one)
    # the clamp changes the result when it fires
    assert O.swiglu_one(bf(9.0), one, 7.0) != O.swiglu_one(bf(9.0), one)


def test_silu_and_mul_layout():
    # gate columns first, then up columns: row [g0..gI-1, u0..uI-1]
    rng = np.random.default_rng(1)
    I = 128
    x = _rand_bf16(rng, 3 * 2 * I).reshape(3, 2 * I)
    out = O.silu_and_mul(x)
    for r in range(3):
        for i in (0, 5, 127):
            assert out[r, i] == O.swiglu_one(int(x[r, i]), int(x[r, I + i]))


# ---------------------------------------------------------------- act + quant

@pytest.mark.parametrize("fmt", [O.SCALE_FP32, O.SCALE_UE8M0])
def test_act_quant_filtering_leaves_rows_untouched(fmt):
    rng = np.random.default_rng(9)
    rows, I, E = 16, 256, 12
    x = _rand_bf16(rng, rows * 2 * I, 2.0).reshape(rows, 2 * I)
    ids = rng.integers(0, E, rows).astype(np.int32)
    ids[[1, 4, 9]] = -1
    emap = np.arange(E, dtype=np.int32)
    emap[[2, 3]] = -1
    sentinel_q = np.full((rows, I), 0xA5, np.uint8)
    sentinel_s = np.full((rows, I // 128), -7.0, np.float32)
    ref_q, ref_s = O.quant_fp8(O.silu_and_mul(x, 7.0), fmt)
    for mode in ("none", "ids", "map"):
        q, s = O.silu_and_mul_quant_fp8(x, None if mode == "none" else ids, emap if mode == "map" else None, E,
                                        7.0, fmt, q_init=sentinel_q, s_init=sentinel_s)
        for r in range(rows):
            live = mode == "none" or (ids[r] >= 0 and (mode == "ids" or emap[ids[r]] >= 0))
            if live:
                assert (q[r] == ref_q[r]).all() and (s[r] == ref_s[r]).all()
            else:
                assert (q[r] == 0xA5).all() and (s[r] == -7.0).all()
