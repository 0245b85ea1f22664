"""Pins for the oracle's W8A8 variant (per-row activation scales, per-channel
weight scales):

* per-row quantisation against exact rationals: the scale from the row's amax
  (fp32 division, or rounded up to a power of two), codes the nearest E4M3 of
  the fp32 quotient, saturating; a static scale replaces the row's;
* fused SwiGLU + per-row quantisation equals the two steps one after the
  other, bit for bit, and leaves filtered rows untouched;
* the channel-scaled GEMM on integer codes against numpy int64 products;
* the whole W8A8 layer equals the pinned block layer bit for bit where the two
  readings coincide: every hidden group has the same amax (so row and group
  scales agree), weight scales are constant along K and across each 128-row
  block, and I = 128 (one SwiGLU group per row);
* a static scale equal to the dynamic one changes nothing.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests import exact
from tests.parity import f32_of_bits


def _row_scale(amax: float, fmt: int) -> Fraction:
    v = exact.round_f32(max(Fraction(amax), Fraction(1e-10)) / 448) if amax > 1e-10 else \
        exact.round_f32(Fraction(np.float32(1e-10).item()) / 448)
    if fmt == O.SCALE_UE8M0:
        e = 0
        while Fraction(2) ** e < v:
            e += 1
        while Fraction(2) ** (e - 1) >= v:
            e -= 1
        return Fraction(2) ** e
    return v


@pytest.mark.parametrize("fmt", [O.SCALE_FP32, O.SCALE_UE8M0])
@pytest.mark.parametrize("static", [0.0, 0.015625, 0.0123])
def test_quant_rows_against_exact_rounding(fmt, static):
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(5, 256, generator=g) * torch.tensor([0.01, 1, 3, 100, 0]).view(5, 1)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    q, s = O.quant_fp8_rows(xb, fmt, static)
    for r in range(5):
        vals = f32_of_bits(xb[r]).astype(np.float64)
        sc = Fraction(np.float32(static).item()) if static > 0 else _row_scale(np.abs(vals).max(), fmt)
        assert Fraction(float(s[r])) == sc
        for i in range(256):
            qv = exact.round_f32(Fraction(float(vals[i])) / sc)
            assert q[r, i] == exact.e4m3_nearest(Fraction(qv), vals[i] < 0 or (vals[i] == 0 and np.signbit(vals[i]))), (r, i)


def test_fused_rows_equal_two_steps_and_skip_filtered_rows():
    x, ids = synth.act_rows(64, 256, 16, "w8a8_rows", masked_frac=0.25)
    for clamp, fmt, static in ((float("inf"), O.SCALE_FP32, 0.0), (7.0, O.SCALE_UE8M0, 0.0),
                               (7.0, O.SCALE_FP32, 0.01)):
        q0 = np.full((64, 256), 0xAB, np.uint8)
        s0 = np.full(64, -1.0, np.float32)
        q, s = O.silu_and_mul_quant_fp8_rows(x, ids, None, 16, clamp, fmt, static, q0, s0)
        q2, s2 = O.quant_fp8_rows(O.silu_and_mul(x, clamp), fmt, static)
        live = ids.numpy() >= 0
        assert np.array_equal(q[live], q2[live]) and np.array_equal(s[live].view(np.uint32), s2[live].view(np.uint32))
        assert (q[~live] == 0xAB).all() and (s[~live] == -1.0).all()


def test_channel_gemm_on_integer_codes():
    hidden, ids, w, W = synth.exact_layer_inputs(2, 5, 3, 1024, 128, "w8a8_gemm")
    hb = hidden.view(torch.int16).numpy().view(np.uint16)
    aq, as_ = O.quant_fp8_rows(hb, O.SCALE_FP32)
    ws = np.exp2(np.random.default_rng(1).integers(-9, -6, (5, 256))).astype(np.float32)
    acc, mag = O.grouped_gemm_channel(aq, as_, 3, W.w13, ws, ids, 0, 5, exact=True)
    C = O.grouped_gemm_channel(aq, as_, 3, W.w13, ws, ids, 0, 5)
    lut = np.zeros(256, np.int64)
    for c in range(256):
        v = exact.e4m3_spec_value(c)
        if v is not None and v.denominator == 1:
            lut[c] = int(v)
    ai = lut[aq]
    wi = lut[W.w13.numpy()]
    for r, e in enumerate(ids.numpy().reshape(-1)):
        if e < 0:
            assert np.isnan(acc[r]).all()
            continue
        t = r // 3
        dots = (wi[e] * ai[t][None, :]).sum(-1)
        ref = dots * (float(as_[t]) * ws[e].astype(np.float64))
        assert np.array_equal(acc[r], ref)
        assert np.array_equal(mag[r], np.abs(wi[e] * ai[t][None, :]).sum(-1) * np.abs(float(as_[t]) * ws[e]))
        from tests.parity import bf16_bits_rne
        assert np.array_equal(C[r], bf16_bits_rne(ref))


@pytest.mark.parametrize("clamp", [float("inf"), 7.0])
def test_w8a8_layer_equals_block_layer_where_they_coincide(clamp):
    M, E, k, H, I = 3, 6, 4, 1024, 128
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "w8a8_layer")
    rng = np.random.default_rng(2)
    c13 = np.exp2(rng.integers(-9, -6, (E, 2 * I // 128))).astype(np.float32)   # per 128-row block
    c2 = np.exp2(rng.integers(-9, -6, (E, H // 128))).astype(np.float32)
    blk13 = np.repeat(c13[:, :, None], H // 128, axis=2)                           # constant along K
    blk2 = np.repeat(c2[:, :, None], I // 128, axis=2)
    ch13 = np.repeat(c13, 128, axis=1)                                              # per output channel
    ch2 = np.repeat(c2, 128, axis=1)
    ref = O.fused_moe(hidden, ids, w, W.w13, blk13, W.w2, blk2, scale_fmt=O.SCALE_UE8M0, clamp=clamp)
    got = O.fused_moe_w8a8(hidden, ids, w, W.w13, ch13, W.w2, ch2, scale_fmt=O.SCALE_UE8M0, clamp=clamp)
    assert np.array_equal(got, ref)
    assert np.abs(f32_of_bits(ref)).max() > 0


def test_static_scale_equal_to_the_dynamic_one_changes_nothing():
    M, E, k, H, I = 2, 6, 4, 1024, 256
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "w8a8_static")
    hb = hidden.view(torch.int16).numpy().view(np.uint16)
    _, as_ = O.quant_fp8_rows(hb[:1], O.SCALE_FP32)
    rng = np.random.default_rng(3)
    ch13 = np.exp2(rng.integers(-9, -6, (E, 2 * I))).astype(np.float32)
    ch2 = np.exp2(rng.integers(-9, -6, (E, H))).astype(np.float32)
    one = slice(0, 1)
    dyn = O.fused_moe_w8a8(hidden[one], ids[one], w[one], W.w13, ch13, W.w2, ch2)
    sta = O.fused_moe_w8a8(hidden[one], ids[one], w[one], W.w13, ch13, W.w2, ch2, a1_static=float(as_[0]))
    assert np.array_equal(dyn, sta)
