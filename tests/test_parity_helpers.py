"""CPU checks of the element-wise parity machinery (tests/parity.py).

The oracle's own outputs must pass every check with nothing flagged as
different, and outputs the oracle computes with a planted mistake -- one
block scale taken from the wrong block, one K group dropped, one route weight
on the wrong route -- must fail them.  So the bounds are loose enough for a
correct kernel and tight enough to catch the mistakes the normwise bound
lets through."""
import math

import numpy as np
import pytest
import torch

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.parity import (ActAllowed, bf16_step, check_layer, e4m3_encode, f32_of_bits, gate_up_exact,
                          layer_out_bound)

M, E, K, H, I = 2, 8, 4, 1024, 256


def _case(fmt, seed="helpers"):
    c = synth.LayerCase("helpers", M=M, E=E, k=K, H=H, I=I, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 0, only_active=False)
    return hidden, ids, w, W


def _act(hidden, ids, W, fmt, clamp):
    _, inter = O.fused_moe(hidden, ids, torch.ones(M, K), W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=fmt,
                           clamp=clamp, want_intermediates=True)
    return O.silu_and_mul(inter["h13"], clamp)


@pytest.mark.parametrize("fmt,clamp", [(O.SCALE_FP32, math.inf), (O.SCALE_UE8M0, 7.0)])
def test_oracle_passes_its_own_checks(fmt, clamp):
    hidden, ids, w, W = _case(fmt)
    acc, mag, _ = gate_up_exact(hidden, ids, W.w13, W.w13_s, K, fmt)
    allowed = ActAllowed(acc, mag, H, clamp, mfma=False)
    amb, wide, nd = allowed.check(_act(hidden, ids, W, fmt, clamp), "oracle SwiGLU")
    assert nd == 0 and amb < allowed.exp.size // 2
    out = O.fused_moe(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=fmt, clamp=clamp)
    ref, lo, hi, stats = layer_out_bound(hidden, ids, w, W, fmt, clamp)
    ndiff, steps = check_layer(out, ref, lo, hi, "oracle output")
    assert ndiff == 0 and steps == 0
    # an output's latitude is at most one BF16 step for most outputs (more
    # only where the weighted sum cancels), and none at all for many
    span = np.abs(f32_of_bits(hi).astype(np.float64) - f32_of_bits(lo))
    step = bf16_step(np.abs(f32_of_bits(ref).astype(np.float64)) + 1e-30)
    assert (span <= step).mean() > 0.6 and (span == 0).mean() > 0.3


def _planted(W, which):
    """A copy of the weights with one mistake a kernel could make."""
    W2 = synth.MoEWeights(W.w13.clone(), W.w13_s.clone(), W.w2.clone(), W.w2_s.clone())
    if which == "w13 block scale of the next block":
        W2.w13_s[:, 1, 3] = W.w13_s[:, 1, 4]
    elif which == "w13 group dropped":
        W2.w13[:, :, 256:384] = 0
    elif which == "w2 block scale of the next block":
        W2.w2_s[:, 2, 0] = W.w2_s[:, 2, 1]
    elif which == "w2 transposed block":
        blk = W2.w2[:, 0:128, 0:128].clone()
        W2.w2[:, 0:128, 0:128] = blk.transpose(1, 2)
    return W2


@pytest.mark.parametrize("which", ["w13 block scale of the next block", "w13 group dropped"])
def test_planted_gate_up_mistakes_fail_the_swiglu_check(which):
    fmt, clamp = O.SCALE_FP32, math.inf
    hidden, ids, w, W = _case(fmt)
    acc, mag, _ = gate_up_exact(hidden, ids, W.w13, W.w13_s, K, fmt)
    allowed = ActAllowed(acc, mag, H, clamp)
    with pytest.raises(AssertionError):
        allowed.check(_act(hidden, ids, _planted(W, which), fmt, clamp), which)


@pytest.mark.parametrize("which", ["w13 block scale of the next block", "w2 block scale of the next block",
                                   "w2 transposed block", "route weight on the wrong route"])
def test_planted_mistakes_fail_the_layer_check(which):
    fmt, clamp = O.SCALE_UE8M0, 7.0
    hidden, ids, w, W = _case(fmt)
    ref, lo, hi, _ = layer_out_bound(hidden, ids, w, W, fmt, clamp)
    if which == "route weight on the wrong route":
        w_bad = w.clone()
        w_bad[0, [0, 1]] = w[0, [1, 0]]
        bad = O.fused_moe(hidden, ids, w_bad, W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=fmt, clamp=clamp)
    else:
        Wb = _planted(W, which)
        bad = O.fused_moe(hidden, ids, w, Wb.w13, Wb.w13_s, Wb.w2, Wb.w2_s, scale_fmt=fmt, clamp=clamp)
    with pytest.raises(AssertionError):
        check_layer(bad, ref, lo, hi, which)


def test_vectorised_encoder_matches_the_oracle():
    # every finite BF16 value, scaled into and beyond the E4M3 range
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = f32_of_bits(bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16))
    for scale in (1.0, 2.0 ** -7, 2.0 ** 9):
        v = (x.astype(np.float64) * scale).astype(np.float32)
        v = v[np.isfinite(v)]
        ref = np.array([O.e4m3_encode(float(t)) for t in v], np.uint8)
        assert np.array_equal(e4m3_encode(v), ref)
