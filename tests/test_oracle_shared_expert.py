"""Pin for running a shared expert as routes: a SwiGLU expert of width 2048
applied to every token equals, in the oracle, the sum of 8 pseudo-experts of
width 256 (its gate/up rows and down columns in chunks of 256, whole 128x128
blocks) taken with weight 1, up to the BF16 rounding of each pseudo-expert's
output before the weighted sum.  SwiGLU is elementwise over the width, the
activation's quantisation groups of 128 fall inside the chunks, and the down
projection is a sum over the width, so no other step differs."""
import numpy as np
import torch

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_shared_expert_split_into_routes():
    M, H, I, C = 3, 256, 2048, 8
    c = I // C
    hidden = synth.hidden_states(M, H, "shared_pin")
    W = synth.moe_weights(1, H, I, "shared_pin")  # the shared expert, one expert of width 2048
    ones = np.ones((M, 1), np.float32)
    mono = O.fused_moe(hidden, np.zeros((M, 1), np.int32), ones, W.w13, W.w13_s, W.w2, W.w2_s)
    # pseudo-expert j: gate rows [c j, c j + c), up rows I + the same, down columns [c j, c j + c)
    w13 = torch.stack([torch.cat([W.w13[0, c * j:c * (j + 1)], W.w13[0, I + c * j:I + c * (j + 1)]]) for j in range(C)])
    g = c // 128
    w13_s = torch.stack([torch.cat([W.w13_s[0, g * j:g * (j + 1)], W.w13_s[0, I // 128 + g * j:I // 128 + g * (j + 1)]])
                         for j in range(C)])
    w2 = torch.stack([W.w2[0, :, c * j:c * (j + 1)] for j in range(C)]).contiguous()
    w2_s = torch.stack([W.w2_s[0, :, g * j:g * (j + 1)] for j in range(C)]).contiguous()
    ids = np.tile(np.arange(C, dtype=np.int32), (M, 1))
    split, inter = O.fused_moe(hidden, ids, np.ones((M, C), np.float32), w13.contiguous(), w13_s.contiguous(), w2,
                               w2_s, want_intermediates=True)
    a, b = f32(mono), f32(split)
    parts = np.abs(f32(inter["y"])).reshape(M, C, H).sum(axis=1)
    # BF16 keeps 8 significant bits: a rounding moves a value by at most 2^-8 of
    # it.  Each part is rounded once, their fp32 sum is exact to 2^-24, and the
    # two results are rounded once more each
    bound = 2.0 ** -8 * (parts + np.abs(a) + np.abs(b)) + 2.0 ** -20 * parts
    assert np.all(np.abs(a - b) <= bound)
    assert np.abs(a).max() > 0
    # the SwiGLU codes agree exactly: the activation of pseudo-expert j is
    # columns [c j, c j + c) of the shared expert's
    _, mi = O.fused_moe(hidden, np.zeros((M, 1), np.int32), ones, W.w13, W.w13_s, W.w2, W.w2_s,
                        want_intermediates=True)
    for j in range(C):
        assert np.array_equal(inter["q"].reshape(M, C, c)[:, j], mi["q"][:, c * j:c * (j + 1)])
