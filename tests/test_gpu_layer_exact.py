"""GPU parity of the whole layer, element by element.

1. Exact-arithmetic workloads (synth.exact_layer_inputs): every sum the layer
   forms is exact in fp32 in any order, so every correct implementation gives
   the oracle's output bit for bit, and its SwiGLU rows too.  Checked on every
   path that takes the shape: the few-token and small-batch kernels (whose
   SwiGLU rows are read from the workspace after their first stage) and the
   general path.
2. Seeded Gaussian workloads: the SwiGLU rows of the first stage must be the
   oracle's, except where a gate/up value lies within the fp32 error bound of a
   BF16 rounding boundary (counted and printed), and every output must lie
   within the element-wise bound of tests/parity.py.

The shapes cover the branches the decode workload alone leaves out: a hidden
width that is not a multiple of 1024 (a half-filled last 1 KB chunk of the
gate/up rows), down workgroups whose row count does not divide H, 16 routes
per token, 6 and 8 tokens on the small-batch path, and intermediate widths 384
and 512 there."""
import math

import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import assert_layer_elementwise, bf16_np, dev, oracle_inputs_for_tokens, print_case
from tests.parity import ActAllowed, gate_up_exact

pytestmark = pytest.mark.gpu

PATH_FLAGS = {"token": bfp8.FLAG_LAYER_TOKEN, "decode": bfp8.FLAG_LAYER_DECODE, "general": bfp8.FLAG_LAYER_GENERAL}
FIRST_STAGE = {"token": "token_gate_up_swiglu", "decode": "decode_gate_up_swiglu"}

# (M, E, k, H, I)
SHAPES = [
    (1, 16, 8, 7168, 256),   # the decode workload's widths
    (4, 32, 8, 7168, 256),
    (1, 16, 8, 2560, 256),   # H not a multiple of 1024; 12-row down blocks
    (2, 24, 16, 3200, 256),  # 16 routes per token, H not a multiple of 1024
    (3, 12, 4, 256, 128),
    (6, 16, 8, 2048, 384),   # small-batch path: 6 tokens, I = 384
    (8, 16, 8, 1024, 512),   # small-batch path: 8 tokens, I = 512
    (1, 16, 8, 4096, 512),
]


def _paths(M, H, k, E, I):
    """Paths that take this shape (a forced path outside its limits is
    rejected, so the stage list tells)."""
    out = []
    for name, flag in PATH_FLAGS.items():
        try:
            st = bfp8.fused_moe_stages(M, H, k, E, I, bfp8.opts(flags=flag))
        except bfp8.BFP8MoEError:
            continue
        if name == "general" or st[0] == FIRST_STAGE[name]:
            out.append(name)
    return out


def _stage0_act(path, hidden, ids, w, W, E, I, fmt, clamp):
    """SwiGLU rows [M*k, I] BF16 of the path's first stage, read from the
    workspace (the few-token and small-batch paths keep them at its start)."""
    M, H = hidden.shape
    k = ids.shape[1]
    o = bfp8.opts(scale_fmt=fmt, clamp_limit=clamp, flags=PATH_FLAGS[path] | bfp8.FLAG_ONLY_STAGE(0))
    need = bfp8.fused_moe_workspace_size(M, H, k, E, I, o)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev())
    bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o, ws=ws)
    torch.cuda.synchronize()
    return ws[: M * k * I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(M * k, I)


def _dev_weights(W):
    return synth.MoEWeights(W.w13.to(dev()), W.w13_s.to(dev()), W.w2.to(dev()), W.w2_s.to(dev()))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_E%d_k%d_H%d_I%d" % s)
def test_exact_workload_bit_exact(shape):
    M, E, k, H, I = shape
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "gpu_exact")
    Wd = _dev_weights(W)
    paths = _paths(M, H, k, E, I)
    assert "general" in paths
    for clamp in (math.inf, 7.0):
        ref, inter = O.fused_moe(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=bfp8.SCALE_UE8M0,
                                 clamp=clamp, want_intermediates=True)
        ref_act = O.silu_and_mul(inter["h13"], clamp)
        live = ids.reshape(-1).numpy() >= 0
        for path in paths:
            print_case("exact layer", shape, path, clamp)
            out = bfp8.fused_moe_block_fp8(hidden.to(dev()), ids.to(dev()), w.to(dev()), Wd.w13, Wd.w13_s, Wd.w2,
                                           Wd.w2_s, E=E, o=bfp8.opts(scale_fmt=bfp8.SCALE_UE8M0, clamp_limit=clamp,
                                                                     flags=PATH_FLAGS[path]))
            torch.cuda.synchronize()
            got = bf16_np(out)
            nd = int((got != ref).sum())
            print(f"  {path}: {nd} of {got.size} outputs differ", flush=True)
            assert nd == 0, f"{path}: first difference at {np.argwhere(got != ref)[0]}"
            if path in FIRST_STAGE:
                for fmt in (bfp8.SCALE_FP32, bfp8.SCALE_UE8M0):
                    # the hidden scales are exact powers of two in both formats
                    act = _stage0_act(path, hidden.to(dev()), ids.to(dev()), w.to(dev()), Wd, E, I, fmt, clamp)
                    assert np.array_equal(act[live], ref_act[live]), f"{path}: SwiGLU rows differ"


# Gaussian workloads: (name, M, E, k, H, I, fmt, clamp)
RANDOM = [
    ("decode_m1", 1, 256, 8, 7168, 256, bfp8.SCALE_FP32, math.inf),
    ("decode_m4_ue8m0_clamp", 4, 256, 8, 7168, 256, bfp8.SCALE_UE8M0, 7.0),
    ("h2560", 1, 64, 8, 2560, 256, bfp8.SCALE_FP32, math.inf),
    ("k16_h3200", 2, 64, 16, 3200, 256, bfp8.SCALE_UE8M0, 7.0),
    ("m6_i384", 6, 64, 8, 2048, 384, bfp8.SCALE_FP32, math.inf),
    ("m8_i512", 8, 64, 8, 1024, 512, bfp8.SCALE_UE8M0, 7.0),
    ("m1_i384", 1, 64, 8, 7168, 384, bfp8.SCALE_FP32, math.inf),
    ("tiny", 4, 8, 2, 256, 128, bfp8.SCALE_FP32, math.inf),
]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: c[0])
def test_gaussian_workload_elementwise(case):
    name, M, E, k, H, I, fmt, clamp = case
    c = synth.LayerCase(name, M=M, E=E, k=k, H=H, I=I, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev())
    for path in _paths(M, H, k, E, I):
        print_case("gaussian layer", name, path)
        if path in FIRST_STAGE:
            act = _stage0_act(path, hidden, ids, w, W, E, I, fmt, clamp)
            hid, ids_l, w_l, Wl = oracle_inputs_for_tokens(hidden, ids, w, W, list(range(M)), E)
            acc, mag, extra = gate_up_exact(hid, ids_l, Wl.w13, Wl.w13_s, k, fmt, mfma=path != "token")
            allowed = ActAllowed(acc, mag, H, clamp, extra, mfma=path != "token")
            amb, wide, nd = allowed.check(act, f"{name} {path} SwiGLU rows")
            print(f"  {path} SwiGLU rows: {nd} of {int(allowed.live.sum()) * I} differ from the oracle; "
                  f"{amb} within the fp32 error bound of a BF16 boundary ({wide} checked by interval)", flush=True)
        out = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E,
                                       o=bfp8.opts(scale_fmt=fmt, clamp_limit=clamp, flags=PATH_FLAGS[path]))
        torch.cuda.synchronize()
        assert_layer_elementwise(out, hidden, ids, w, W, fmt, clamp, E=E, what=f"  {name} {path} output",
                                 o=bfp8.opts(scale_fmt=fmt, clamp_limit=clamp, flags=PATH_FLAGS[path]))
