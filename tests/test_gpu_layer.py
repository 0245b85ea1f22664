"""GPU parity (through the C ABI) for the whole layer, fused_moe_block_fp8,
on every layer workload: every GPU output must lie within the element-wise
bound of tests/parity.py around the oracle's (all tokens where the oracle is
quick, a seeded sample of tokens at the large sizes; the normwise 2e-2 bound
holds too), repeated calls must be bit-identical, and each forced
implementation must pass the same check."""
import math

import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import assert_layer_elementwise, bf16_np, dev, print_case

pytestmark = pytest.mark.gpu

# tokens the oracle evaluates per workload (None = all)
SAMPLE = {"tiny": None, "decode_m1": None, "decode_m4": None, "decode_m16": None, "decode_m32": 16,
          "small_m128": 12, "small_m512": 12, "large_m2048": 12}


def _inputs(case, instance=0):
    c = synth.LAYER_CASES[case]
    hidden, ids, w, W = synth.layer_inputs(c, instance, device=dev())
    return c, hidden, ids, w, W


def _run(c, hidden, ids, w, W, **kw):
    o = bfp8.opts(**kw)
    out = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E, o=o)
    torch.cuda.synchronize()
    return out


def _tokens(case, M):
    n = SAMPLE[case]
    if n is None or n >= M:
        return list(range(M))
    g = torch.Generator().manual_seed(M)
    return sorted(torch.randperm(M, generator=g)[:n].tolist())


@pytest.mark.parametrize("case", list(SAMPLE))
def test_layer_matches_oracle(case):
    print_case("layer", case)
    c, hidden, ids, w, W = _inputs(case)
    toks = _tokens(case, c.M)
    out = _run(c, hidden, ids, w, W, scale_fmt=c.scale_fmt, clamp_limit=c.clamp)
    assert_layer_elementwise(out, hidden, ids, w, W, c.scale_fmt, c.clamp, tokens=toks, E=c.E, what=case)
    # determinism: a second call gives the same bits
    out2 = _run(c, hidden, ids, w, W, scale_fmt=c.scale_fmt, clamp_limit=c.clamp)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


PATHS = [bfp8.FLAG_LAYER_GENERAL, bfp8.FLAG_LAYER_DECODE, bfp8.FLAG_LAYER_TOKEN]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", ["tiny", "decode_m1", "decode_m4"])
@pytest.mark.parametrize("fmt,clamp", [(bfp8.SCALE_FP32, math.inf), (bfp8.SCALE_UE8M0, 7.0)])
def test_layer_paths_fmt_clamp(case, path, fmt, clamp):
    print_case("layer path", case, path, fmt, clamp)
    c, hidden, ids, w, W = _inputs(case, 1)
    if path == bfp8.FLAG_LAYER_TOKEN and c.M > 32:
        with pytest.raises(bfp8.BFP8MoEError) as ei:
            _run(c, hidden, ids, w, W, flags=path)
        assert ei.value.status == 2  # unsupported: the few-token path takes at most 32 tokens
        return
    out = _run(c, hidden, ids, w, W, scale_fmt=fmt, clamp_limit=clamp, flags=path)
    assert_layer_elementwise(out, hidden, ids, w, W, fmt, clamp, E=c.E, what=f"{case} path {path}",
                             o=bfp8.opts(scale_fmt=fmt, clamp_limit=clamp, flags=path))


@pytest.mark.parametrize("path", PATHS)
def test_one_token_masked_and_duplicate_experts(path):
    # one token whose routes include masked ids (-1, out of range) and an
    # expert chosen twice: every path must agree with the oracle
    print_case("one token masked/duplicate", path)
    c = synth.LAYER_CASES["decode_m1"]
    hidden, ids, w, W = synth.layer_inputs(c, 5, device=dev())
    ids = ids.clone()
    ids[0, 2] = -1
    ids[0, 5] = 999
    ids[0, 6] = ids[0, 1]
    used = sorted(set(ids[ids >= 0].tolist()) & set(range(c.E)))
    for e in used:
        if e not in W.real:
            cw, sw = synth.block_fp8_weight(2 * c.I, c.H, "dup", e, device=dev())
            W.w13[e].copy_(cw); W.w13_s[e].copy_(sw)
            cw, sw = synth.block_fp8_weight(c.H, c.I, "dup2", e, device=dev())
            W.w2[e].copy_(cw); W.w2_s[e].copy_(sw)
    out = _run(c, hidden, ids, w, W, flags=path)
    assert_layer_elementwise(out, hidden, ids, w, W, c.scale_fmt, c.clamp, E=c.E, what=f"masked/duplicate {path}",
                             o=bfp8.opts(flags=path))


def test_workspace_shared_across_paths():
    # one workspace, filled with NaN bytes first (its contents need no
    # initialisation), used by the one-token, small-batch and general paths in
    # turn, twice
    print_case("workspace shared")
    c = synth.LAYER_CASES["decode_m1"]
    hidden, ids, w, W = synth.layer_inputs(c, 6, device=dev())
    sizes = [bfp8.fused_moe_workspace_size(1, c.H, c.k, c.E, c.I, bfp8.opts(flags=f)) for f in PATHS]
    ws = torch.full((max(sizes),), 0xFF, dtype=torch.uint8, device=dev())
    for _ in range(2):
        for f in [bfp8.FLAG_LAYER_TOKEN, bfp8.FLAG_LAYER_GENERAL, bfp8.FLAG_LAYER_DECODE, bfp8.FLAG_LAYER_TOKEN]:
            out = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                           o=bfp8.opts(flags=f), ws=ws)
            torch.cuda.synchronize()
            assert_layer_elementwise(out, hidden, ids, w, W, c.scale_fmt, c.clamp, E=c.E, what=f"shared ws {f}",
                                     o=bfp8.opts(flags=f))


@pytest.mark.parametrize("path", PATHS)
def test_stages_run_one_at_a_time(path):
    # BFP8MOE_FLAG_ONLY_STAGE: the stages of a path launched one by one on one
    # workspace give the whole call's output bit for bit, and a later stage
    # alone reads what a whole call left in the workspace
    print_case("stages one at a time", path)
    c = synth.LAYER_CASES["decode_m1"]
    hidden, ids, w, W = synth.layer_inputs(c, 7, device=dev())
    o = bfp8.opts(flags=path)
    n = len(bfp8.fused_moe_stages(1, c.H, c.k, c.E, c.I, o))
    ws = torch.empty(bfp8.fused_moe_workspace_size(1, c.H, c.k, c.E, c.I, o), dtype=torch.uint8, device=dev())
    whole = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E, o=o, ws=ws)
    out = torch.zeros_like(whole)
    for s_ in range(n):
        bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                 o=bfp8.opts(flags=path | bfp8.FLAG_ONLY_STAGE(s_)), ws=ws, out=out)
    last = torch.zeros_like(whole)
    bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                             o=bfp8.opts(flags=path | bfp8.FLAG_ONLY_STAGE(n - 1)), ws=ws, out=last)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), whole.view(torch.int16))
    assert torch.equal(last.view(torch.int16), whole.view(torch.int16))


@pytest.mark.parametrize("case", ["decode_m16", "decode_m32"])
def test_few_token_path_at_its_limits(case):
    # the few-token path forced at 16 and 32 tokens (each route reads its
    # expert's rows; tokens share experts), sampled tokens against the oracle
    print_case("few-token path", case)
    c, hidden, ids, w, W = _inputs(case, 2)
    toks = _tokens(case, c.M)
    out = _run(c, hidden, ids, w, W, scale_fmt=c.scale_fmt, clamp_limit=c.clamp, flags=bfp8.FLAG_LAYER_TOKEN)
    assert_layer_elementwise(out, hidden, ids, w, W, c.scale_fmt, c.clamp, tokens=toks, E=c.E, what=case,
                             o=bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN))


def test_one_token_local_slice():
    # one token under expert parallelism: only the routes whose expert lies in
    # [offset, offset + L) count (the others are skipped by both kernels, on a
    # NaN-filled workspace), and a token with no local route gives zeros
    print_case("one token local slice")
    c = synth.LayerCase("tok_slice", M=1, E=64, k=8, H=2048, I=256, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 4, device=dev())
    off, L = 16, 24
    ids = ids.clone()
    ids[0] = torch.tensor([3, 17, 40, 63, 20, -1, 39, 16], dtype=ids.dtype)
    Wl = synth.MoEWeights(W.w13[off:off + L].contiguous(), W.w13_s[off:off + L].contiguous(),
                          W.w2[off:off + L].contiguous(), W.w2_s[off:off + L].contiguous())
    for e in (17, 20, 39, 16):
        if W.real is not None and e not in W.real:
            cw, sw = synth.block_fp8_weight(2 * c.I, c.H, "slice", e, device=dev())
            Wl.w13[e - off].copy_(cw); Wl.w13_s[e - off].copy_(sw)
            cw, sw = synth.block_fp8_weight(c.H, c.I, "slice2", e, device=dev())
            Wl.w2[e - off].copy_(cw); Wl.w2_s[e - off].copy_(sw)
    o = bfp8.opts(expert_offset=off, local_num_experts=L, flags=bfp8.FLAG_LAYER_TOKEN)
    need = bfp8.fused_moe_workspace_size(1, c.H, c.k, c.E, c.I, o)
    for case_ids in (ids, torch.full_like(ids, 5)):
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev())
        out = bfp8.fused_moe_block_fp8(hidden, case_ids, w, Wl.w13, Wl.w13_s, Wl.w2, Wl.w2_s, E=c.E, o=o, ws=ws)
        torch.cuda.synchronize()
        got = bf16_np(out)
        if (case_ids == 5).all():
            assert (got == 0).all()
        else:
            assert_layer_elementwise(out, hidden, case_ids, w, Wl, c.scale_fmt, c.clamp, E=c.E, expert_offset=off,
                                     L=L, what="one token local slice", o=o)


@pytest.mark.parametrize("path", [bfp8.FLAG_LAYER_GENERAL, bfp8.FLAG_LAYER_DECODE, bfp8.FLAG_LAYER_TOKEN])
def test_layer_masked_routes_and_local_slice(path):
    # ids outside the local slice [offset, offset + L) are skipped; a token
    # whose routes are all non-local gives zeros
    print_case("layer slice", path)
    c = synth.LAYER_CASES["tiny"]
    hidden, ids, w, W = synth.layer_inputs(c, 3, device=dev())
    ids = ids.clone()
    ids[0, 0] = -1
    ids[1, :] = 9  # beyond E: masked
    off, L = 2, 4
    Wl = synth.MoEWeights(W.w13[off:off + L].contiguous(), W.w13_s[off:off + L].contiguous(),
                          W.w2[off:off + L].contiguous(), W.w2_s[off:off + L].contiguous())
    out = bfp8.fused_moe_block_fp8(hidden, ids, w, Wl.w13, Wl.w13_s, Wl.w2, Wl.w2_s, E=c.E,
                                   o=bfp8.opts(expert_offset=off, local_num_experts=L, flags=path))
    torch.cuda.synchronize()
    got = bf16_np(out)
    assert (got[1] == 0).all()
    assert_layer_elementwise(out, hidden, ids, w, Wl, c.scale_fmt, c.clamp, E=c.E, expert_offset=off, L=L,
                             what=f"tiny slice {path}",
                             o=bfp8.opts(expert_offset=off, local_num_experts=L, flags=path))


def test_layer_rejects_bad_arguments():
    print_case("layer bad args")
    c, hidden, ids, w, W = _inputs("tiny")
    with pytest.raises(bfp8.BFP8MoEError):
        _run(c, hidden, ids, w, W, expert_offset=6, local_num_experts=4)  # slice beyond E
    with pytest.raises(bfp8.BFP8MoEError):
        _run(c, hidden, ids, w, W, block_m=24)
    small = torch.empty(16, dtype=torch.uint8, device=dev())
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E, ws=small)


# one-token shapes other than the decode workload: W13 rows of 1 to 8 loads,
# I = 128, 256 and 512 (1 KB W2 units of 8, 4 and 2 rows), down workgroups of
# 8 to 32 rows
TOKEN_SHAPES = [
    synth.LayerCase("tok_h256_i128_k2", M=1, E=8, k=2, H=256, I=128, routing="uniform"),
    synth.LayerCase("tok_h2048_i128_k4", M=1, E=16, k=4, H=2048, I=128, routing="uniform"),
    synth.LayerCase("tok_h4096_i128_k8", M=1, E=64, k=8, H=4096, I=128, routing="uniform"),
    synth.LayerCase("tok_h3072_i512_k3", M=1, E=32, k=3, H=3072, I=512, routing="uniform"),
    synth.LayerCase("tok_h8192_i256_k8", M=1, E=32, k=8, H=8192, I=256, routing="uniform"),
]


@pytest.mark.parametrize("c", TOKEN_SHAPES, ids=lambda c: c.name)
def test_one_token_shapes(c):
    print_case("one-token shape", c.name)
    assert bfp8.fused_moe_stages(1, c.H, c.k, c.E, c.I, bfp8.opts()) == ["token_gate_up_swiglu",
                                                                        "token_down_reduce"]
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev())
    out = _run(c, hidden, ids, w, W, scale_fmt=bfp8.SCALE_UE8M0, clamp_limit=7.0, flags=bfp8.FLAG_LAYER_TOKEN)
    assert_layer_elementwise(out, hidden, ids, w, W, bfp8.SCALE_UE8M0, 7.0, E=c.E, what=c.name,
                             o=bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN))


def test_one_token_grid_changes_on_one_workspace():
    # launches with different grids share one workspace
    print_case("one-token grid changes")
    cases = [TOKEN_SHAPES[0], synth.LAYER_CASES["decode_m1"], TOKEN_SHAPES[1], TOKEN_SHAPES[0]]
    data = []
    for c in dict((c.name, c) for c in cases).values():
        hidden, ids, w, W = synth.layer_inputs(c, 2, device=dev())
        data.append((c.name, (c, hidden, ids, w, W)))
    data = dict(data)
    need = max(bfp8.fused_moe_workspace_size(1, c.H, c.k, c.E, c.I, bfp8.opts()) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for _ in range(2):
        for c in cases:
            c, hidden, ids, w, W = data[c.name]
            out = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                           o=bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN), ws=ws)
            torch.cuda.synchronize()
            assert_layer_elementwise(out, hidden, ids, w, W, c.scale_fmt, c.clamp, E=c.E, what=c.name,
                                     o=bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN))


@pytest.mark.parametrize("path", [0] + PATHS)
def test_layer_zero_tokens(path):
    # M = 0: nothing to do, every path returns an empty output without error
    print_case("layer zero tokens", path)
    c = synth.LAYER_CASES["tiny"]
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev())
    out = bfp8.fused_moe_block_fp8(hidden[:0], ids[:0], w[:0], W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                   o=bfp8.opts(flags=path))
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, c.H)


# more routes than top-8 on the few-token path (its down kernel is built for 8
# and for 16 routes per token), among them the shape of 8 routed experts plus
# a shared expert of width 2048 split into 8 pseudo-experts of width 256 that
# every token takes with weight 1 (experts 256..263)
@pytest.mark.parametrize("M,E,k,H,I", [(1, 264, 16, 7168, 256), (3, 64, 12, 2048, 512), (2, 40, 9, 1024, 128)])
def test_token_path_more_routes(M, E, k, H, I):
    print_case("token path k", M, E, k, H, I)
    if E == 264:
        rid, rw = synth.uniform_routing(M, 256, 8, "k16", M)
        ids = torch.cat([rid, torch.arange(256, 264, dtype=torch.int32).expand(M, 8)], dim=1).contiguous()
        w = torch.cat([rw, torch.ones(M, 8)], dim=1).contiguous()
    else:
        ids, w = synth.uniform_routing(M, E, k, "k16", M)
    W = synth.moe_weights(E, H, I, "k16", M, experts=np.unique(ids.numpy()).tolist(), device=dev())
    hidden = synth.hidden_states(M, H, "k16", M).to(dev())
    o = bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN)
    assert bfp8.fused_moe_stages(M, H, k, E, I, o)[0] == "token_gate_up_swiglu"
    out = bfp8.fused_moe_block_fp8(hidden, ids.to(dev()), w.to(dev()), W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o)
    gen = bfp8.fused_moe_block_fp8(hidden, ids.to(dev()), w.to(dev()), W.w13, W.w13_s, W.w2, W.w2_s, E=E,
                                   o=bfp8.opts(flags=bfp8.FLAG_LAYER_GENERAL))
    torch.cuda.synchronize()
    for o_, what, f in ((out, "few tokens", bfp8.FLAG_LAYER_TOKEN), (gen, "general", bfp8.FLAG_LAYER_GENERAL)):
        assert_layer_elementwise(o_, hidden.cpu(), ids, w, W, bfp8.SCALE_FP32, math.inf, E=E,
                                 what=f"k={k} {what}", o=bfp8.opts(flags=f))
