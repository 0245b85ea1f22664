"""GPU parity (through the C ABI) for quant_fp8, silu_and_mul,
silu_and_mul_quant_fp8 and moe_reduce: bit-exact against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import bf16_np, dev, print_case

pytestmark = pytest.mark.gpu

ALL_BF16 = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


def _bits(t):
    return bf16_np(t)


@pytest.mark.parametrize("fmt", [bfp8.SCALE_FP32, bfp8.SCALE_UE8M0])
@pytest.mark.parametrize("rows,K", [(1, 128), (3, 384), (17, 7168), (64, 4096), (1000, 256)])
def test_quant_fp8_bitexact(rows, K, fmt):
    print_case("quant_fp8", rows, K, fmt)
    x = synth.hidden_states(rows, K, "quant_test", rows, K)
    x[0, :128] = 0  # an all-zero group
    q, s = bfp8.quant_fp8(x.to(dev()), fmt)
    torch.cuda.synchronize()
    rq, rs = O.quant_fp8(x, fmt)
    assert (q.cpu().numpy() == rq).all()
    assert (s.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("fmt", [bfp8.SCALE_FP32, bfp8.SCALE_UE8M0])
def test_quant_fp8_every_bf16_pattern(fmt):
    # 512 rows x 128: every finite BF16 bit pattern once (zeros of both signs,
    # subnormals, the extremes), shuffled so groups mix magnitudes.  Infinities
    # and NaNs are outside the contract: a group holding +-inf divides inf by
    # inf, and the sign of the NaN that makes is not fixed by IEEE (x86 and the
    # GPU differ), so they are replaced by zeros here.
    print_case("quant_fp8 all patterns", fmt)
    g = torch.Generator().manual_seed(5)
    x = ALL_BF16[torch.randperm(1 << 16, generator=g)].reshape(512, 128).contiguous()
    x = torch.where(torch.isfinite(x.float()), x, torch.zeros_like(x))
    q, s = bfp8.quant_fp8(x.to(dev()), fmt)
    torch.cuda.synchronize()
    rq, rs = O.quant_fp8(x, fmt)
    assert (q.cpu().numpy() == rq).all()
    assert (s.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("I", [128, 4096])
@pytest.mark.parametrize("clamp", [math.inf, 7.0, 7.1])
def test_silu_and_mul_exhaustive_gate(clamp, I):
    # every BF16 gate value (finite or not) against up = 1 and against random ups;
    # a clamp limit that is not a BF16 value (7.1) gives gates that are not
    # either.  512 rows of width 128 take the fp64 exp; width 4096 (every gate
    # value 32 times, 16384 groups) takes the table
    print_case("silu_and_mul exhaustive", clamp, I)
    gates = ALL_BF16.reshape(512, 128).repeat(1, I // 128)
    for up_kind in ("one", "random"):
        if up_kind == "one":
            ups = torch.ones(512, I, dtype=torch.bfloat16)
        else:
            ups = (torch.randn(512, I, generator=torch.Generator().manual_seed(2)) * 4).to(torch.bfloat16)
        x = torch.cat([gates, ups], dim=1).contiguous()
        out = bfp8.silu_and_mul(x.to(dev()), clamp)
        torch.cuda.synchronize()
        ref = O.silu_and_mul(x, clamp)
        got = _bits(out)
        # NaN outputs (from NaN gates/ups): compare as NaN-ness, bits elsewhere
        rf = (ref.astype(np.uint32) << 16).view(np.float32)
        gf = (got.astype(np.uint32) << 16).view(np.float32)
        both_nan = np.isnan(rf) & np.isnan(gf)
        assert ((got == ref) | both_nan).all(), np.argwhere(~((got == ref) | both_nan))[:5]


@pytest.mark.parametrize("clamp", [math.inf, 7.0, 7.1])
def test_act_quant_filtered_every_bf16_gate(clamp):
    # every BF16 gate value, 32 times, through the filtered act + quant (row
    # ids, all rows local: 16384 groups of 128, so the kernel whose exp table
    # sits in LDS); codes and scales bit-exact
    print_case("act_quant filtered exhaustive", clamp)
    I = 4096
    gates = ALL_BF16.reshape(512, 128).repeat(1, I // 128)
    # ups within +-0.5, so that every product stays finite; the two rows of
    # NaN and inf gate codes are dropped (their groups' scales are not finite)
    ups = (torch.randn(512, I, generator=torch.Generator().manual_seed(3)) * 0.2).clamp(-0.5, 0.5)
    x = torch.cat([gates, ups.to(torch.bfloat16)], dim=1).contiguous()
    x = x[torch.isfinite(x.float()).all(dim=1)].contiguous()
    rows = x.shape[0]
    ids = torch.zeros(rows, dtype=torch.int32)
    qs = torch.full((rows, I), 0x5A, dtype=torch.uint8)
    ss = torch.full((rows, I // 128), -3.0)
    q, s = bfp8.silu_and_mul_quant_fp8(x.to(dev()), q=qs.to(dev()), scales=ss.to(dev()), row_expert_ids=ids.to(dev()),
                                       expert_map=None, E=4, clamp_limit=clamp, scale_fmt=bfp8.SCALE_FP32)
    torch.cuda.synchronize()
    rq, rs = O.silu_and_mul_quant_fp8(x, ids, None, 4, clamp, bfp8.SCALE_FP32, q_init=qs.numpy(), s_init=ss.numpy())
    assert (q.cpu().numpy() == rq).all()
    assert (s.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("fmt", [bfp8.SCALE_FP32, bfp8.SCALE_UE8M0])
@pytest.mark.parametrize("I", [512, 2048])
@pytest.mark.parametrize("rows", [8, 128, 1024])
@pytest.mark.parametrize("mode", ["none", "ids", "map"])
def test_act_quant_regression_grid(I, rows, mode, fmt):
    # widths 512/2048 x 8/128/1024 rows x {no filter, ids, expert map} x {fp32, ue8m0}
    print_case("act_quant grid", I, rows, mode, fmt)
    E = 288
    x, ids = synth.act_rows(rows, I, E, "grid", I, rows)
    emap = torch.arange(E, dtype=torch.int32)
    emap[torch.randperm(E, generator=torch.Generator().manual_seed(rows))[: E // 3]] = -1
    qs = torch.full((rows, I), 0xA5, dtype=torch.uint8)
    ss = torch.full((rows, I // 128), -7.0)
    args = dict(row_expert_ids=None if mode == "none" else ids.to(dev()),
                expert_map=emap.to(dev()) if mode == "map" else None, E=E, clamp_limit=7.0, scale_fmt=fmt)
    q, s = bfp8.silu_and_mul_quant_fp8(x.to(dev()), q=qs.to(dev()), scales=ss.to(dev()), **args)
    torch.cuda.synchronize()
    rq, rs = O.silu_and_mul_quant_fp8(x, None if mode == "none" else ids, emap if mode == "map" else None, E,
                                      7.0, fmt, q_init=qs.numpy(), s_init=ss.numpy())
    assert (q.cpu().numpy() == rq).all()
    assert (s.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("tokens", [1, 64, 1024])
def test_act_quant_expert_parallel_workload(tokens):
    # 8-way expert parallelism: top-k 6 rows, width 2048, 32 of 256 experts
    # local through the expert map; the 7/8 non-local rows keep their
    # sentinel bytes, the local ones are bit-exact
    print_case("act_quant ep8", tokens)
    x, ids, emap = synth.ep_act_inputs(tokens, "ep8")
    rows, I = x.shape[0], synth.EP_I
    qs = torch.full((rows, I), 0x3C, dtype=torch.uint8)
    ss = torch.full((rows, I // 128), -5.0)
    q, s = bfp8.silu_and_mul_quant_fp8(x.to(dev()), q=qs.to(dev()), scales=ss.to(dev()), row_expert_ids=ids.to(dev()),
                                       expert_map=emap.to(dev()), E=synth.EP_E, clamp_limit=7.0,
                                       scale_fmt=bfp8.SCALE_UE8M0)
    torch.cuda.synchronize()
    rq, rs = O.silu_and_mul_quant_fp8(x, ids, emap, synth.EP_E, 7.0, bfp8.SCALE_UE8M0, q_init=qs.numpy(),
                                      s_init=ss.numpy())
    assert (q.cpu().numpy() == rq).all()
    assert (s.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all()
    live = (emap[ids.long()] >= 0).numpy()
    assert 0 < live.sum() < rows or rows == 6


@pytest.mark.parametrize("tokens", list(synth.ACT_TOKENS))
def test_act_quant_workload_and_two_kernel_invariant(tokens):
    # the clamped UE8M0 workload: rows = tokens x 8, I = 512, E = 288, ~10 % masked
    rows = tokens * 8
    print_case("act_quant workload", rows)
    x, ids = synth.act_rows(rows, synth.ACT_I, synth.ACT_E, "act_quant", tokens)
    xd, idd = x.to(dev()), ids.to(dev())
    sentinel_q = torch.full((rows, synth.ACT_I), 0x5A, dtype=torch.uint8, device=dev())
    sentinel_s = torch.full((rows, synth.ACT_I // 128), 3.0, device=dev())
    q, s = bfp8.silu_and_mul_quant_fp8(xd, idd, None, synth.ACT_E, synth.ACT_CLAMP, bfp8.SCALE_UE8M0,
                                       q=sentinel_q.clone(), scales=sentinel_s.clone())
    # the unfused two-kernel path on the GPU: silu_and_mul -> BF16 -> quant_fp8
    act = bfp8.silu_and_mul(xd, synth.ACT_CLAMP)
    q2, s2 = bfp8.quant_fp8(act, bfp8.SCALE_UE8M0)
    torch.cuda.synchronize()
    live = (ids >= 0).numpy()
    qn, sn, q2n, s2n = q.cpu().numpy(), s.cpu().numpy(), q2.cpu().numpy(), s2.cpu().numpy()
    # fused == quant_fp8(silu_and_mul(x)) on live rows, codes and scales
    assert (qn[live] == q2n[live]).all() and (sn[live].view(np.uint32) == s2n[live].view(np.uint32)).all()
    # masked rows untouched
    assert (qn[~live] == 0x5A).all() and (sn[~live] == 3.0).all()
    rq, rs = O.silu_and_mul_quant_fp8(x, ids, None, synth.ACT_E, synth.ACT_CLAMP, O.SCALE_UE8M0,
                                      q_init=np.full((rows, synth.ACT_I), 0x5A, np.uint8),
                                      s_init=np.full((rows, synth.ACT_I // 128), 3.0, np.float32))
    assert (qn == rq).all() and (sn.view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("M,k,H", [(1, 8, 7168), (5, 8, 256), (128, 8, 4096), (33, 2, 1024), (7, 1, 128)])
def test_moe_reduce_bitexact(M, k, H):
    print_case("moe_reduce", M, k, H)
    y = synth.hidden_states(M * k, H, "reduce", M, k, H)
    ids, w = synth.uniform_routing(M, 64, k, "reduce", M, k, H)
    ids[0, 0] = -1
    if M > 2:
        ids[2, :] = 70  # outside [0, 64): the token has no live route -> +0
    out = bfp8.moe_reduce(y.to(dev()), w.to(dev()), ids.to(dev()), 0, 64)
    torch.cuda.synchronize()
    ref = O.moe_reduce(y, w, ids, 0, 64)
    assert (bf16_np(out) == ref).all()
    out2 = bfp8.moe_reduce(y.to(dev()), w.to(dev()))
    torch.cuda.synchronize()
    assert (bf16_np(out2) == O.moe_reduce(y, w)).all()


def test_zero_rows():
    # empty inputs: every elementwise entry point accepts zero rows and writes nothing
    print_case("zero rows")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=dev())
    q, s = bfp8.quant_fp8(x)
    assert tuple(q.shape) == (0, 256) and tuple(s.shape) == (0, 2)
    gu = torch.empty(0, 512, dtype=torch.bfloat16, device=dev())
    assert tuple(bfp8.silu_and_mul(gu).shape) == (0, 256)
    q, s = bfp8.silu_and_mul_quant_fp8(gu, clamp_limit=7.0)
    assert tuple(q.shape) == (0, 256)
    y = torch.empty(0, 256, dtype=torch.bfloat16, device=dev())
    out = bfp8.moe_reduce(y, torch.empty(0, 2, device=dev()))
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 256)
