"""GPU parity (through the C ABI) of the W8A8 variant: per-row quantisation
and fused SwiGLU + per-row quantisation bit-exact against the oracle; the
channel-scaled grouped GEMM element by element within the fp32 and FP8 MFMA
bounds of tests/parity.py; the layer bit-exact on the exact-arithmetic
workload (dynamic and static scales) and within the stated normwise bound on
Gaussian inputs."""
import math

import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import LAYER_TOL, bf16_np, dev, normwise_err, print_case
from tests.parity import check_gemm, mfma_f8_error

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [128, 1024, 7168, 8192])
@pytest.mark.parametrize("fmt", [bfp8.SCALE_FP32, bfp8.SCALE_UE8M0])
@pytest.mark.parametrize("static", [0.0, 0.01, 1e-3])
def test_quant_rows_bit_exact(K, fmt, static):
    print_case("quant rows", K, fmt, static)
    g = torch.Generator().manual_seed(K)
    x = torch.randn(37, K, generator=g) * torch.logspace(-3, 2, 37).view(37, 1)
    x[3] = 0.0
    x = x.to(torch.bfloat16)
    q, s = bfp8.quant_fp8_rows(x.to(dev()), fmt, static)
    torch.cuda.synchronize()
    rq, rs = O.quant_fp8_rows(x, fmt, static)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("I", [256, 2048, 4096])
@pytest.mark.parametrize("fmt,clamp,static", [(bfp8.SCALE_FP32, math.inf, 0.0), (bfp8.SCALE_UE8M0, 7.0, 0.0),
                                               (bfp8.SCALE_FP32, 7.0, 0.004)])
def test_act_quant_rows_bit_exact(I, fmt, clamp, static):
    print_case("act quant rows", I, fmt, clamp, static)
    x, ids = synth.act_rows(130, I, 32, "w8a8_act", I)
    qd = torch.full((130, I), 0xAB, dtype=torch.uint8, device=dev())
    sd = torch.full((130,), -1.0, device=dev())
    bfp8.silu_and_mul_quant_fp8_rows(x.to(dev()), ids.to(dev()), None, 32, clamp, fmt, static, qd, sd)
    torch.cuda.synchronize()
    rq, rs = O.silu_and_mul_quant_fp8_rows(x, ids, None, 32, clamp, fmt, static,
                                           np.full((130, I), 0xAB, np.uint8), np.full(130, -1.0, np.float32))
    assert np.array_equal(qd.cpu().numpy(), rq)
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("M,E,k,N,K,block_m", [(1, 256, 8, 512, 7168, 16), (16, 16, 8, 2048, 2048, 32),
                                               (64, 16, 8, 1024, 768, 64),
                                               # 1, 3 and 5 K chunks (the K loop's remainders)
                                               (8, 8, 4, 256, 128, 16), (8, 8, 4, 256, 384, 64),
                                               (8, 8, 4, 256, 640, 32)])
def test_channel_gemm_elementwise(M, E, k, N, K, block_m):
    print_case("channel gemm", M, E, k, N, K, block_m)
    ids, _ = synth.uniform_routing(M, E, k, "w8a8_gemm", M)
    x = synth.hidden_states(M, K, "w8a8_gemm", M)
    aq, as_ = O.quant_fp8_rows(x, bfp8.SCALE_FP32)
    g = torch.Generator().manual_seed(M)
    B = (torch.randn(E, N, K, generator=g) * 0.02)
    bs = (B.abs().amax(-1) / 448.0).float()
    Bq = (B / bs[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    route = bfp8.moe_route_prepare(ids.to(dev()), 0, E, block_m)
    C = bfp8.moe_fp8_grouped_gemm_channel(torch.from_numpy(aq).to(dev()), torch.from_numpy(as_).to(dev()), k,
                                          Bq.to(dev()), bs.to(dev()), route, block_m, M * k)
    torch.cuda.synchronize()
    acc, mag = O.grouped_gemm_channel(aq, as_, k, Bq, bs, ids, 0, E, exact=True)
    extra = np.zeros_like(acc)
    Bn = Bq.numpy()
    for r, e in enumerate(ids.numpy().reshape(-1)):
        cs = np.repeat((float(as_[r // k]) * bs[e].numpy().astype(np.float64))[:, None], K // 128, axis=1)
        extra[r] = mfma_f8_error(aq[r // k], Bn[e], cs)
    amb, nd = check_gemm(bf16_np(C), acc, mag, K, "channel gemm", extra)
    print(f"  {nd} of {C.numel()} differ from the exact value's rounding, {amb} may", flush=True)


def _channel_weights(W, E, H, I, key):
    rng = np.random.default_rng(synth.seed_of(key) % (1 << 32))
    c13 = torch.from_numpy(np.exp2(rng.integers(-9, -6, (E, 2 * I))).astype(np.float32))
    c2 = torch.from_numpy(np.exp2(rng.integers(-9, -6, (E, H))).astype(np.float32))
    return c13, c2


W8A8_PATHS = {"token": bfp8.FLAG_LAYER_TOKEN, "general": bfp8.FLAG_LAYER_GENERAL}


def _w8a8_paths(M, H, k, E, I):
    out = []
    for name, flag in W8A8_PATHS.items():
        try:
            bfp8.fused_moe_stages(M, H, k, E, I, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL, flags=flag))
        except bfp8.BFP8MoEError:
            continue
        out.append((name, flag))
    return out


# (M, E, k, H, I): the few-token kernels (their W8A8 form: one scale per hidden
# row from all 8 hidden-row waves, one per SwiGLU row from its groups' maxima;
# H not a multiple of 1024 and 16 routes per token included) and the general path
@pytest.mark.parametrize("M,E,k,H,I", [(1, 16, 8, 7168, 256), (5, 16, 8, 2048, 512), (2, 24, 16, 2560, 128),
                                       (40, 24, 8, 1024, 256)])
# static scales: none; the hidden rows' (no value saturates); both, the SwiGLU
# rows saturating; both saturating (quotients past 448 clamp as quant_fp8's do)
@pytest.mark.parametrize("statics", [(0.0, 0.0), (0.25, 0.0), (0.25, 2.0 ** -6), (2.0 ** -6, 2.0 ** -6)])
def test_w8a8_layer_exact_workload(M, E, k, H, I, statics):
    print_case("w8a8 layer exact", M, E, k, H, I, statics)
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "w8a8_exact")
    c13, c2 = _channel_weights(W, E, H, I, "w8a8_exact")
    paths = _w8a8_paths(M, H, k, E, I)
    assert paths
    for clamp in (math.inf, 7.0):
        ref = O.fused_moe_w8a8(hidden, ids, w, W.w13, c13, W.w2, c2, scale_fmt=O.SCALE_UE8M0, a1_static=statics[0],
                               a2_static=statics[1], clamp=clamp)
        for name, flag in paths:
            o = bfp8.opts(scale_fmt=bfp8.SCALE_UE8M0, clamp_limit=clamp, weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL,
                          act_static_scale=statics[0], inter_static_scale=statics[1], flags=flag)
            out = bfp8.fused_moe_block_fp8(hidden.to(dev()), ids.to(dev()), w.to(dev()), W.w13.to(dev()),
                                           c13.to(dev()), W.w2.to(dev()), c2.to(dev()), E=E, o=o)
            torch.cuda.synchronize()
            got = bf16_np(out)
            nd = int((got != ref).sum())
            print(f"  {name}, clamp {clamp}: {nd} of {got.size} outputs differ", flush=True)
            assert nd == 0


@pytest.mark.parametrize("M,E,k,H,I", [(1, 64, 8, 7168, 256), (64, 32, 8, 4096, 768)])
def test_w8a8_layer_gaussian(M, E, k, H, I):
    print_case("w8a8 layer gaussian", M, E, k, H, I)
    c = synth.LayerCase("w8a8", M=M, E=E, k=k, H=H, I=I, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev())
    # per-channel scales from the block-quantised weights' rows: each row's
    # amax over its codes times its block scale, re-encoded per row
    w13f = (W.w13.view(torch.float8_e4m3fn).float() * W.w13_s.repeat_interleave(128, 1).repeat_interleave(128, 2))
    w2f = (W.w2.view(torch.float8_e4m3fn).float() * W.w2_s.repeat_interleave(128, 1).repeat_interleave(128, 2))
    s13 = (w13f.abs().amax(-1) / 448.0).clamp_min(1e-12)
    s2 = (w2f.abs().amax(-1) / 448.0).clamp_min(1e-12)
    q13 = (w13f / s13[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    q2 = (w2f / s2[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    used = torch.unique(ids).long()
    remap = torch.full((E,), -1, dtype=torch.int32, device=dev())
    remap[used] = torch.arange(used.numel(), dtype=torch.int32, device=dev())
    ids_l = remap[ids.long()]
    ref = O.fused_moe_w8a8(hidden.cpu(), ids_l.cpu(), w.cpu(), q13[used].cpu(), s13[used].cpu(), q2[used].cpu(),
                           s2[used].cpu())
    for name, flag in _w8a8_paths(M, H, k, E, I):
        o = bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL, flags=flag)
        out = bfp8.fused_moe_block_fp8(hidden, ids, w, q13, s13.contiguous(), q2, s2.contiguous(), E=E, o=o)
        torch.cuda.synchronize()
        err = normwise_err(bf16_np(out), ref)
        print(f"  {name}: normwise {err:.2e}", flush=True)
        assert err <= LAYER_TOL
