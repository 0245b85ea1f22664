"""GPU parity (through the C ABI) of the MXFP4-weight variant:

* the FP4 x FP8 MFMA's operand layout: with one non-zero weight element per
  row, every one of a 256-wide chunk's K positions selects its own activation
  and its own block's E8M0 scale, exactly;
* the grouped GEMM bit-exact against the oracle where every sum is exact in
  any order (integer E2M1 values, one scale per 128-wide group), and on
  random codes with a scale per 32-element block within the fp32 bound plus
  the MFMA's in-chunk cutting (tests.parity.mfma_f4f8_error: the FP8 form's
  model, which bounds every output seen);
* the layer, on the few-token path (VALU dot products of FP4 values widened
  to FP16) and on the general path, bit-exact on the exact-arithmetic
  workload (partial last row chunks, 16 routes per token, I = 512 included)
  and within the stated normwise bound on random weights."""
import math

import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import LAYER_TOL, bf16_np, dev, normwise_err, print_case
from tests.parity import SAFETY, U, bf16_bits_rne, bf16_candidates, depth, f32_of_bits, mfma_f4f8_error

pytestmark = pytest.mark.gpu


def _e4m3(v: float) -> int:
    c = int(torch.tensor([v]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    assert O.e4m3_decode(c) == v
    return c


def _gemm(aq, as_, k, W, Ws, ids, block_m=16):
    E = W.shape[0]
    route = bfp8.moe_route_prepare(ids.to(dev()), 0, E, block_m)
    C = bfp8.moe_mxfp4_grouped_gemm(torch.from_numpy(aq).to(dev()), torch.from_numpy(as_).to(dev()), k,
                                    W.to(dev()), Ws.to(dev()), route, block_m, ids.numel())
    torch.cuda.synchronize()
    return C


def test_operand_layout_and_block_scales():
    print_case("mxfp4 layout")
    K, N = 256, 256
    vals = [float(1 + (i % 7)) for i in range(K)]
    a = np.array([_e4m3(v) for v in vals], np.uint8)[None, :]
    a_s = np.ones((1, K // 128), np.float32)
    codes = torch.zeros(1, N, K, dtype=torch.uint8)
    codes[0, torch.arange(N), torch.arange(K)] = 2                       # element i of row i: 1.0
    ws = torch.full((1, N, K // 32), 127, dtype=torch.uint8)
    ws[0, torch.arange(N), torch.arange(K) // 32] = (127 + (torch.arange(K) % 5) - 2).to(torch.uint8)
    C = _gemm(a, a_s, 1, synth.pack_e2m1(codes), ws, torch.zeros(1, 1, dtype=torch.int32))
    got = C.float().cpu().numpy()[0]
    want = np.array([vals[i] * 2.0 ** ((i % 5) - 2) for i in range(K)])
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(int(i), float(got[i]), float(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("M,E,k,N,K,block_m", [(1, 4, 2, 256, 512, 16), (16, 8, 4, 512, 2048, 32),
                                               (40, 16, 8, 256, 1024, 64)])
def test_gemm_exact_integers(M, E, k, N, K, block_m):
    print_case("mxfp4 gemm exact", M, E, k, N, K, block_m)
    hidden, ids, _, W = synth.exact_mxfp4_layer_inputs(M, E, k, K, N // 2, "mx_gemm", M)
    aq, as_ = O.quant_fp8(hidden, O.SCALE_UE8M0)
    C = _gemm(aq, as_, k, W.w13, W.w13_s, ids, block_m)
    ref = O.grouped_gemm_mxfp4(aq, as_, k, W.w13, W.w13_s, ids, 0, E)
    live = (ids.reshape(-1) >= 0).numpy()
    got = bf16_np(C)
    nd = int((got[live] != ref[live]).sum())
    print(f"  {nd} of {got[live].size} differ", flush=True)
    assert nd == 0


@pytest.mark.parametrize("M,E,k,N,K,block_m", [(4, 8, 8, 512, 2048, 16), (64, 16, 8, 1024, 4096, 32),
                                               (128, 16, 8, 512, 1024, 64),
                                               # 1, 3 and 5 chunks of 256 (activation scales staged
                                               # from 4 groups of 128: not, then staged)
                                               (8, 8, 4, 256, 256, 32), (8, 8, 4, 256, 768, 16),
                                               (8, 8, 4, 256, 1280, 64)])
def test_gemm_random_codes_within_fp32_bound(M, E, k, N, K, block_m):
    print_case("mxfp4 gemm random", M, E, k, N, K, block_m)
    ids, _ = synth.uniform_routing(M, E, k, "mx_rand", M)
    aq, as_ = O.quant_fp8(synth.hidden_states(M, K, "mx_rand", M))
    W = synth.mxfp4_weights(E, K, N // 2, "mx_rand", M)
    C = _gemm(aq, as_, k, W.w13, W.w13_s, ids, block_m)
    acc, mag = O.grouped_gemm_mxfp4(aq, as_, k, W.w13, W.w13_s, ids, 0, E, exact=True)
    got = bf16_np(C)
    # every route at the small shapes, an even sample of 48 at the others
    R = ids.numel()
    rows = np.arange(R) if R <= 64 else np.linspace(0, R - 1, 48).astype(int)
    extra = np.stack([mfma_f4f8_error(aq[r // k], W.w13[e].numpy(), W.w13_s[e].numpy(), as_[r // k])
                      for r, e in ((r, int(ids.reshape(-1)[r])) for r in rows)])
    lo, hi = bf16_candidates(acc[rows], SAFETY * (depth(K) * U * mag[rows] + extra))
    g = f32_of_bits(got[rows])
    ok = (g >= f32_of_bits(lo)) & (g <= f32_of_bits(hi))
    nd = int((got[rows] != bf16_bits_rne(acc[rows])).sum())
    print(f"  {rows.size} routes checked: {int((~ok).sum())} of {ok.size} outside the bound, {nd} differ from the "
          f"exact value's rounding, {int((lo != hi).sum())} may", flush=True)
    assert ok.all()


MX_PATHS = {"token": bfp8.FLAG_LAYER_TOKEN, "general": bfp8.FLAG_LAYER_GENERAL}


def _mx_paths(M, H, k, E, I):
    """The paths that take this shape: (name, flags, first stage)."""
    out = []
    for name, flag in MX_PATHS.items():
        try:
            st = bfp8.fused_moe_stages(M, H, k, E, I, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4, flags=flag))
        except bfp8.BFP8MoEError:
            continue
        out.append((name, flag, st[0]))
    return out


# (M, E, k, H, I): few-token shapes (the decode widths, a row of 1,280 bytes
# whose last 1 KB chunk is a quarter filled, 16 routes per token, I = 512) and
# general-path ones
@pytest.mark.parametrize("M,E,k,H,I", [(1, 16, 8, 2048, 256), (1, 16, 8, 7168, 256), (1, 16, 8, 2560, 256),
                                       (5, 16, 8, 2048, 512), (3, 24, 16, 3072, 256), (40, 24, 8, 1024, 256)])
def test_layer_exact_workload(M, E, k, H, I):
    print_case("mxfp4 layer exact", M, E, k, H, I)
    hidden, ids, w, W = synth.exact_mxfp4_layer_inputs(M, E, k, H, I, "mx_layer")
    paths = _mx_paths(M, H, k, E, I)
    assert paths
    for clamp in (math.inf, 7.0):
        ref = O.fused_moe_mxfp4(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=O.SCALE_UE8M0, clamp=clamp)
        for name, flag, first in paths:
            o = bfp8.opts(scale_fmt=bfp8.SCALE_UE8M0, clamp_limit=clamp, weight_scale_mode=bfp8.WEIGHT_MXFP4,
                          flags=flag)
            out = bfp8.fused_moe_mxfp4(hidden.to(dev()), ids.to(dev()), w.to(dev()), W.w13.to(dev()),
                                       W.w13_s.to(dev()), W.w2.to(dev()), W.w2_s.to(dev()), E=E, o=o)
            torch.cuda.synchronize()
            got = bf16_np(out)
            nd = int((got != ref).sum())
            print(f"  {name} ({first}), clamp {clamp}: {nd} of {got.size} outputs differ", flush=True)
            assert nd == 0


@pytest.mark.parametrize("M,E,k,H,I", [(1, 32, 8, 4096, 256), (4, 64, 8, 7168, 256), (64, 32, 8, 2048, 768)])
def test_layer_random_weights(M, E, k, H, I):
    print_case("mxfp4 layer random", M, E, k, H, I)
    ids, w = synth.uniform_routing(M, E, k, "mx_layer_r", M)
    hidden = synth.hidden_states(M, H, "mx_layer_r", M)
    W = synth.mxfp4_weights(E, H, I, "mx_layer_r", M)
    auto = bfp8.fused_moe_stages(M, H, k, E, I, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4))
    if M <= 4:
        assert auto == ["token_gate_up_swiglu_mxfp4", "token_down_reduce_mxfp4"]
    else:
        assert auto == ["route_prepare_quant", "gate_up_gemm_mxfp4", "silu_and_mul_quant", "down_gemm_mxfp4",
                        "moe_reduce"]
    ref = O.fused_moe_mxfp4(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s)
    for name, flag, _ in _mx_paths(M, H, k, E, I):
        o = bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4, flags=flag)
        out = bfp8.fused_moe_mxfp4(hidden.to(dev()), ids.to(dev()), w.to(dev()), W.w13.to(dev()),
                                   W.w13_s.to(dev()), W.w2.to(dev()), W.w2_s.to(dev()), E=E, o=o)
        torch.cuda.synchronize()
        err = normwise_err(bf16_np(out), ref)
        print(f"  {name}: normwise {err:.2e}", flush=True)
        assert err <= LAYER_TOL


def test_mxfp4_layer_small_shape():
    print_case("mxfp4 layer small")
    M, E, k, H, I = 4, 8, 2, 256, 256
    ids, w = synth.uniform_routing(M, E, k, "mx_small")
    hidden = synth.hidden_states(M, H, "mx_small")
    W = synth.mxfp4_weights(E, H, I, "mx_small")
    out = bfp8.fused_moe_mxfp4(hidden.to(dev()), ids.to(dev()), w.to(dev()), W.w13.to(dev()), W.w13_s.to(dev()),
                               W.w2.to(dev()), W.w2_s.to(dev()), E=E)
    torch.cuda.synchronize()
    ref = O.fused_moe_mxfp4(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s)
    assert normwise_err(bf16_np(out), ref) <= LAYER_TOL
