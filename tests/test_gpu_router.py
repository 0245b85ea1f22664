"""GPU parity (through the C ABI) for the single-group top-k router: expert
ids bit-exact against the CPU oracle, weights within one fp32 ulp (both sides
form them in fp64 and round once; the exp and the sum order may differ in the
last fp64 bit)."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import assert_layer_elementwise, dev, print_case

pytestmark = pytest.mark.gpu

# (M, E, k): decode and prefill shapes of the layer's configurations (256 and
# 512 experts, top-8), a width that is not a multiple of 64, k = E, the
# largest E and k, one expert, and ragged token counts; from 8,192 tokens with
# E <= 256 and k <= 16 the 16-lanes-per-token kernel runs (its largest k, a
# width that is not a multiple of 16, token counts that leave rows idle)
SHAPES = [(1, 256, 8), (7, 256, 8), (2048, 512, 8), (33, 64, 6), (5, 72, 6), (4, 8, 8), (3, 1024, 64),
          (9, 1, 1), (130, 160, 2), (1000, 256, 8), (4099, 256, 8), (8200, 256, 8), (8192, 200, 16),
          (8259, 256, 1)]


def ulps(a, b):
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    return np.abs(a - b) / np.spacing(np.abs(b).astype(np.float32)).astype(np.float64)


def check(lg, k, score_fn, bias=None, renorm=True, scale=1.0):
    ids, w = bfp8.router_topk(lg.to(dev()), k, score_fn, None if bias is None else bias.to(dev()), renorm, scale)
    torch.cuda.synchronize()
    rid, rw = O.router_topk(lg, k, score_fn, bias, renorm, scale)
    assert (ids.cpu().numpy() == rid).all(), np.argwhere(ids.cpu().numpy() != rid)[:5]
    assert ulps(w.cpu().numpy(), rw).max() <= 1.0


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("score_fn", [bfp8.SCORE_SOFTMAX, bfp8.SCORE_SIGMOID])
@pytest.mark.parametrize("M,E,k", SHAPES)
def test_router_parity(M, E, k, score_fn, renorm):
    print_case("router", M, E, k, score_fn, renorm)
    # BF16-valued logits (equal values within a token are common) and plain fp32 ones
    for bf16_valued in (True, False):
        lg = synth.router_logits(M, E, "router", bf16_valued, std=2.0, bf16_valued=bf16_valued)
        bias = synth.router_bias(E, "router", std=0.1) if score_fn == bfp8.SCORE_SIGMOID else None
        check(lg, k, score_fn, bias, renorm, 2.5 if score_fn == bfp8.SCORE_SIGMOID else 1.0)
        if bias is not None:
            check(lg, k, score_fn, None, renorm)


def test_router_edge_values():
    print_case("router edge values")
    # all equal, signed zeros, infinities, logits near +-800 (exp without the
    # max subtracted over- or underflows), huge sigmoid arguments
    lg = torch.zeros(8, 96)
    lg[1, 10] = -0.0
    lg[1, 20] = 1.0
    lg[2] = torch.linspace(-800, 800, 96)
    lg[3, :] = float("-inf")
    lg[3, 50] = 0.0
    lg[4, 7] = float("inf")
    lg[5] = 800.0 + torch.randn(96, generator=torch.Generator().manual_seed(3))
    lg[6] = -800.0 + torch.randn(96, generator=torch.Generator().manual_seed(4))
    lg[7, ::2] = -0.0
    for score_fn in (bfp8.SCORE_SOFTMAX, bfp8.SCORE_SIGMOID):
        ids, _ = bfp8.router_topk(lg.to(dev()), 8, score_fn)
        torch.cuda.synchronize()
        rid, _ = O.router_topk(lg, 8, score_fn)
        assert (ids.cpu().numpy() == rid).all()
    ids, w = bfp8.router_topk(lg[[0, 1, 2, 5, 6, 7]].contiguous().to(dev()), 8)
    torch.cuda.synchronize()
    rid, rw = O.router_topk(lg[[0, 1, 2, 5, 6, 7]], 8)
    assert (ids.cpu().numpy() == rid).all() and ulps(w.cpu().numpy(), rw).max() <= 1.0
    assert ids[0].tolist() == list(range(8))


def test_router_zero_tokens_and_layer_feed():
    print_case("router zero tokens / layer feed")
    ids, w = bfp8.router_topk(torch.empty(0, 256, device=dev()), 8)
    assert tuple(ids.shape) == (0, 8)
    # the router's output drives the layer: same result as the oracle's routing
    M, E, k, H, I = 3, 16, 4, 256, 128
    lg = synth.router_logits(M, E, "feed")
    ids, w = bfp8.router_topk(lg.to(dev()), k)
    mw = synth.moe_weights(E, H, I, "feed", device="cpu")
    hidden = synth.hidden_states(M, H, "feed")
    out = bfp8.fused_moe_block_fp8(hidden.to(dev()), ids, w, mw.w13.to(dev()), mw.w13_s.to(dev()), mw.w2.to(dev()),
                                   mw.w2_s.to(dev()), E=E)
    torch.cuda.synchronize()
    rid, rw = O.router_topk(lg, k)
    assert (ids.cpu().numpy() == rid).all()
    assert_layer_elementwise(out, hidden, torch.from_numpy(rid), torch.from_numpy(rw), mw, bfp8.SCALE_FP32,
                             float("inf"), E=E, what="router feeds the layer")


# routed layer: (M, E, k, H, I, score_fn) -- the decode shape with the router
# folded into the few-token kernel (softmax and biased sigmoid), a small
# few-token case, and two that take the router's own launch (more than 256
# experts; more tokens than the few-token path takes by default)
ROUTED = [(1, 256, 8, 7168, 256, bfp8.SCORE_SOFTMAX), (4, 256, 8, 7168, 256, bfp8.SCORE_SIGMOID),
          (3, 16, 4, 256, 128, bfp8.SCORE_SOFTMAX), (12, 256, 8, 2048, 256, bfp8.SCORE_SOFTMAX), (2, 512, 8, 1024, 256, bfp8.SCORE_SIGMOID),
          (16, 256, 8, 1024, 256, bfp8.SCORE_SOFTMAX), (2, 256, 16, 2048, 256, bfp8.SCORE_SOFTMAX)]


@pytest.mark.parametrize("M,E,k,H,I,score_fn", ROUTED)
def test_routed_layer(M, E, k, H, I, score_fn):
    print_case("routed layer", M, E, k, H, I, score_fn)
    from tests.gpu_util import bf16_np
    lg = synth.router_logits(M, E, "routed", bf16_valued=True, std=2.0)
    bias = synth.router_bias(E, "routed", std=0.1) if score_fn == bfp8.SCORE_SIGMOID else None
    scale = 2.5 if score_fn == bfp8.SCORE_SIGMOID else 1.0
    rid, rw = O.router_topk(lg, k, score_fn, bias, True, scale)
    mw = synth.moe_weights(E, H, I, "routed", M, experts=np.unique(rid).tolist(), device=dev())
    hidden = synth.hidden_states(M, H, "routed", M).to(dev())
    out, ids, w = bfp8.fused_moe_block_fp8_routed(hidden, lg.to(dev()), k, mw.w13, mw.w13_s, mw.w2, mw.w2_s,
                                                  score_fn, None if bias is None else bias.to(dev()), True, scale)
    # the same layer from the router's routing, in two calls
    out2 = bfp8.fused_moe_block_fp8(hidden, ids.clone(), w.clone(), mw.w13, mw.w13_s, mw.w2, mw.w2_s, E=E)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == rid).all()
    assert ulps(w.cpu().numpy(), rw).max() <= 1.0
    assert (bf16_np(out) == bf16_np(out2)).all()
    assert_layer_elementwise(out, hidden, torch.from_numpy(rid), torch.from_numpy(rw), mw, bfp8.SCALE_FP32,
                             float("inf"), E=E, what=f"routed M={M} E={E}", o=bfp8.opts())


# routed layer with group-limited noaux-TC selection: (M, E, k, H, I, n_group,
# topk_group) -- folded into the few-token kernel (1 and 4 tokens), the
# router's own launch before the few-token path (12 tokens) and before the
# general path (40 tokens)
ROUTED_GROUPED = [(1, 256, 8, 7168, 256, 8, 4), (4, 256, 8, 2048, 256, 8, 4), (12, 256, 8, 2048, 256, 8, 4),
                  (40, 256, 8, 1024, 256, 8, 4), (2, 64, 6, 1024, 128, 4, 2)]


@pytest.mark.parametrize("M,E,k,H,I,n_group,topk_group", ROUTED_GROUPED)
def test_routed_layer_grouped(M, E, k, H, I, n_group, topk_group):
    print_case("routed layer grouped", M, E, k, H, I, n_group, topk_group)
    from tests.gpu_util import bf16_np
    lg = synth.router_logits(M, E, "routed_grp", bf16_valued=True, std=2.0)
    bias = synth.router_bias(E, "routed_grp", std=0.1)
    rid, rw = O.router_noaux_tc(lg, k, n_group, topk_group, bias, True, 2.5)
    mw = synth.moe_weights(E, H, I, "routed_grp", M, experts=np.unique(rid).tolist(), device=dev())
    hidden = synth.hidden_states(M, H, "routed_grp", M).to(dev())
    out, ids, w = bfp8.fused_moe_block_fp8_routed(hidden, lg.to(dev()), k, mw.w13, mw.w13_s, mw.w2, mw.w2_s,
                                                  bfp8.SCORE_SIGMOID, bias.to(dev()), True, 2.5, n_group=n_group,
                                                  topk_group=topk_group)
    ids2, w2 = bfp8.router_noaux_tc(lg.to(dev()), k, n_group, topk_group, bias.to(dev()), True, 2.5)
    out2 = bfp8.fused_moe_block_fp8(hidden, ids2, w2, mw.w13, mw.w13_s, mw.w2, mw.w2_s, E=E)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == rid).all()
    assert ulps(w.cpu().numpy(), rw).max() <= 1.0
    assert (bf16_np(out) == bf16_np(out2)).all()
    assert_layer_elementwise(out, hidden, torch.from_numpy(rid), torch.from_numpy(rw), mw, bfp8.SCALE_FP32,
                             float("inf"), E=E, what=f"routed grouped M={M}", o=bfp8.opts())


@pytest.mark.parametrize("M", [3, 6])
def test_routed_layer_expert_slice_and_options(M):
    # 64 experts of which [16, 40) are local, UE8M0 scales, clamp 7: the
    # folded path (3 tokens) and the router's own launch (6 tokens) give the
    # two-call result bit for bit, and the oracle's to the layer tolerance
    print_case("routed layer slice", M)
    from tests.gpu_util import bf16_np
    E, k, H, I, off, L = 64, 8, 1024, 256, 16, 24
    lg = synth.router_logits(M, E, "routed_slice", std=2.0)
    lg[1, off:off + L] -= 20.0  # token 1 has no local route: its output row is zero
    W = synth.moe_weights(L, H, I, "routed_slice", device=dev())
    hidden = (synth.hidden_states(M, H, "routed_slice").float() * 4).to(torch.bfloat16).to(dev())
    o = bfp8.opts(scale_fmt=bfp8.SCALE_UE8M0, clamp_limit=7.0, expert_offset=off, local_num_experts=L)
    out, ids, w = bfp8.fused_moe_block_fp8_routed(hidden, lg.to(dev()), k, W.w13, W.w13_s, W.w2, W.w2_s, o=o)
    ids2, w2 = bfp8.router_topk(lg.to(dev()), k)
    out2 = bfp8.fused_moe_block_fp8(hidden, ids2, w2, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o)
    torch.cuda.synchronize()
    rid, rw = O.router_topk(lg, k)
    assert (ids.cpu().numpy() == rid).all() and ulps(w.cpu().numpy(), rw).max() <= 1.0
    assert (bf16_np(out) == bf16_np(out2)).all()
    local = ((rid >= off) & (rid < off + L)).any(axis=1)
    assert local.any() and not local[1]
    assert (bf16_np(out)[1] == 0).all()
    assert_layer_elementwise(out, hidden, torch.from_numpy(rid), torch.from_numpy(rw), W, bfp8.SCALE_UE8M0, 7.0,
                             E=E, expert_offset=off, L=L, what=f"routed slice M={M}", o=o)


# routed layer on the general path with FLAG_ROUTER_IN_ROUTE_PREP: route
# preparation ranks the tokens itself (router and route preparation one
# launch).  ids as the oracle's router and weights within 1 ulp, ids and
# weights bit for bit the router kernel's, and the output bit for bit the
# router kernel followed by the layer.  (M, E, k, H, I, score_fn, n_group,
# topk_group, local experts); 65 tokens are past the fold: the flag is refused
# and, without it, the router takes its own launch.
GENERAL_ROUTED = [
    (16, 256, 8, 2048, 256, bfp8.SCORE_SOFTMAX, 1, 1, None),
    (32, 256, 8, 1024, 256, bfp8.SCORE_SIGMOID, 1, 1, None),
    (64, 256, 8, 1024, 256, bfp8.SCORE_SIGMOID, 8, 4, None),
    (64, 128, 6, 512, 256, bfp8.SCORE_SOFTMAX, 1, 1, "slice"),
    (48, 256, 8, 1024, 256, bfp8.SCORE_SIGMOID, 8, 4, "map"),
    (40, 256, 8, 1024, 256, bfp8.SCORE_SOFTMAX, 1, 1, "w8a8"),
    (1, 64, 4, 256, 128, bfp8.SCORE_SOFTMAX, 1, 1, None),
    (65, 256, 8, 1024, 256, bfp8.SCORE_SOFTMAX, 1, 1, None),
]


@pytest.mark.parametrize("M,E,k,H,I,score_fn,n_group,topk_group,local", GENERAL_ROUTED)
def test_routed_layer_general_path(M, E, k, H, I, score_fn, n_group, topk_group, local):
    print_case("routed general", M, E, k, H, I, score_fn, n_group, topk_group, local)
    from tests.gpu_util import bf16_np
    key = ("routed_gen", M, E)
    lg = synth.router_logits(M, E, *key, bf16_valued=True, std=2.0)
    bias = synth.router_bias(E, *key, std=0.1) if score_fn == bfp8.SCORE_SIGMOID else None
    scale = 2.5 if score_fn == bfp8.SCORE_SIGMOID else 1.0
    if n_group > 1:
        rid, rw = O.router_noaux_tc(lg, k, n_group, topk_group, bias, True, scale)
    else:
        rid, rw = O.router_topk(lg, k, score_fn, bias, True, scale)
    fold = M <= 64
    flags = bfp8.FLAG_LAYER_GENERAL | (bfp8.FLAG_ROUTER_IN_ROUTE_PREP if fold else 0)
    if local == "slice":
        off, L = 32, 64
        W = synth.moe_weights(L, H, I, *key, device=dev())
        o = bfp8.opts(flags=flags, expert_offset=off, local_num_experts=L)
    elif local == "map":
        L = E // 4
        m = np.full(E, -1, np.int32)
        m[1::4] = np.arange(L, dtype=np.int32)[::-1]  # every fourth expert is local, in reverse order
        W = synth.moe_weights(L, H, I, *key, device=dev())
        o = bfp8.opts(flags=flags, local_num_experts=L, expert_map=torch.from_numpy(m).to(dev()))
    elif local == "w8a8":
        g = torch.Generator(device=dev()).manual_seed(synth.seed_of(*key))
        c13 = torch.randint(0, 0x7F, (E, 2 * I, H), generator=g, device=dev(), dtype=torch.uint8)
        c2 = torch.randint(0, 0x7F, (E, H, I), generator=g, device=dev(), dtype=torch.uint8)
        s13 = torch.rand(E, 2 * I, generator=g, device=dev()) * 1e-3 + 1e-4
        s2 = torch.rand(E, H, generator=g, device=dev()) * 1e-3 + 1e-4
        W = synth.MoEWeights(c13, s13, c2, s2)
        o = bfp8.opts(flags=flags, weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL)
    else:
        W = synth.moe_weights(E, H, I, *key, experts=np.unique(rid).tolist(), device=dev())
        o = bfp8.opts(flags=flags)
    assert bfp8.fused_moe_stages(M, H, k, E, I, o)[0].startswith("route_prepare")
    hidden = synth.hidden_states(M, H, *key).to(dev())
    if not fold:
        o_fold = bfp8.opts(flags=flags | bfp8.FLAG_ROUTER_IN_ROUTE_PREP)
        with pytest.raises(bfp8.BFP8MoEError) as ei:
            bfp8.fused_moe_block_fp8_routed(hidden, lg.to(dev()), k, W.w13, W.w13_s, W.w2, W.w2_s, score_fn, None,
                                            True, scale, o=o_fold)
        assert ei.value.status == 2
    out, ids, w = bfp8.fused_moe_block_fp8_routed(hidden, lg.to(dev()), k, W.w13, W.w13_s, W.w2, W.w2_s, score_fn,
                                                  None if bias is None else bias.to(dev()), True, scale, o=o,
                                                  n_group=n_group, topk_group=topk_group)
    # the router kernel, then the layer
    if n_group > 1:
        ids2, w2 = bfp8.router_noaux_tc(lg.to(dev()), k, n_group, topk_group, bias.to(dev()), True, scale)
    else:
        ids2, w2 = bfp8.router_topk(lg.to(dev()), k, score_fn, None if bias is None else bias.to(dev()), True,
                                    scale)
    out2 = bfp8.fused_moe_block_fp8(hidden, ids2, w2, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == rid).all()
    assert ulps(w.cpu().numpy(), rw).max() <= 1.0
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    nd = int((bf16_np(out) != bf16_np(out2)).sum())
    print(f"  {nd} of {out.numel()} outputs differ from the two-call layer", flush=True)
    assert nd == 0
