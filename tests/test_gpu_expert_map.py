"""GPU parity (through the C ABI) of the expert-map form of the local expert
set: route preparation and moe_reduce bit-exact against the oracle on the
mapped ids; the layer on every path bit-exact on the exact-arithmetic
workload and within the element-wise bound on Gaussian inputs; the general
path's act+quant over route preparation's compact list (expert-parallel
shapes where most routes are remote)."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import assert_layer_elementwise, bf16_np, dev, print_case

pytestmark = pytest.mark.gpu

PATH_FLAGS = {"token": bfp8.FLAG_LAYER_TOKEN, "decode": bfp8.FLAG_LAYER_DECODE, "general": bfp8.FLAG_LAYER_GENERAL}
ROUTE_FLAGS = {"single": bfp8.FLAG_ROUTE_SINGLE_WG, "multi": bfp8.FLAG_ROUTE_MULTI_WG}


def _map(E, L, key, extra=True):
    """A map with L local experts at random global ids in random order; with
    extra, a few remote entries hold values >= L or below -1 (also remote)
    and one local expert has two global ids."""
    rng = np.random.default_rng(synth.seed_of(key) % (1 << 32))
    g = rng.permutation(E)[:L]
    m = np.full(E, -1, np.int32)
    m[g] = rng.permutation(L).astype(np.int32)
    if extra and E > L + 3:
        rem = np.flatnonzero(m < 0)
        m[rem[0]] = L
        m[rem[1]] = -7
        m[rem[2]] = int(m[g[0]])  # an alias of a local expert
    return m


def _local_weights(W, m, L):
    """Local weights: local expert e holds the weights of the first global id
    the map sends to e."""
    inv = np.array([int(np.flatnonzero(m == e)[0]) for e in range(L)])
    sel = torch.from_numpy(inv).to(W.w13.device)
    return synth.MoEWeights(W.w13[sel].contiguous(), W.w13_s[sel].contiguous(), W.w2[sel].contiguous(),
                            W.w2_s[sel].contiguous()), inv


@pytest.mark.parametrize("path", ["single", "multi"])
@pytest.mark.parametrize("R,E,L,B", [(1, 8, 2, 16), (300, 64, 8, 16), (5000, 256, 32, 64), (2048, 512, 512, 7),
                                     (4097, 128, 100, 32)])
def test_route_prepare_map(path, R, E, L, B):
    print_case("route map", path, R, E, L, B)
    g = torch.Generator().manual_seed(R + E)
    ids = torch.randint(-1, E + 3, (R,), generator=g, dtype=torch.int32)
    m = _map(E, L, ("route_map", R, E))
    loc = O.apply_expert_map(ids.numpy(), m, L)
    ref = O.route_prepare(loc, 0, L, B)
    for with_blocks in (True, False):
        got = bfp8.moe_route_prepare(ids.to(dev()), 0, L, B, with_blocks=with_blocks, flags=ROUTE_FLAGS[path],
                                     expert_map=torch.from_numpy(m).to(dev()))
        torch.cuda.synchronize()
        assert np.array_equal(got["sorted_routes"].cpu().numpy(), ref["sorted_routes"])
        assert np.array_equal(got["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
        assert int(got["num_blocks"].item()) == ref["num_blocks"]
        if with_blocks:
            mb = ref["max_blocks"]
            assert np.array_equal(got["block_expert"][:mb].cpu().numpy(), ref["block_expert"])
            assert np.array_equal(got["block_start"][:mb].cpu().numpy(), ref["block_start"])


def test_route_prepare_map_rejects_bad_arguments():
    print_case("route map bad args")
    ids = torch.zeros(8, dtype=torch.int32, device=dev())
    m = torch.zeros(4, dtype=torch.int32, device=dev())
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.moe_route_prepare(ids, 0, 0, 16, expert_map=m)  # L = 0
    with pytest.raises(ValueError):
        bfp8.moe_route_prepare(ids, 2, 4, 16, expert_map=m)  # map and offset


@pytest.mark.parametrize("M,k,E,L,H", [(7, 8, 64, 8, 1024), (300, 6, 256, 32, 2048), (1, 8, 16, 16, 7168)])
def test_moe_reduce_map(M, k, E, L, H):
    print_case("reduce map", M, k, E, L, H)
    ids, w = synth.uniform_routing(M, E, k, "reduce_map", M)
    m = _map(E, L, ("reduce_map", M))
    y = synth.act_rows(M * k, H // 2, E, "reduce_map_y", M)[0]  # [M k, H] BF16
    got = bfp8.moe_reduce(y.to(dev()), w.to(dev()), ids.to(dev()), 0, L, expert_map=torch.from_numpy(m).to(dev()))
    torch.cuda.synchronize()
    ref = O.moe_reduce(y, w, O.apply_expert_map(ids.numpy(), m, L), 0, L)
    assert np.array_equal(bf16_np(got), ref)


# (M, E, k, H, I, L): few-token and small-batch shapes, and general-path
# shapes where most routes are remote (the act+quant list is short)
LAYER_SHAPES = [(1, 32, 8, 7168, 256, 12), (4, 48, 8, 2048, 256, 16), (3, 24, 8, 1024, 384, 9),
                (64, 64, 8, 1024, 256, 8), (200, 256, 8, 2048, 512, 32)]


def _paths(M, H, k, E, I, L, m):
    out = []
    for name, flag in PATH_FLAGS.items():
        o = bfp8.opts(flags=flag, local_num_experts=L, expert_map=m)
        try:
            st = bfp8.fused_moe_stages(M, H, k, E, I, o)
        except bfp8.BFP8MoEError:
            continue
        if name == "general" or st[0].startswith(name):
            out.append((name, o))
    return out


@pytest.mark.parametrize("M,E,k,H,I,L", LAYER_SHAPES)
def test_layer_map_exact_workload(M, E, k, H, I, L):
    print_case("layer map exact", M, E, k, H, I, L)
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "layer_map", device=dev())
    m = _map(E, L, ("layer_map", M, E))
    md = torch.from_numpy(m).to(dev())
    Wl, _ = _local_weights(W, m, L)
    loc = O.apply_expert_map(ids.cpu().numpy(), m, L)
    ref = O.fused_moe(hidden.cpu(), loc, w.cpu(), Wl.w13.cpu(), Wl.w13_s.cpu(), Wl.w2.cpu(), Wl.w2_s.cpu(),
                      scale_fmt=O.SCALE_UE8M0, L=L)
    paths = _paths(M, H, k, E, I, L, md)
    assert paths
    for name, o in paths:
        o.scale_fmt = bfp8.SCALE_UE8M0
        need = bfp8.fused_moe_workspace_size(M, H, k, E, I, o)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev())  # NaN-filled
        out = bfp8.fused_moe_block_fp8(hidden, ids, w, Wl.w13, Wl.w13_s, Wl.w2, Wl.w2_s, E=E, o=o, ws=ws)
        torch.cuda.synchronize()
        nd = int((bf16_np(out) != ref).sum())
        print(f"  {name}: {nd} of {ref.size} outputs differ", flush=True)
        assert nd == 0


@pytest.mark.parametrize("M,E,k,H,I,L", [(1, 64, 8, 2048, 256, 16), (6, 32, 8, 1024, 256, 8),
                                         (128, 128, 8, 1024, 256, 16)])
def test_layer_map_gaussian(M, E, k, H, I, L):
    print_case("layer map gaussian", M, E, k, H, I, L)
    c = synth.LayerCase("layer_map_g", M=M, E=E, k=k, H=H, I=I, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev(), only_active=False)
    m = _map(E, L, ("layer_map_g", M))
    md = torch.from_numpy(m).to(dev())
    Wl, _ = _local_weights(W, m, L)
    loc = torch.from_numpy(O.apply_expert_map(ids.cpu().numpy(), m, L)).to(dev())
    for name, o in _paths(M, H, k, E, I, L, md):
        out = bfp8.fused_moe_block_fp8(hidden, ids, w, Wl.w13, Wl.w13_s, Wl.w2, Wl.w2_s, E=E, o=o)
        torch.cuda.synchronize()
        # the oracle on the mapped ids: the same layer with the slice [0, L)
        assert_layer_elementwise(out, hidden, loc, w, Wl, bfp8.SCALE_FP32, float("inf"), E=L, L=L,
                                 what=f"map {name}", o=o)


def test_layer_map_rejects_offset():
    print_case("layer map bad args")
    c = synth.LAYER_CASES["tiny"]
    hidden, ids, w, W = synth.layer_inputs(c, 0, device=dev())
    m = torch.zeros(c.E, dtype=torch.int32, device=dev())
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                 o=bfp8.opts(expert_offset=1, local_num_experts=2, expert_map=m))
    with pytest.raises(ValueError):  # a map of the wrong length
        bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=c.E,
                                 o=bfp8.opts(local_num_experts=2, expert_map=m[:-1]))
