"""GPU parity (through the C ABI) for the group-limited noaux-TC router:
expert ids bit-exact against the CPU oracle, weights within one fp32 ulp (fp64
on both sides, rounded once)."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import dev, print_case
from tests.test_gpu_router import ulps

pytestmark = pytest.mark.gpu

# (M, E, k, n_group, topk_group): the DeepSeek-V3-style 256 experts in 8
# groups keeping 4, at decode and prefill token counts; 160 experts in 8
# groups keeping 3; a width that is not a multiple of 64; groups of one
# expert; 64 groups of 16 over 1024 experts; every group kept
SHAPES = [(1, 256, 8, 8, 4), (7, 256, 8, 8, 4), (1000, 256, 8, 8, 4), (33, 160, 6, 8, 3), (64, 64, 6, 4, 2),
          (16, 72, 8, 9, 2), (5, 1024, 8, 64, 8), (9, 16, 4, 16, 6), (3, 256, 8, 8, 8), (4, 512, 8, 16, 2)]


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("M,E,k,n_group,topk_group", SHAPES)
def test_noaux_tc_parity(M, E, k, n_group, topk_group, renorm):
    print_case("noaux-tc", M, E, k, n_group, topk_group, renorm)
    for bf16_valued in (True, False):
        lg = synth.router_logits(M, E, "noaux", bf16_valued, std=2.0, bf16_valued=bf16_valued)
        for bias in (synth.router_bias(E, "noaux", std=0.1), None):
            ids, w = bfp8.router_noaux_tc(lg.to(dev()), k, n_group, topk_group,
                                          None if bias is None else bias.to(dev()), renorm, 2.5)
            torch.cuda.synchronize()
            rid, rw = O.router_noaux_tc(lg, k, n_group, topk_group, bias, renorm, 2.5)
            got = ids.cpu().numpy()
            assert (got == rid).all(), np.argwhere(got != rid)[:5]
            assert ulps(w.cpu().numpy(), rw).max() <= 1.0


def test_noaux_tc_one_group_is_the_sigmoid_router():
    print_case("noaux-tc one group")
    lg = synth.router_logits(40, 256, "noaux1", std=2.0).to(dev())
    bias = synth.router_bias(256, "noaux1").to(dev())
    a = bfp8.router_noaux_tc(lg, 8, 1, 1, bias)
    b = bfp8.router_topk(lg, 8, bfp8.SCORE_SIGMOID, bias)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_noaux_tc_rejects_bad_grouping():
    print_case("noaux-tc bad args")
    lg = torch.zeros(2, 96, device=dev())
    for args in ((8, 7, 2), (8, 8, 9), (8, 96, 2), (40, 8, 2)):  # n_group not dividing E; too many; k too big
        with pytest.raises(bfp8.BFP8MoEError):
            bfp8.router_noaux_tc(lg, *args)
