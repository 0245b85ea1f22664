"""fused_moe_block_fp8_noalloc (workspace in the library's own device array)
against fused_moe_block_fp8 (caller's workspace), through the C ABI: the same
bits on two calls in a row, the second with fewer tokens, on each layer path;
and a call whose workspace would exceed the array is refused before any
launch."""
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from tests.gpu_util import dev, print_case

pytestmark = pytest.mark.gpu


def _case(name, M, E, k, H, I, instance):
    c = synth.LayerCase(name, M=M, E=E, k=k, H=H, I=I, routing="uniform")
    return synth.layer_inputs(c, instance, device=dev())


@pytest.mark.parametrize("flags,shape", [
    (0, (256, 8, 7168, 256)),                               # few-token path by default
    (bfp8.FLAG_LAYER_DECODE, (64, 8, 2048, 384)),
    (bfp8.FLAG_LAYER_GENERAL, (128, 8, 4096, 768)),
])
def test_no_alloc_matches_the_workspace_entry_point(flags, shape):
    E, k, H, I = shape
    for M, inst in ((4, 0), (1, 1)):  # the second call is smaller
        print_case("no-alloc", flags, M, shape)
        hidden, ids, w, W = _case("noalloc", M, E, k, H, I, inst)
        o = bfp8.opts(flags=flags)
        ref = bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o)
        out = torch.full_like(ref, float("nan"))
        bfp8.fused_moe_block_fp8_noalloc(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"M={M}"


def test_no_alloc_refuses_a_workspace_beyond_its_array():
    print_case("no-alloc too large")
    M, E, k, H, I = 2048, 8, 8, 4096, 1024
    o = bfp8.opts(flags=bfp8.FLAG_LAYER_GENERAL)
    assert bfp8.fused_moe_workspace_size(M, H, k, E, I, o) > bfp8.NOALLOC_SCRATCH_BYTES
    hidden = torch.zeros(M, H, dtype=torch.bfloat16, device=dev())
    ids = torch.zeros(M, k, dtype=torch.int32, device=dev())
    w = torch.zeros(M, k, dtype=torch.float32, device=dev())
    W = synth.MoEWeights(torch.zeros(E, 2 * I, H, dtype=torch.uint8, device=dev()),
                         torch.zeros(E, 2 * I // 128, H // 128, dtype=torch.float32, device=dev()),
                         torch.zeros(E, H, I, dtype=torch.uint8, device=dev()),
                         torch.zeros(E, H // 128, I // 128, dtype=torch.float32, device=dev()))
    out = torch.full((M, H), 3.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(bfp8.BFP8MoEError) as ei:
        bfp8.fused_moe_block_fp8_noalloc(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E, o=o, out=out)
    assert ei.value.status == 3 and "limit" in str(ei.value)
    torch.cuda.synchronize()
    assert (out == 3.0).all()  # nothing was launched
