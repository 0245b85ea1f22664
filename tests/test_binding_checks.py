"""The Python binding refuses buffers whose dtype or shape the library would
misread (CPU; nothing is launched): int64 routing ids, float32 hidden
states, weights with fewer experts than the call addresses, scales of the
wrong block shape, outputs of the wrong size."""
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8

M, k, E, H, I = 2, 4, 8, 256, 128


def _layer_args(**over):
    a = dict(hidden=torch.zeros(M, H, dtype=torch.bfloat16),
             topk_ids=torch.zeros(M, k, dtype=torch.int32),
             topk_w=torch.zeros(M, k, dtype=torch.float32),
             w13=torch.zeros(E, 2 * I, H, dtype=torch.uint8),
             w13_scale=torch.zeros(E, 2 * I // 128, H // 128, dtype=torch.float32),
             w2=torch.zeros(E, H, I, dtype=torch.uint8),
             w2_scale=torch.zeros(E, H // 128, I // 128, dtype=torch.float32))
    a.update(over)
    return a


BAD = {
    "int64 ids": dict(topk_ids=torch.zeros(M, k, dtype=torch.int64)),
    "float32 hidden": dict(hidden=torch.zeros(M, H, dtype=torch.float32)),
    "float16 hidden": dict(hidden=torch.zeros(M, H, dtype=torch.float16)),
    "weights of the wrong row count": dict(topk_w=torch.zeros(M + 1, k, dtype=torch.float32)),
    "bf16 weights": dict(topk_w=torch.zeros(M, k, dtype=torch.bfloat16)),
    "w13 of the wrong width": dict(w13=torch.zeros(E, 2 * I, 2 * H, dtype=torch.uint8)),
    "w13 scale blocks": dict(w13_scale=torch.zeros(E, 2 * I // 128, H // 64, dtype=torch.float32)),
    "w2 scale dtype": dict(w2_scale=torch.zeros(E, H // 128, I // 128, dtype=torch.float64)),
    "w2 experts differ from w13": dict(w2=torch.zeros(E - 1, H, I, dtype=torch.uint8)),
}


@pytest.mark.parametrize("what", list(BAD))
def test_layer_binding_rejects(what):
    with pytest.raises(ValueError):
        bfp8.fused_moe_block_fp8(**_layer_args(**BAD[what]))


def test_layer_binding_rejects_more_experts_than_the_weights_hold():
    with pytest.raises(ValueError):
        bfp8.fused_moe_block_fp8(**_layer_args(), E=2 * E)
    with pytest.raises(ValueError):
        bfp8.fused_moe_block_fp8(**_layer_args(), E=4 * E, o=bfp8.opts(expert_offset=8, local_num_experts=E + 1))


def test_layer_binding_rejects_a_wrong_output():
    with pytest.raises(ValueError):
        bfp8.fused_moe_block_fp8(**_layer_args(), out=torch.zeros(M, H + 8, dtype=torch.bfloat16))


def test_layer_binding_reaches_the_device_check_with_good_buffers():
    # well-formed CPU buffers pass every dtype and shape check and stop at the
    # device check (the library takes device memory only)
    with pytest.raises(ValueError, match="device"):
        bfp8.fused_moe_block_fp8(**_layer_args())


def test_step_bindings_reject():
    with pytest.raises(ValueError):
        bfp8.moe_route_prepare(torch.zeros(8, dtype=torch.int64), 0, 4, 16)
    with pytest.raises(ValueError):
        bfp8.quant_fp8(torch.zeros(2, 128, dtype=torch.float32))
    with pytest.raises(ValueError):
        bfp8.silu_and_mul_quant_fp8(torch.zeros(2, 256, dtype=torch.bfloat16),
                                    row_expert_ids=torch.zeros(2, dtype=torch.int64), E=4)
    with pytest.raises(ValueError):
        bfp8.moe_reduce(torch.zeros(M * k, H, dtype=torch.bfloat16), torch.zeros(M, k, dtype=torch.float32),
                        topk_ids=torch.zeros(M, k, dtype=torch.int64))
    with pytest.raises(ValueError):
        bfp8.moe_reduce(torch.zeros(M * k - 1, H, dtype=torch.bfloat16), torch.zeros(M, k, dtype=torch.float32))
