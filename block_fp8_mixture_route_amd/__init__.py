"""Block-FP8 fused MoE layer for AMD Instinct MI355X (gfx950).

The computation lives in libbfp8moe.so (hand-written HIP kernels behind the C
ABI of include/bfp8moe.h); this package is its thin Python binding plus the
seeded synthetic-input generator used by the tests and the benchmark.
"""
from ._lib import (  # noqa: F401
    BFP8MoEError,
    FLAG_LAYER_DECODE,
    FLAG_LAYER_GENERAL,
    FLAG_LAYER_TOKEN,
    FLAG_ONLY_STAGE,
    FLAG_ROUTE_MULTI_WG,
    FLAG_ROUTE_SINGLE_WG,
    SCALE_FP32,
    SCALE_UE8M0,
    SCORE_SIGMOID,
    SCORE_SOFTMAX,
    WEIGHT_SCALE_BLOCK,
    WEIGHT_SCALE_CHANNEL,
    Opts,
    NOALLOC_SCRATCH_BYTES,
    fused_moe_block_fp8,
    fused_moe_block_fp8_noalloc,
    fused_moe_block_fp8_routed,
    fused_moe_stages,
    fused_moe_workspace_size,
    lib,
    max_blocks,
    moe_fp8_grouped_gemm,
    moe_fp8_grouped_gemm_channel,
    moe_reduce,
    moe_route_prepare,
    opts,
    quant_fp8,
    quant_fp8_rows,
    router_noaux_tc,
    router_topk,
    silu_and_mul,
    silu_and_mul_quant_fp8,
    silu_and_mul_quant_fp8_rows,
    wait_faults,
)
