"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

# Spec bound on BF16 outputs of the GEMMs and the layer: normwise
# max|gpu - oracle| / max|oracle| <= 2e-2.
LAYER_TOL = 2e-2


def dev():
    return torch.device("cuda:0")


def f32_of_bf16_bits(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def normwise_err(gpu_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    g = f32_of_bf16_bits(gpu_bits).astype(np.float64)
    r = f32_of_bf16_bits(ref_bits).astype(np.float64)
    denom = np.abs(r).max()
    return float(np.abs(g - r).max() / denom) if denom > 0 else float(np.abs(g).max())


def assert_gemm_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, what=""):
    """GEMM outputs from identical inputs: the GPU accumulates in fp32 in its
    own order, the oracle in fp64; both round once to BF16.  Each element may
    differ by one BF16 rounding step (2^-8 relative) plus fp32 accumulation
    error, bounded here by 2^-12 of the largest magnitude; the north-star
    normwise bound must hold too."""
    g = f32_of_bf16_bits(gpu_bits).astype(np.float64)
    r = f32_of_bf16_bits(ref_bits).astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    scale = np.abs(r).max()
    bound = np.abs(r) * 2.0 ** -7 + scale * 2.0 ** -12
    bad = np.abs(g - r) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {np.abs(g - r)[bad].max()} (scale {scale})"
    assert normwise_err(gpu_bits, ref_bits) <= LAYER_TOL


def print_case(*parts):
    print("CASE", *parts, flush=True)
