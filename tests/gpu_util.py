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


def oracle_inputs_for_tokens(hidden, ids, w, W, tokens, E, expert_offset=0, L=None):
    """Host copies of what the oracle needs for the listed tokens: their rows,
    and only the experts their live routes use (re-numbered in id order), so
    that large expert tensors never travel to the host."""
    import torch
    from block_fp8_mixture_route_amd import synth
    L = W.w13.shape[0] if L is None else L
    ids_t = ids[tokens].cpu()
    loc = ids_t.to(torch.int64) - expert_offset
    live = (loc >= 0) & (loc < L)
    used = torch.unique(loc[live])
    remap = torch.full((L,), -1, dtype=torch.int64)
    remap[used] = torch.arange(used.numel())
    ids_local = torch.where(live, remap[loc.clamp(0, L - 1)], torch.full_like(loc, -1)).to(torch.int32)
    sel = used.to(W.w13.device)
    Wl = synth.MoEWeights(W.w13[sel].cpu(), W.w13_s[sel].cpu(), W.w2[sel].cpu(), W.w2_s[sel].cpu())
    return hidden[tokens].cpu(), ids_local, w[tokens].cpu(), Wl


def uses_mfma(M, H, k, E, I, o) -> bool:
    """Whether a fused_moe_block_fp8 call with these sizes and options runs its
    GEMMs on FP8 MFMA (every path but the few-token one)."""
    import block_fp8_mixture_route_amd as bfp8
    return bfp8.fused_moe_stages(M, H, k, E, I, o)[0] != "token_gate_up_swiglu"


def assert_layer_elementwise(out, hidden, ids, w, W, fmt, clamp, tokens=None, E=None, expert_offset=0, L=None,
                             what="", o=None):
    """The layer output of the listed tokens (all by default) against the
    oracle, element by element: each output must lie in the interval of
    tests.parity.layer_out_bound (the oracle's value itself wherever no BF16
    rounding boundary is within the GPU's error bound); also the normwise
    error.  o: the options of the call (its path decides whether the FP8
    MFMA's error counts).  Prints the observed differences and the allowance
    counts."""
    import block_fp8_mixture_route_amd as bfp8
    from tests.parity import check_layer, layer_out_bound
    M = hidden.shape[0]
    k = ids.shape[1]
    o = bfp8.opts(scale_fmt=fmt, clamp_limit=clamp, expert_offset=expert_offset,
                  local_num_experts=0 if L is None else L) if o is None else o
    mfma = uses_mfma(M, hidden.shape[1], k, E, W.w2.shape[2], o)
    tokens = list(range(M)) if tokens is None else list(tokens)
    hid, ids_l, w_l, Wl = oracle_inputs_for_tokens(hidden, ids, w, W, tokens, E, expert_offset, L)
    ref, lo, hi, st = layer_out_bound(hid, ids_l, w_l, Wl, fmt, clamp, mfma=mfma)
    got = bf16_np(out)[tokens]
    ndiff, steps = check_layer(got, ref, lo, hi, what)
    nerr = normwise_err(got, ref)
    print(f"{what} ({'FP8 MFMA' if mfma else 'fp32 VALU'} sums): {ndiff} of {got.size} outputs differ from the oracle (at most {steps:.0f} BF16 steps), "
          f"{st['ambiguous_out']} may; normwise {nerr:.2e}; ambiguous SwiGLU values {st['ambiguous_act']} "
          f"(in {st['act_groups_with_ambiguity']} groups), down outputs {st['ambiguous_y']}", flush=True)
    assert nerr <= LAYER_TOL
    return ndiff
