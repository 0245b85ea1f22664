"""Seeded synthetic inputs for the block-FP8 MoE layer.

This module only draws random numbers and casts them with torch's own dtype
conversions (``torch.bfloat16``, ``torch.float8_e4m3fn``).  It holds none of the
layer's arithmetic, so both the HIP library and the CPU oracle can be fed the
same bytes from here without sharing any computation.

Recipes (the workloads of the block-FP8 MoE pages and their benchmark shapes):

* hidden states: N(0, 1) fp32 rounded to BF16;
* expert weights: N(0, 0.02) fp32 per expert, split into 128x128 blocks, each
  block scaled by its amax / 448 and cast to E4M3FN (offline weight
  preparation, as a checkpoint would ship it);
* uniform routing: N(0, 1) router logits -> softmax -> top-k -> weights
  renormalised to sum 1;
* Zipf(s) routing: expert e has probability proportional to (pi(e)+1)^-s for a
  seeded permutation pi; k distinct experts are drawn without replacement by
  Gumbel-top-k; their weights are a softmax of N(0, 1) logits over the k;
* activation-only rows: gate/up BF16 from N(0, std 2); about 10 % of rows get
  expert id -1 (masked), the rest a uniform id.

Every stream is seeded from the tuple (1234, config, instance, stream name,
index) through SHA-256, so any slice can be regenerated on its own.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Iterable, Optional, Sequence

import torch

BASE_SEED = 1234
GROUP = 128


def seed_of(*parts) -> int:
    h = hashlib.sha256(repr((BASE_SEED,) + tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


# --------------------------------------------------------------------------
# activations and routing
# --------------------------------------------------------------------------

def hidden_states(M: int, H: int, *key, device="cpu") -> torch.Tensor:
    g = gen(device, *key, "hidden")
    return torch.randn(M, H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def uniform_routing(M: int, E: int, k: int, *key, device="cpu"):
    """Softmax top-k over N(0,1) logits, renormalised weights."""
    g = gen(device, *key, "router_uniform")
    logits = torch.randn(M, E, generator=g, device=device, dtype=torch.float32)
    p = torch.softmax(logits, dim=-1)
    w, ids = torch.topk(p, k, dim=-1)
    w = w / w.sum(dim=-1, keepdim=True)
    return ids.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


def zipf_routing(M: int, E: int, k: int, s: float, *key, device="cpu"):
    """k distinct experts per token drawn without replacement from a Zipf(s)
    popularity over a seeded expert permutation (Gumbel-top-k)."""
    g = gen(device, *key, "router_zipf", s)
    perm = torch.randperm(E, generator=g, device=device)
    rank = torch.empty(E, dtype=torch.float64, device=device)
    rank[perm] = torch.arange(E, dtype=torch.float64, device=device)
    logp = -s * torch.log(rank + 1.0)
    u = torch.rand(M, E, generator=g, device=device, dtype=torch.float64).clamp_(1e-300, 1.0)
    keys = logp[None, :] - torch.log(-torch.log(u))
    ids = torch.topk(keys, k, dim=-1).indices
    logits = torch.randn(M, k, generator=g, device=device, dtype=torch.float32)
    w = torch.softmax(logits, dim=-1)
    w = w / w.sum(dim=-1, keepdim=True)
    return ids.to(torch.int32).contiguous(), w.contiguous()


def mixed_routing(M: int, E: int, k: int, s: float, *key, device="cpu"):
    """First half of the tokens uniform, second half Zipf(s)."""
    h = M // 2
    ids_u, w_u = uniform_routing(h, E, k, *key, "first_half", device=device)
    ids_z, w_z = zipf_routing(M - h, E, k, s, *key, "second_half", device=device)
    return torch.cat([ids_u, ids_z]).contiguous(), torch.cat([w_u, w_z]).contiguous()


def act_rows(rows: int, I: int, E: int, *key, masked_frac=0.1, std=2.0, device="cpu"):
    """Gate/up rows [rows, 2I] BF16 and their expert ids (-1 = masked)."""
    g = gen(device, *key, "act_rows")
    x = (torch.randn(rows, 2 * I, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    ids = torch.randint(0, E, (rows,), generator=g, device=device, dtype=torch.int32)
    drop = torch.rand(rows, generator=g, device=device) < masked_frac
    ids = torch.where(drop, torch.full_like(ids, -1), ids)
    return x.contiguous(), ids.contiguous()


# --------------------------------------------------------------------------
# block-FP8 expert weights
# --------------------------------------------------------------------------

def block_fp8_weight(N: int, K: int, *key, std=0.02, device="cpu"):
    """One expert's [N, K] weight as E4M3FN bytes plus [N/128, K/128] fp32
    block scales (amax / 448 per block)."""
    g = gen(device, *key)
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * std
    blocks = w.view(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = amax / 448.0
    codes = (blocks / scale[:, None, :, None]).to(torch.float8_e4m3fn)
    return codes.view(N, K).view(torch.uint8), scale.contiguous()


def fill_random_codes(t: torch.Tensor, *key):
    """Fill a uint8 tensor with seeded random bytes (used for experts no route
    reads: they must exist, their values never matter, and a kernel that reads
    them by mistake picks up garbage, NaN codes included, that parity catches).
    A seeded 1 MiB pattern is tiled over the tensor to keep this cheap."""
    g = gen(t.device, *key, "filler")
    flat = t.view(-1)
    n = flat.numel()
    chunk = min(n, 1 << 20)
    pattern = torch.randint(0, 256, (chunk,), generator=g, device=t.device, dtype=torch.uint8)
    full = n // chunk
    if full:
        flat[: full * chunk].view(full, chunk).copy_(pattern.expand(full, chunk))
    if n > full * chunk:
        flat[full * chunk:].copy_(pattern[: n - full * chunk])
    return t


@dataclass
class MoEWeights:
    w13: torch.Tensor      # [L, 2I, H] uint8 (E4M3FN), gate rows 0..I-1, up rows I..2I-1
    w13_s: torch.Tensor    # [L, 2I/128, H/128] fp32
    w2: torch.Tensor       # [L, H, I] uint8
    w2_s: torch.Tensor     # [L, H/128, I/128] fp32
    real: Optional[set] = field(default=None)  # experts holding real N(0,0.02) weights (None: all)


def moe_weights(L: int, H: int, I: int, *key, experts: Optional[Iterable[int]] = None, device="cpu") -> MoEWeights:
    """All L experts' weights.  With ``experts`` given, only those experts get
    quantised Gaussian weights; the others are filled with random bytes and
    unit-free random scales (never read by a correct kernel)."""
    real = set(range(L)) if experts is None else set(int(e) for e in experts)
    if len(real) < L:
        w13 = fill_random_codes(torch.empty(L, 2 * I, H, dtype=torch.uint8, device=device), *key, "w13_idle")
        w2 = fill_random_codes(torch.empty(L, H, I, dtype=torch.uint8, device=device), *key, "w2_idle")
    else:
        w13 = torch.empty(L, 2 * I, H, dtype=torch.uint8, device=device)
        w2 = torch.empty(L, H, I, dtype=torch.uint8, device=device)
    w13_s = torch.full((L, 2 * I // GROUP, H // GROUP), 1.0e-4, dtype=torch.float32, device=device)
    w2_s = torch.full((L, H // GROUP, I // GROUP), 1.0e-4, dtype=torch.float32, device=device)
    for e in sorted(real):
        c, s = block_fp8_weight(2 * I, H, *key, "w13", e, device=device)
        w13[e].copy_(c); w13_s[e].copy_(s)
        c, s = block_fp8_weight(H, I, *key, "w2", e, device=device)
        w2[e].copy_(c); w2_s[e].copy_(s)
    return MoEWeights(w13, w13_s, w2, w2_s, None if experts is None else real)


# --------------------------------------------------------------------------
# the benchmark workloads
# --------------------------------------------------------------------------

@dataclass
class LayerCase:
    name: str
    M: int
    E: int
    k: int
    H: int
    I: int
    routing: str           # "uniform" | "zipf" | "mixed"
    zipf_s: float = 0.0
    scale_fmt: int = 0     # 0 fp32, 1 UE8M0
    clamp: float = float("inf")


LAYER_CASES = {
    "tiny": LayerCase("tiny", M=4, E=8, k=2, H=256, I=128, routing="uniform"),
    "decode_m1": LayerCase("decode_m1", M=1, E=256, k=8, H=7168, I=256, routing="uniform"),
    "decode_m4": LayerCase("decode_m4", M=4, E=256, k=8, H=7168, I=256, routing="uniform"),
    "decode_m16": LayerCase("decode_m16", M=16, E=256, k=8, H=7168, I=256, routing="uniform"),
    "decode_m32": LayerCase("decode_m32", M=32, E=256, k=8, H=7168, I=256, routing="uniform"),
    "small_m128": LayerCase("small_m128", M=128, E=256, k=8, H=4096, I=768, routing="mixed", zipf_s=1.2),
    "small_m512": LayerCase("small_m512", M=512, E=256, k=8, H=4096, I=768, routing="mixed", zipf_s=1.2),
    "large_m2048": LayerCase("large_m2048", M=2048, E=512, k=8, H=4096, I=1024, routing="zipf", zipf_s=1.0),
}

# activation + quant only: routed rows = tokens x 8, E = 288, I = 512
ACT_TOKENS = (1, 4, 16, 64, 128, 256)
ACT_E = 288
ACT_I = 512
ACT_CLAMP = 7.0

# activation + quant under 8-way expert parallelism: routed rows = tokens x 6
# (top-k 6), width I = 2048, 256 experts of which this rank holds 32
EP_TOKENS = (1, 8, 64, 512, 1024)
EP_TOPK = 6
EP_E = 256
EP_LOCAL = 32
EP_I = 2048


def ep_act_inputs(tokens: int, *key, device="cpu"):
    """Gate/up rows [tokens * 6, 2 I] BF16 (N(0, 2)), each row's expert id
    (top-k 6 distinct experts per token, uniform over 256) and the rank's
    expert map (experts [0, 32) local, the rest -1)."""
    g = gen(device, *key, "ep_act", tokens)
    rows = tokens * EP_TOPK
    x = (torch.randn(rows, 2 * EP_I, generator=g, device=device, dtype=torch.float32) * 2.0).to(torch.bfloat16)
    ids = torch.stack([torch.randperm(EP_E, generator=g, device=device)[:EP_TOPK] for _ in range(tokens)])
    emap = torch.where(torch.arange(EP_E, device=device) < EP_LOCAL, torch.arange(EP_E, device=device),
                       torch.full((EP_E,), -1, device=device))
    return x.contiguous(), ids.reshape(-1).to(torch.int32).contiguous(), emap.to(torch.int32).contiguous()


def routing_for(case: LayerCase, *key, device="cpu"):
    if case.routing == "uniform":
        return uniform_routing(case.M, case.E, case.k, case.name, *key, device=device)
    if case.routing == "zipf":
        return zipf_routing(case.M, case.E, case.k, case.zipf_s, case.name, *key, device=device)
    if case.routing == "mixed":
        return mixed_routing(case.M, case.E, case.k, case.zipf_s, case.name, *key, device=device)
    raise ValueError(case.routing)


def layer_inputs(case: LayerCase, instance: int = 0, device="cpu", only_active=True):
    """hidden, topk ids, topk weights and expert weights for one layer instance."""
    ids, w = routing_for(case, instance, device=device)
    hidden = hidden_states(case.M, case.H, case.name, instance, device=device)
    active = torch.unique(ids).tolist() if only_active else None
    weights = moe_weights(case.E, case.H, case.I, case.name, instance, experts=active, device=device)
    return hidden, ids, w, weights


# router inputs: [M, E] fp32 logits, N(0, std); with bf16_valued the logits are
# rounded to BF16 values first (a router GEMM computed in BF16), which makes
# equal logits within a token common at E = 256
def router_logits(M: int, E: int, *key, std=1.0, bf16_valued=False, device="cpu"):
    g = gen(device, *key, "router_logits", M, E)
    x = torch.randn(M, E, generator=g, device=device, dtype=torch.float32) * std
    if bf16_valued:
        x = x.to(torch.bfloat16).to(torch.float32)
    return x.contiguous()


def router_bias(E: int, *key, std=0.05, device="cpu"):
    """Per-expert selection bias of sigmoid routing, N(0, std) fp32."""
    g = gen(device, *key, "router_bias", E)
    return (torch.randn(E, generator=g, device=device, dtype=torch.float32) * std).contiguous()


# --------------------------------------------------------------------------
# a layer instance whose arithmetic is exact up to its final roundings
# --------------------------------------------------------------------------

def _e4m3_codes_of(values: torch.Tensor) -> torch.Tensor:
    """E4M3FN bytes of values that are exactly representable (small integers,
    448): torch's cast, which is exact on them."""
    return values.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def exact_layer_inputs(M: int, E: int, k: int, H: int, I: int, *key, device="cpu"):
    """hidden, topk ids, topk weights and weights of one layer instance built so
    that every sum the layer forms is exact in fp32, whatever the order:

    * hidden row t: integers in [-4, 4] times 2^m_t (m_t in {-4, -3, -2}), and in
      every group of 128 one position holding +-448 * 2^m_t, so that each group's
      amax is 448 * 2^m_t and its scale (fp32 or UE8M0) is exactly 2^m_t; the
      quantised row is the integers and +-448 themselves;
    * W13: integer codes in [-2, 2], block scales 2^b with b in {-9, -8, -7}: a
      gate/up sum is a multiple of 2^(m_t - 9) below 2^(m_t + 10);
    * W2: in each row n, two non-zero codes (+-1, +-2), one in each half of one
      16-wide slice of K (the slice varies with n), the rest zero, block
      scales 2^b as above: with power-of-two (UE8M0) activation scales a down
      output is at most two products of E4M3 values times powers of two, and
      two such products never lie in one run of 8 consecutive K (where FP8
      MFMA hardware aligns products to their largest before adding them);
    * routing: uniform top-k, with a few routes of token 0 masked (-1) when
      k > 2, and fp32 renormalised weights.

    With UE8M0 activation scales the two GEMMs are then exact in any
    accumulation order, so the BF16 gate/up values, the SwiGLU row, its codes
    and scales, the down outputs and the reduction are each determined by
    their definition alone."""
    g = gen(device, *key, "exact_layer", M, E, k, H, I)
    G, GI = H // GROUP, I // GROUP
    m = torch.randint(-4, -1, (M, 1), generator=g, device=device).to(torch.float32)
    n = torch.randint(-4, 5, (M, H), generator=g, device=device).to(torch.float32)
    pos = torch.randint(0, GROUP, (M, G), generator=g, device=device)
    sign = torch.randint(0, 2, (M, G), generator=g, device=device).to(torch.float32) * 2 - 1
    n.view(M, G, GROUP).scatter_(2, pos[:, :, None], (448.0 * sign)[:, :, None])
    hidden = (n * torch.exp2(m)).to(torch.bfloat16).contiguous()

    ids, w = uniform_routing(M, E, k, *key, "exact_routing", device=device)
    if k > 2:
        ids = ids.clone()
        ids[0, 1] = -1
        ids[0, k - 1] = -1

    w13i = torch.randint(-2, 3, (E, 2 * I, H), generator=g, device=device)
    w13 = _e4m3_codes_of(w13i).contiguous()
    w13_s = torch.exp2(torch.randint(-9, -6, (E, 2 * I // GROUP, G), generator=g, device=device).to(torch.float32))
    # W2 row n: two non-zero codes, one in each half of one 16-wide K slice
    # (the slice varies with n), so each down output is one or two products
    w2i = torch.zeros(E, H, I, dtype=torch.float32, device=device)
    sl = torch.randint(0, I // 16, (E, H, 1), generator=g, device=device)
    off = torch.randint(0, 8, (E, H, 2), generator=g, device=device)
    pos = sl * 16 + torch.tensor([0, 8], device=device) + off
    val = torch.randint(1, 3, (E, H, 2), generator=g, device=device).to(torch.float32)
    val = val * (torch.randint(0, 2, (E, H, 2), generator=g, device=device).to(torch.float32) * 2 - 1)
    w2i.scatter_(2, pos, val)
    w2 = _e4m3_codes_of(w2i).contiguous()
    w2_s = torch.exp2(torch.randint(-9, -6, (E, H // GROUP, GI), generator=g, device=device).to(torch.float32))
    return hidden, ids.contiguous(), w, MoEWeights(w13, w13_s.contiguous(), w2, w2_s.contiguous())


# ------------------------------------------------------------------ MXFP4 weights

MX_BLOCK = 32


class MxWeights:
    """MXFP4 expert weights: w13 [L, 2I, H/2] and w2 [L, H, I/2] packed E2M1
    codes (the even element of a pair in the low nibble), w13_s [L, 2I, H/32]
    and w2_s [L, H, I/32] E8M0 scale bytes (all uint8)."""

    def __init__(self, w13, w13_s, w2, w2_s):
        self.w13, self.w13_s, self.w2, self.w2_s = w13, w13_s, w2, w2_s


def pack_e2m1(codes: torch.Tensor) -> torch.Tensor:
    """[..., K] E2M1 codes (0..15) -> [..., K/2] bytes, element 2j in the low
    nibble of byte j."""
    c = codes.to(torch.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).contiguous()


def mxfp4_weights(L: int, H: int, I: int, *key, scale_lo=118, scale_hi=124, device="cpu") -> MxWeights:
    """Random MXFP4 experts: uniform E2M1 codes, scale bytes uniform in
    [scale_lo, scale_hi) independently per 32-element block.  Drawn one
    expert at a time, so that no single random tensor grows with L."""
    g = gen(device, *key, "mxfp4_weights", L, H, I)
    W = MxWeights(torch.empty(L, 2 * I, H // 2, dtype=torch.uint8, device=device),
                  torch.empty(L, 2 * I, H // MX_BLOCK, dtype=torch.uint8, device=device),
                  torch.empty(L, H, I // 2, dtype=torch.uint8, device=device),
                  torch.empty(L, H, I // MX_BLOCK, dtype=torch.uint8, device=device))
    for e in range(L):
        W.w13[e].copy_(pack_e2m1(torch.randint(0, 16, (2 * I, H), generator=g, device=device)))
        W.w2[e].copy_(pack_e2m1(torch.randint(0, 16, (H, I), generator=g, device=device)))
        W.w13_s[e].copy_(torch.randint(scale_lo, scale_hi, (2 * I, H // MX_BLOCK), generator=g, device=device))
        W.w2_s[e].copy_(torch.randint(scale_lo, scale_hi, (H, I // MX_BLOCK), generator=g, device=device))
    return W


# E2M1 codes of the integer values 0, 1, 2, 3, 4, 6 (negatives: | 8)
_E2M1_INT = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}


def _e2m1_codes_of(values: torch.Tensor) -> torch.Tensor:
    mag = values.abs().to(torch.int64)
    lut = torch.zeros(7, dtype=torch.int64, device=values.device)
    for v, c in _E2M1_INT.items():
        lut[v] = c
    return (lut[mag] | ((values < 0).to(torch.int64) << 3)).to(torch.uint8)


def exact_mxfp4_layer_inputs(M: int, E: int, k: int, H: int, I: int, *key, device="cpu"):
    """hidden, topk ids, topk weights and MXFP4 weights of one layer instance
    built like exact_layer_inputs so that every sum is exact in fp32 whatever
    the order: the hidden rows and routing as there; W13 integer E2M1 values in
    {0, +-1, +-2, +-3} with one scale byte 2^b (b in {-9, -8, -7}) shared by the
    four blocks of each 128-wide group of a row; W2 rows with two non-zero
    values (+-1, +-2) in different runs of 8 consecutive K, scales as W13."""
    g = gen(device, *key, "exact_mxfp4_layer", M, E, k, H, I)
    G, GI = H // GROUP, I // GROUP
    m = torch.randint(-4, -1, (M, 1), generator=g, device=device).to(torch.float32)
    n = torch.randint(-4, 5, (M, H), generator=g, device=device).to(torch.float32)
    pos = torch.randint(0, GROUP, (M, G), generator=g, device=device)
    sign = torch.randint(0, 2, (M, G), generator=g, device=device).to(torch.float32) * 2 - 1
    n.view(M, G, GROUP).scatter_(2, pos[:, :, None], (448.0 * sign)[:, :, None])
    hidden = (n * torch.exp2(m)).to(torch.bfloat16).contiguous()
    ids, w = uniform_routing(M, E, k, *key, "exact_mx_routing", device=device)
    if k > 2:
        ids = ids.clone()
        ids[0, 1] = -1
        ids[0, k - 1] = -1
    w13v = torch.randint(-3, 4, (E, 2 * I, H), generator=g, device=device)
    b13 = torch.randint(127 - 9, 127 - 6, (E, 2 * I, G), generator=g, device=device)
    w2v = torch.zeros(E, H, I, dtype=torch.int64, device=device)
    sl = torch.randint(0, I // 16, (E, H, 1), generator=g, device=device)
    off = torch.randint(0, 8, (E, H, 2), generator=g, device=device)
    p2 = sl * 16 + torch.tensor([0, 8], device=device) + off
    val = torch.randint(1, 3, (E, H, 2), generator=g, device=device)
    val = val * (torch.randint(0, 2, (E, H, 2), generator=g, device=device) * 2 - 1)
    w2v.scatter_(2, p2, val)
    b2 = torch.randint(127 - 9, 127 - 6, (E, H, GI), generator=g, device=device)
    W = MxWeights(pack_e2m1(_e2m1_codes_of(w13v)), b13.repeat_interleave(GROUP // MX_BLOCK, 2).to(torch.uint8).contiguous(),
                  pack_e2m1(_e2m1_codes_of(w2v)), b2.repeat_interleave(GROUP // MX_BLOCK, 2).to(torch.uint8).contiguous())
    return hidden, ids.contiguous(), w, W
