"""Pins for the oracle's expert-map form (vLLM PR "[Kernel][Perf] Fuse clamped
MoE activation and UE8M0 FP8 block quantization", Purpose: expert_map):

* route preparation on mapped ids against brute force (Python's sorted() on
  (map[id], route)) for maps that permute, drop and alias experts, with ids
  and entries out of range;
* a map that sends the slice [offset, offset + L) to [0, L) in order reproduces
  the slice form of route preparation, moe_reduce and the whole layer bit for
  bit;
* the rows the act+quant filter (ids plus map, entries >= 0) keeps are the
  rows whose mapped id is local when L covers every entry.
"""
import numpy as np
import pytest

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.test_oracle_route_gemm_reduce import brute_route_prepare


def _brute_mapped(ids, emap, L, B):
    loc = []
    for g in ids:
        e = int(emap[g]) if 0 <= g < len(emap) else -1
        loc.append(e if 0 <= e < L else -1)
    # the slice brute force with offset 0 on the mapped ids
    return brute_route_prepare(loc, 0, L, B)


@pytest.mark.parametrize("E,L,seed", [(8, 3, 0), (16, 16, 1), (32, 5, 2), (64, 64, 3)])
def test_route_prepare_mapped_brute_force(E, L, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, 200).astype(np.int32)       # some ids out of range
    emap = rng.integers(-1, L + 2, E).astype(np.int32)         # remote, local, beyond L
    emap[rng.integers(0, E)] = 0                               # at least one local expert
    loc = O.apply_expert_map(ids, emap, L)
    for B in (1, 4, 16):
        got = O.route_prepare(loc, 0, L, B)
        sr, off, blocks = _brute_mapped(ids.tolist(), emap.tolist(), L, B)
        assert got["sorted_routes"].tolist() == sr
        assert got["expert_offsets"].tolist() == off
        nb = got["num_blocks"]
        assert list(zip(got["block_expert"][:nb].tolist(), got["block_start"][:nb].tolist())) == blocks


def test_apply_expert_map_cases():
    emap = np.array([2, -1, 0, 5, 1], np.int32)
    ids = np.array([[0, 1, 2], [3, 4, -1], [5, 7, 2]], np.int32)
    got = O.apply_expert_map(ids, emap, 3)
    assert got.tolist() == [[2, -1, 0], [-1, 1, -1], [-1, -1, 0]]
    assert got.shape == ids.shape and got.dtype == np.int32


def _slice_map(E, offset, L):
    m = np.full(E, -1, np.int32)
    m[offset:offset + L] = np.arange(L, dtype=np.int32)
    return m


@pytest.mark.parametrize("E,offset,L", [(16, 0, 16), (16, 4, 6), (64, 40, 8)])
def test_slice_map_reproduces_slice_route_prepare_and_reduce(E, offset, L):
    ids, w = synth.uniform_routing(37, E, 6, "map_slice", E)
    emap = _slice_map(E, offset, L)
    loc = O.apply_expert_map(ids, emap, L)
    for B in (4, 16):
        a = O.route_prepare(ids, offset, L, B)
        b = O.route_prepare(loc, 0, L, B)
        for key in ("sorted_routes", "expert_offsets", "block_expert", "block_start"):
            assert np.array_equal(a[key], b[key]), key
        assert a["num_blocks"] == b["num_blocks"]
    y = synth.act_rows(37 * 6, 64, E, "map_slice_y")[0][:, :64].contiguous()
    ra = O.moe_reduce(y, w, ids, offset, L)
    rb = O.moe_reduce(y, w, loc, 0, L)
    assert np.array_equal(ra, rb)


@pytest.mark.parametrize("offset,L", [(0, 4), (3, 5)])
def test_slice_map_reproduces_slice_layer(offset, L):
    E = 12
    M, k, H, I = 5, 4, 256, 128
    c = synth.LayerCase("map_layer", M=M, E=E, k=k, H=H, I=I, routing="uniform")
    hidden, ids, w, W = synth.layer_inputs(c, 0, device="cpu")
    w13, w13_s, w2, w2_s = W.w13[offset:offset + L], W.w13_s[offset:offset + L], W.w2[offset:offset + L], \
        W.w2_s[offset:offset + L]
    a = O.fused_moe(hidden, ids, w, w13, w13_s, w2, w2_s, expert_offset=offset, L=L)
    loc = O.apply_expert_map(ids, _slice_map(E, offset, L), L)
    b = O.fused_moe(hidden, loc, w, w13, w13_s, w2, w2_s, expert_offset=0, L=L)
    assert np.array_equal(a, b)


def test_act_quant_map_filter_keeps_the_mapped_local_rows():
    E = 24
    x, ids = synth.act_rows(96, 256, E, "map_filter", masked_frac=0.2)
    rng = np.random.default_rng(5)
    emap = rng.integers(-1, 3, E).astype(np.int32)
    q0 = np.full((96, 256), 0xAB, np.uint8)
    s0 = np.full((96, 2), -1.0, np.float32)
    q, s = O.silu_and_mul_quant_fp8(x, ids, emap, E, q_init=q0, s_init=s0)
    live = O.apply_expert_map(ids.numpy(), emap, 1 << 30) >= 0
    assert live.any() and (~live).any()
    assert (q[~live] == 0xAB).all() and (s[~live] == -1.0).all()
    q2, s2 = O.quant_fp8(O.silu_and_mul(x))
    assert np.array_equal(q[live], q2[live]) and np.array_equal(s[live].view(np.uint32), s2[live].view(np.uint32))
