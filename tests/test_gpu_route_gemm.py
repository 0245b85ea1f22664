"""GPU parity (through the C ABI) for moe_route_prepare (bit-exact, both
implementations at every size) and moe_fp8_grouped_gemm (within tolerance)."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests.gpu_util import assert_gemm_close, bf16_np, dev, print_case

pytestmark = pytest.mark.gpu

ROUTE_FLAGS = {"auto": 0, "single": bfp8.FLAG_ROUTE_SINGLE_WG, "multi": bfp8.FLAG_ROUTE_MULTI_WG}


def _cmp_route(ids_cpu, offset, L, B, flags, with_blocks=True):
    got = bfp8.moe_route_prepare(ids_cpu.to(dev()), offset, L, B, with_blocks=with_blocks, flags=flags)
    torch.cuda.synchronize()
    ref = O.route_prepare(ids_cpu, offset, L, B)
    assert (got["sorted_routes"].cpu().numpy() == ref["sorted_routes"]).all()
    assert (got["expert_offsets"].cpu().numpy() == ref["expert_offsets"]).all()
    assert int(got["num_blocks"].item()) == ref["num_blocks"]
    if with_blocks:
        mb = ref["max_blocks"]
        assert (got["block_expert"][:mb].cpu().numpy() == ref["block_expert"]).all()
        assert (got["block_start"][:mb].cpu().numpy() == ref["block_start"]).all()
    return got


@pytest.mark.parametrize("path", ["auto", "single", "multi"])
@pytest.mark.parametrize("case", ["tiny", "decode_m1", "decode_m4", "decode_m16", "decode_m32", "small_m128",
                                  "small_m512", "large_m2048"])
@pytest.mark.parametrize("B", [16, 64])
def test_route_prepare_workloads(case, path, B):
    c = synth.LAYER_CASES[case]
    if path == "single" and c.M * c.k > 16384:
        pytest.skip("single workgroup path is exercised up to 16384 routes")
    print_case("route", case, path, B)
    ids, _ = synth.routing_for(c, 0)
    _cmp_route(ids, 0, c.E, B, ROUTE_FLAGS[path])


@pytest.mark.parametrize("path", ["single", "multi"])
def test_route_prepare_edges(path):
    f = ROUTE_FLAGS[path]
    print_case("route edges", path)
    g = torch.Generator().manual_seed(3)
    # random ids with invalid entries, local slices, odd block sizes
    for R, E, off, L, B in [(1, 1, 0, 1, 1), (37, 10, 0, 10, 3), (5000, 300, 100, 150, 16), (2048, 512, 0, 512, 7),
                            (3000, 2048, 0, 2048, 16), (4097, 64, 32, 32, 64)]:
        ids = torch.randint(-1, E + 5, (R,), generator=g, dtype=torch.int32)
        _cmp_route(ids, off, L, B, f)
        _cmp_route(ids, off, L, B, f, with_blocks=False)
    # every route masked
    _cmp_route(torch.full((100,), -1, dtype=torch.int32), 0, 8, 16, f)
    # a single expert takes every route
    _cmp_route(torch.full((3000,), 5, dtype=torch.int32), 0, 8, 16, f)


def test_route_prepare_zero_routes():
    print_case("route zero")
    for f in ROUTE_FLAGS.values():
        got = bfp8.moe_route_prepare(torch.empty(0, dtype=torch.int32, device=dev()), 0, 8, 16, flags=f)
        torch.cuda.synchronize()
        assert int(got["num_blocks"].item()) == 0
        assert (got["expert_offsets"].cpu() == 0).all()


def _gemm_case(R_tokens, k, E, N, K, B, seed, a_row_div_mode="gate_up", invalid=True):
    ids, _ = synth.uniform_routing(R_tokens, E, k, "gemm", seed)
    if invalid:
        ids.view(-1)[::7] = -1
    R = R_tokens * k
    rows = R_tokens if a_row_div_mode == "gate_up" else R
    a_row_div = k if a_row_div_mode == "gate_up" else 1
    A, As = O.quant_fp8(synth.hidden_states(rows, K, "gemm_a", seed))
    Bw = torch.empty(E, N, K, dtype=torch.uint8)
    Bs = torch.empty(E, N // 128, K // 128)
    for e in range(E):
        c, s = synth.block_fp8_weight(N, K, "gemm_b", seed, e)
        Bw[e], Bs[e] = c, s
    route = bfp8.moe_route_prepare(ids.to(dev()), 0, E, B)
    C0 = torch.full((R, N), 1.5, dtype=torch.bfloat16)
    C = bfp8.moe_fp8_grouped_gemm(torch.from_numpy(A).to(dev()), torch.from_numpy(As).to(dev()), a_row_div,
                                  Bw.to(dev()), Bs.to(dev()), route, B, R, C=C0.to(dev()))
    torch.cuda.synchronize()
    ref = O.grouped_gemm(A, As, a_row_div, Bw, Bs, ids, 0, E, C_init=bf16_np(C0))
    return bf16_np(C), ref, ids


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("shape", [(4, 2, 8, 256, 256), (16, 8, 32, 512, 1024), (64, 8, 16, 384, 512),
                                   (3, 8, 32, 512, 7168), (40, 4, 4, 256, 768)])
def test_grouped_gemm_gate_up(shape, B):
    Mt, k, E, N, K = shape
    print_case("gemm gate_up", shape, B)
    got, ref, ids = _gemm_case(Mt, k, E, N, K, B, seed=Mt * 31 + E)
    valid = (ids.view(-1) >= 0).numpy()
    assert (got[~valid] == ref[~valid]).all()  # untouched rows
    assert_gemm_close(got[valid], ref[valid], f"gate_up {shape} B={B}")


@pytest.mark.parametrize("B", [16, 64])
@pytest.mark.parametrize("shape", [(2, 8, 16, 7168, 256), (32, 8, 8, 1024, 384), (8, 8, 64, 4096, 768)])
def test_grouped_gemm_down(shape, B):
    Mt, k, E, N, K = shape
    print_case("gemm down", shape, B)
    got, ref, ids = _gemm_case(Mt, k, E, N, K, B, seed=Mt * 17 + N, a_row_div_mode="down")
    valid = (ids.view(-1) >= 0).numpy()
    assert (got[~valid] == ref[~valid]).all()
    assert_gemm_close(got[valid], ref[valid], f"down {shape} B={B}")


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("K", [128, 256, 384, 512, 640, 768, 896, 1152])
def test_grouped_gemm_k_loop_tails(K, B):
    # 1 to 7 and 9 K chunks: every remainder of the loops that keep two
    # chunks in flight (three steps per iteration) and one (two steps), twice
    # over, and both sides of the chunk count from which the block scales are
    # staged in LDS
    print_case("gemm k tails", K, B)
    got, ref, ids = _gemm_case(8, 4, 8, 256, K, B, seed=K + B)
    valid = (ids.view(-1) >= 0).numpy()
    assert (got[~valid] == ref[~valid]).all()
    assert_gemm_close(got[valid], ref[valid], f"k tails K={K} B={B}")


def test_grouped_gemm_hot_expert():
    # one expert takes 200 routes (13 blocks of 16): blocks of one expert in a row
    print_case("gemm hot expert")
    E, N, K, k, Mt = 4, 256, 512, 8, 25
    ids = torch.zeros(Mt, k, dtype=torch.int32)
    ids[:, 1::2] = torch.arange(Mt * k // 2, dtype=torch.int32).reshape(Mt, k // 2) % 3 + 1
    A, As = O.quant_fp8(synth.hidden_states(Mt, K, "hot", 0))
    Bw = torch.empty(E, N, K, dtype=torch.uint8)
    Bs = torch.empty(E, N // 128, K // 128)
    for e in range(E):
        Bw[e], Bs[e] = synth.block_fp8_weight(N, K, "hot_b", e)
    route = bfp8.moe_route_prepare(ids.to(dev()), 0, E, 16)
    C = bfp8.moe_fp8_grouped_gemm(torch.from_numpy(A).to(dev()), torch.from_numpy(As).to(dev()), k, Bw.to(dev()),
                                  Bs.to(dev()), route, 16, Mt * k)
    torch.cuda.synchronize()
    ref = O.grouped_gemm(A, As, k, Bw, Bs, ids, 0, E)
    assert_gemm_close(bf16_np(C), ref, "hot expert")


@pytest.mark.parametrize("B", [16, 32])
def test_grouped_gemm_many_blocks(B):
    # 601 experts of one route each: 601 blocks, all in use, the most the
    # routing allows; from 512 blocks up the tiles go to the XCDs in pairs of
    # blocks, and 601 leaves a last pair of one block
    print_case("gemm many blocks", B)
    E, N, K, k, Mt = 601, 256, 256, 1, 601
    g = torch.Generator().manual_seed(601)
    ids = torch.randperm(E, generator=g).to(torch.int32).reshape(Mt, k)
    A, As = O.quant_fp8(synth.hidden_states(Mt, K, "many", 0))
    Bw = torch.empty(E, N, K, dtype=torch.uint8)
    Bs = torch.empty(E, N // 128, K // 128)
    for e in range(E):
        Bw[e], Bs[e] = synth.block_fp8_weight(N, K, "many_b", e)
    route = bfp8.moe_route_prepare(ids.to(dev()), 0, E, B)
    torch.cuda.synchronize()
    assert int(route["num_blocks"].item()) == E == bfp8.max_blocks(Mt * k, E, B)
    C = bfp8.moe_fp8_grouped_gemm(torch.from_numpy(A).to(dev()), torch.from_numpy(As).to(dev()), k, Bw.to(dev()),
                                  Bs.to(dev()), route, B, Mt * k)
    torch.cuda.synchronize()
    ref = O.grouped_gemm(A, As, k, Bw, Bs, ids, 0, E)
    assert_gemm_close(bf16_np(C), ref, f"many blocks B={B}")
