"""The C-ABI library loads and exports every function include/bfp8moe.h
declares, and its host-side argument checks reject bad calls before anything
reaches the GPU (no device needed)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import block_fp8_mixture_route_amd as bfp8
from block_fp8_mixture_route_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp8moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route_prepare", "quant_fp8", "moe_fp8_grouped_gemm", "silu_and_mul_quant_fp8", "moe_reduce",
              "fused_moe_block_fp8", "silu_and_mul", "fused_moe_block_fp8_workspace_size", "bfp8moe_max_blocks", "moe_router_topk",
              "fused_moe_block_fp8_routed", "moe_router_noaux_tc", "fused_moe_block_fp8_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = bfp8.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    # and the binding's signature table covers them all
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_opts_layout_and_defaults():
    assert ctypes.sizeof(_lib.Opts) == 56  # 6 words, a pointer, 3 words and padding, a pointer
    o = bfp8.opts()
    assert o.block_m == 0 and o.scale_fmt == 0 and math.isinf(o.clamp_limit) and o.flags == 0
    assert o.weight_scale_mode == bfp8.WEIGHT_SCALE_BLOCK and o.act_static_scale == 0 and o.inter_static_scale == 0
    assert not o.expert_map


def test_opts_layout_matches_the_c_compiler(tmp_path):
    # every field's offset and the struct's size as gcc lays out the header's
    # struct, against the binding's ctypes mirror
    fields = [f for f, _ in _lib.Opts._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "bfp8moe.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(bfp8moe_opts_t));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(bfp8moe_opts_t, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert got[0] == ctypes.sizeof(_lib.Opts)
    assert got[1:] == [getattr(_lib.Opts, f).offset for f in fields]


def test_w8a8_layer_paths():
    o = bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL)
    # a few tokens: the few-token kernels in their W8A8 form, by default or forced
    token = ["token_gate_up_swiglu_channel", "token_down_reduce_channel"]
    assert bfp8.fused_moe_stages(1, 7168, 8, 256, 256, o) == token
    assert bfp8.fused_moe_stages(30, 2048, 8, 64, 128, bfp8.opts(weight_scale_mode=1,
                                                                  flags=bfp8.FLAG_LAYER_TOKEN)) == token
    general = ["route_prepare", "quant_fp8_rows", "gate_up_gemm_channel", "silu_and_mul_quant_rows",
               "down_gemm_channel", "moe_reduce"]
    assert bfp8.fused_moe_stages(1, 7168, 8, 256, 256, bfp8.opts(weight_scale_mode=1,
                                                                  flags=bfp8.FLAG_LAYER_GENERAL)) == general
    assert bfp8.fused_moe_stages(64, 7168, 8, 256, 256, o) == general
    # not the small-batch path, nor the few-token path at I = 768
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_stages(1, 7168, 8, 256, 256, bfp8.opts(weight_scale_mode=1, flags=bfp8.FLAG_LAYER_DECODE))
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_stages(1, 7168, 8, 256, 768, bfp8.opts(weight_scale_mode=1, flags=bfp8.FLAG_LAYER_TOKEN))
    with pytest.raises(bfp8.BFP8MoEError):  # rows beyond 8192
        bfp8.fused_moe_stages(1, 8320, 8, 256, 256, o)
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_stages(1, 7168, 8, 256, 256, bfp8.opts(weight_scale_mode=1, act_static_scale=-1.0))


def test_stage_lists():
    o = bfp8.opts()
    assert bfp8.fused_moe_stages(1, 7168, 8, 256, 256, o) == ["token_gate_up_swiglu", "token_down_reduce"]
    # the one-token path needs I in {128, 256, 512}; other shapes fall back
    assert bfp8.fused_moe_stages(1, 4096, 8, 256, 384, o) == ["decode_gate_up_swiglu", "decode_down_reduce"]
    # the few-token path up to 15 tokens (12 with per-channel weight scales);
    # the others when forced
    assert bfp8.fused_moe_stages(4, 7168, 8, 256, 256, o) == ["token_gate_up_swiglu", "token_down_reduce"]
    assert bfp8.fused_moe_stages(15, 7168, 8, 256, 256, o) == ["token_gate_up_swiglu", "token_down_reduce"]
    ch = bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL)
    assert bfp8.fused_moe_stages(12, 7168, 8, 256, 256, ch)[0] == "token_gate_up_swiglu_channel"
    assert not bfp8.fused_moe_stages(13, 7168, 8, 256, 256, ch)[0].startswith("token_")
    # the general path: route preparation carries the input quantisation
    # (one launch fewer) unless one workgroup sorts for more than 512 experts
    fused = ["route_prepare_quant", "gate_up_gemm", "silu_and_mul_quant", "down_gemm", "moe_reduce"]
    assert bfp8.fused_moe_stages(16, 7168, 8, 256, 256, o) == fused
    assert bfp8.fused_moe_stages(32, 7168, 8, 256, 256, o) == fused
    assert bfp8.fused_moe_stages(2048, 4096, 8, 512, 1024, o) == fused  # many-workgroup route prep
    assert bfp8.fused_moe_stages(64, 4096, 8, 1024, 256, o) == [
        "route_prepare", "quant_fp8", "gate_up_gemm", "silu_and_mul_quant", "down_gemm", "moe_reduce"]
    assert bfp8.fused_moe_stages(4, 7168, 8, 256, 256, bfp8.opts(flags=bfp8.FLAG_LAYER_DECODE)) == [
        "decode_gate_up_swiglu", "decode_down_reduce"]
    assert bfp8.fused_moe_stages(32, 7168, 8, 256, 256, bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN)) == [
        "token_gate_up_swiglu", "token_down_reduce"]
    assert bfp8.fused_moe_stages(512, 4096, 8, 256, 768, o)[1] == "gate_up_gemm"
    assert len(bfp8.fused_moe_stages(1, 7168, 8, 256, 256, bfp8.opts(flags=bfp8.FLAG_LAYER_GENERAL))) == 5
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_stages(64, 7168, 8, 256, 256, bfp8.opts(flags=bfp8.FLAG_LAYER_DECODE))
    with pytest.raises(bfp8.BFP8MoEError):
        bfp8.fused_moe_stages(33, 7168, 8, 256, 256, bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN))
    with pytest.raises(bfp8.BFP8MoEError):  # exclusive path flags
        bfp8.fused_moe_stages(1, 7168, 8, 256, 256,
                              bfp8.opts(flags=bfp8.FLAG_LAYER_TOKEN | bfp8.FLAG_LAYER_GENERAL))


def test_max_blocks_formula():
    assert bfp8.max_blocks(8, 256, 16) == 8
    assert bfp8.max_blocks(16384, 512, 64) == (16384 + 512 * 63) // 64
    assert bfp8.max_blocks(0, 8, 16) == 0


def _status(fn, *args):
    st = fn(*args)
    return st, bfp8.lib().bfp8moe_last_error().decode()


def test_stream_probe_rejects_bad_shapes():
    L = bfp8.lib()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    one_gib = 1 << 30
    for args, text in [((fake, one_gib, 3, 0, 128, 0, fake, 1 << 20), "pattern"),
                       ((fake, one_gib, 1, 4096, 512, 0, fake, 1 << 20), "piece"),
                       ((fake, one_gib, 1, 1000, 128, 0, fake, 1 << 20), "row_bytes"),
                       ((fake, one_gib, 1, 4096, 128, 170000, fake, 1 << 20), "lds_bytes"),
                       ((fake, one_gib, 0, 0, 128, 0, fake, 10), "sink holds"),
                       ((fake, 1000, 0, 0, 128, 0, fake, 10), "workgroups"),
                       ((P(0x1001), one_gib, 0, 0, 128, 0, fake, 1 << 20), "aligned")]:
        st, msg = _status(L.bfp8moe_stream_probe, *args, None)
        assert st == 1 and text in msg, (args, msg)


def test_host_validation_rejects_bad_calls():
    L = bfp8.lib()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    st, msg = _status(L.quant_fp8, fake, 4, 100, 0, fake, fake, None)
    assert st == 1 and "multiple of 128" in msg
    st, msg = _status(L.quant_fp8, fake, 4, 128, 7, fake, fake, None)
    assert st == 1 and "scale_fmt" in msg
    st, msg = _status(L.silu_and_mul_quant_fp8, fake, 4, 128, None, fake, 0, math.inf, 0, fake, fake, None)
    assert st == 1 and "expert_map requires" in msg
    st, msg = _status(L.moe_fp8_grouped_gemm, fake, fake, 8, fake, fake, 4, 256, 256, fake, fake, fake, fake, fake,
                      8, 24, 8, fake, None)
    assert st == 1 and "block_m" in msg
    st, msg = _status(L.moe_route_prepare, fake, 10, 0, 8, 16, fake, fake, fake, fake, 1, fake, None, 0, 0, None)
    assert st == 1 and "max_blocks" in msg
    st, msg = _status(L.moe_route_prepare, fake, 10, -1, 8, 16, fake, fake, None, None, 0, fake, None, 0, 0, None)
    assert st == 1 and "expert_offset" in msg
    st, msg = _status(L.moe_route_prepare, fake, 10, 0, 4096, 16, fake, fake, None, None, 0, fake, None, 0, 0, None)
    assert st == 2  # unsupported: more than 2048 local experts
    st, msg = _status(L.moe_route_prepare, fake, 100000, 0, 64, 16, fake, fake, None, None, 0, fake, None, 0, 0,
                      None)
    assert st == 3  # the multi-workgroup path needs a workspace
    o = bfp8.opts(expert_offset=200, local_num_experts=100)
    st, msg = _status(L.fused_moe_block_fp8, fake, 1, 7168, fake, fake, 8, fake, fake, fake, fake, 256, 256,
                      ctypes.byref(o), fake, fake, 1 << 30, None)
    assert st == 1 and "slice" in msg
    o = bfp8.opts()
    st, msg = _status(L.fused_moe_block_fp8, fake, 1, 7168, fake, fake, 8, fake, fake, fake, fake, 256, 256,
                      ctypes.byref(o), fake, fake, 16, None)
    assert st == 3 and "workspace" in msg
    o = bfp8.opts(flags=bfp8.FLAG_ONLY_STAGE(2))  # the one-token path has two stages
    st, msg = _status(L.fused_moe_block_fp8, fake, 1, 7168, fake, fake, 8, fake, fake, fake, fake, 256, 256,
                      ctypes.byref(o), fake, fake, 1 << 30, None)
    assert st == 1 and "stage 2" in msg
    st, msg = _status(L.moe_reduce, fake, fake, None, 0, 0, 2, 8, 100, fake, None)
    assert st == 1 and "multiple of 8" in msg
    st, msg = _status(L.moe_router_topk, fake, 1 << 34, 256, 8, 0, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "out of range" in msg
    st, msg = _status(L.moe_router_topk, fake, 4, 2048, 8, 0, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "E=2048" in msg
    st, msg = _status(L.moe_router_topk, fake, 4, 16, 17, 0, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "k=17" in msg
    st, msg = _status(L.moe_router_topk, fake, 4, 256, 8, 0, fake, 1, 1.0, fake, fake, None)
    assert st == 1 and "sigmoid" in msg
    st, msg = _status(L.moe_router_topk, fake, 4, 256, 8, 2, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "score_fn" in msg
    st, msg = _status(L.moe_router_topk, fake, 4, 256, 8, 1, None, 1, math.nan, fake, fake, None)
    assert st == 1 and "scale" in msg
    o = bfp8.opts(flags=bfp8.FLAG_ONLY_STAGE(0))
    st, msg = _status(L.fused_moe_block_fp8_routed, fake, 1, 7168, fake, None, 0, 1, 1.0, 1, 1, 8, fake, fake, fake, fake,
                      fake, fake, 256, 256, ctypes.byref(o), fake, fake, 1 << 30, None)
    assert st == 1 and "stage" in msg
    o = bfp8.opts()
    st, msg = _status(L.fused_moe_block_fp8_routed, fake, 1, 7168, fake, None, 0, 1, 1.0, 1, 1, 8, fake, fake, fake, fake,
                      fake, fake, 256, 256, ctypes.byref(o), fake, fake, 16, None)
    assert st == 3 and "workspace" in msg
    st, msg = _status(L.fused_moe_block_fp8_routed, fake, 1, 7168, fake, fake, 0, 1, 1.0, 1, 1, 8, fake, fake, fake, fake,
                      fake, fake, 256, 256, ctypes.byref(o), fake, fake, 1 << 30, None)
    assert st == 1 and "sigmoid" in msg
    # grouped selection: n_group must divide E, topk_group <= n_group, sigmoid scoring
    for ng, tg, sf, what in ((7, 1, 1, "n_group"), (8, 9, 1, "topk_group"), (8, 4, 0, "sigmoid")):
        st, msg = _status(L.fused_moe_block_fp8_routed, fake, 1, 7168, fake, None, sf, 1, 1.0, ng, tg, 8, fake, fake,
                          fake, fake, fake, fake, 256, 256, ctypes.byref(o), fake, fake, 1 << 30, None)
        assert st == 1 and what in msg, msg
    # the router in route preparation: general path, one route-prep workgroup, at most 64 tokens
    for M, flags in ((1, 0), (65, bfp8.FLAG_LAYER_GENERAL), (16, bfp8.FLAG_LAYER_GENERAL | bfp8.FLAG_ROUTE_MULTI_WG)):
        o = bfp8.opts(flags=flags | bfp8.FLAG_ROUTER_IN_ROUTE_PREP)
        st, msg = _status(L.fused_moe_block_fp8_routed, fake, M, 7168, fake, None, 0, 1, 1.0, 1, 1, 8, fake, fake,
                          fake, fake, fake, fake, 256, 256, ctypes.byref(o), fake, fake, 1 << 30, None)
        assert st == 2 and "router in route preparation" in msg, msg
    st, msg = _status(L.moe_router_noaux_tc, fake, 4, 256, 8, 6, 2, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "n_group" in msg
    st, msg = _status(L.moe_router_noaux_tc, fake, 4, 256, 80, 8, 2, None, 1, 1.0, fake, fake, None)
    assert st == 1 and "k=80" in msg


def test_router_binding_checks_buffers():
    import torch
    from block_fp8_mixture_route_amd import _lib as B
    with pytest.raises(ValueError):
        B._check_router_buffers(256, 8, 4, torch.zeros(255), None, None)
    with pytest.raises(ValueError):
        B._check_router_buffers(256, 8, 4, None, torch.zeros(4, 8, dtype=torch.int64), None)
    with pytest.raises(ValueError):
        B._check_router_buffers(256, 8, 4, None, None, torch.zeros(4, 7))
    B._check_router_buffers(256, 8, 4, torch.zeros(256), torch.zeros(4, 8, dtype=torch.int32), torch.zeros(4, 8))


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        bfp8.quant_fp8(torch.zeros(1, 128, dtype=torch.bfloat16))


def test_mxfp4_layer_host_checks():
    o = bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4)
    assert bfp8.fused_moe_stages(64, 2048, 8, 32, 768, o) == [
        "route_prepare_quant", "gate_up_gemm_mxfp4", "silu_and_mul_quant", "down_gemm_mxfp4", "moe_reduce"]
    # a few tokens take the few-token kernels in their MXFP4 form, forced or by default
    token = ["token_gate_up_swiglu_mxfp4", "token_down_reduce_mxfp4"]
    assert bfp8.fused_moe_stages(1, 7168, 8, 256, 256, o) == token
    assert bfp8.fused_moe_stages(8, 7168, 8, 256, 256, o) == token
    assert bfp8.fused_moe_stages(9, 7168, 8, 256, 256, o)[0] == "route_prepare_quant"  # the general path from 9
    assert bfp8.fused_moe_stages(20, 2048, 8, 64, 512, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4,
                                                                  flags=bfp8.FLAG_LAYER_TOKEN)) == token
    assert bfp8.fused_moe_stages(1, 7168, 8, 256, 256, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4,
                                                                  flags=bfp8.FLAG_LAYER_GENERAL))[1] == \
        "gate_up_gemm_mxfp4"
    # refused: I = 128 (not whole 256-wide chunks), the few-token path forced at I = 768 or 33 tokens,
    # the small-batch path, static scales
    for M, I, bad in ((4, 128, dict()), (4, 768, dict(flags=bfp8.FLAG_LAYER_TOKEN)),
                      (33, 256, dict(flags=bfp8.FLAG_LAYER_TOKEN)), (4, 256, dict(flags=bfp8.FLAG_LAYER_DECODE)),
                      (4, 256, dict(act_static_scale=0.5))):
        with pytest.raises(bfp8.BFP8MoEError):
            bfp8.fused_moe_stages(M, 256, 2, 8, I, bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4, **bad))
    # byte scales do not go through the fp32-scale entry point, nor block scales through fused_moe_mxfp4
    # (both fail in the host checks, before anything is launched)
    st = _lib.lib().fused_moe_block_fp8(None, 0, 256, None, None, 2, None, None, None, None, 8, 256,
                                        ctypes.byref(o), None, None, 0, None)
    assert st == 1
    st = _lib.lib().fused_moe_mxfp4(None, 0, 256, None, None, 2, None, None, None, None, 8, 256,
                                    ctypes.byref(bfp8.opts()), None, None, 0, None)
    assert st == 1
    assert _lib.lib().fused_moe_mxfp4(None, 0, 256, None, None, 2, None, None, None, None, 8, 256, None, None,
                                      None, 0, None) == 1
