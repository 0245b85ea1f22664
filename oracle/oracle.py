"""ctypes front-end for the C oracle (bfp8moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the library.  Arrays are numpy
(BF16 travels as uint16 bit patterns, E4M3 as uint8 codes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bfp8moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

SCALE_FP32 = 0
SCALE_UE8M0 = 1


SAN_LIB = os.path.join(HERE, "liboracle_san.so")


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile the oracle with gcc: -O2, no FP contraction, no fast-math.
    sanitize: a separate build with AddressSanitizer and
    UndefinedBehaviorSanitizer (gcc's libasan must then be preloaded)."""
    out = SAN_LIB if sanitize else LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(SRC):
        tmp = out + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-std=gnu11", "-Wall", "-shared", "-fPIC", *(san if sanitize else []), SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        # BFP8MOE_ORACLE_LIB names another build (the sanitized one of
        # tests/run_sanitized.py); by default this directory's, built on demand
        path = os.environ.get("BFP8MOE_ORACLE_LIB") or build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "oracle_bf16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [f32]),
            "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "oracle_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [f32]),
            "oracle_group_scale": (f32, [f32, i32]),
            "oracle_quant_fp8": (None, [P, i64, i32, i32, P, P]),
            "oracle_exp_rn": (f32, [f32]),
            "oracle_swiglu_one": (ctypes.c_uint16, [ctypes.c_uint16, ctypes.c_uint16, f32]),
            "oracle_silu_and_mul": (None, [P, i64, i32, f32, P]),
            "oracle_silu_and_mul_quant_fp8": (None, [P, i64, i32, P, P, i32, f32, i32, P, P]),
            "oracle_max_blocks": (i64, [i64, i32, i32]),
            "oracle_route_prepare": (i64, [P, i64, i32, i32, i32, P, P, P, P, i64, P]),
            "oracle_grouped_gemm": (None, [P, P, i32, P, P, i32, i32, P, i64, i32, i32, P]),
            "oracle_grouped_gemm_f64": (None, [P, P, i32, P, P, i32, i32, P, i64, i32, i32, P, P]),
            "oracle_moe_reduce": (None, [P, P, P, i32, i32, i64, i32, i32, P]),
            "oracle_sigmoid_rn": (f32, [f32]),
            "oracle_router_topk": (None, [P, i64, i32, i32, i32, P, i32, ctypes.c_double, P, P]),
            "oracle_router_noaux_tc": (None, [P, i64, i32, i32, i32, i32, P, i32, ctypes.c_double, P, P]),
            "oracle_quant_fp8_rows": (None, [P, i64, i32, i32, f32, P, P]),
            "oracle_silu_and_mul_quant_fp8_rows": (None, [P, i64, i32, P, P, i32, f32, i32, f32, P, P]),
            "oracle_grouped_gemm_channel": (None, [P, P, i32, P, P, i32, i32, P, i64, i32, i32, P, P, P]),
            "oracle_fused_moe_w8a8": (None, [P, i64, i32, P, P, i32, P, P, P, P, i32, i32, i32, i32, f32, f32, f32,
                                             P, P, P, P, P]),
            "oracle_fused_moe": (None, [P, i64, i32, P, P, i32, P, P, P, P, i32, i32, i32, i32, f32,
                                        P, i64, P, P, P, P, P]),
            "oracle_e2m1_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_e8m0_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_grouped_gemm_mxfp4": (None, [P, P, i32, P, P, i32, i32, P, i64, i32, i32, P, P, P]),
            "oracle_fused_moe_mxfp4": (None, [P, i64, i32, P, P, i32, P, P, P, P, i32, i32, i32, i32, f32,
                                              P, P, P, P, P]),
            "oracle_num_threads": (i32, []),
            "oracle_set_threads": (None, [i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def as_np(t, dtype=None):
    """torch tensor (CPU or GPU) or numpy array -> contiguous numpy array.
    BF16 tensors come out as uint16 bit patterns, float8 as uint8 codes."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
                return t.numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                t = t.view(torch.uint8)
            t = t.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(t)
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a


# ---------------------------------------------------------------- scalars

def e4m3_decode(c: int) -> float:
    return lib().oracle_e4m3_decode(c)


def e4m3_encode(x: float) -> int:
    return lib().oracle_e4m3_encode(x)


def f32_to_bf16(x: float) -> int:
    return lib().oracle_f32_to_bf16(x)


def f64_to_bf16(x: float) -> int:
    return lib().oracle_f64_to_bf16(x)


def bf16_to_f64(h: int) -> float:
    return lib().oracle_bf16_to_f64(h)


def exp_rn(x: float) -> float:
    return lib().oracle_exp_rn(x)


def group_scale(amax: float, fmt: int) -> float:
    return lib().oracle_group_scale(amax, fmt)


def swiglu_one(gate: int, up: int, clamp: float = float("inf")) -> int:
    return lib().oracle_swiglu_one(gate, up, clamp)


# ---------------------------------------------------------------- arrays

def quant_fp8(x_bf16: np.ndarray, fmt: int = SCALE_FP32):
    x = as_np(x_bf16, np.uint16)
    rows, K = x.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros((rows, K // 128), np.float32)
    lib().oracle_quant_fp8(_p(x), rows, K, fmt, _p(q), _p(s))
    return q, s


def silu_and_mul(gate_up_bf16, clamp: float = float("inf")):
    x = as_np(gate_up_bf16, np.uint16)
    rows, I2 = x.shape
    out = np.zeros((rows, I2 // 2), np.uint16)
    lib().oracle_silu_and_mul(_p(x), rows, I2 // 2, clamp, _p(out))
    return out


def silu_and_mul_quant_fp8(gate_up_bf16, row_expert_ids=None, expert_map=None, E: int = 0,
                           clamp: float = float("inf"), fmt: int = SCALE_FP32,
                           q_init=None, s_init=None):
    x = as_np(gate_up_bf16, np.uint16)
    rows, I2 = x.shape
    I = I2 // 2
    q = np.zeros((rows, I), np.uint8) if q_init is None else np.array(q_init, np.uint8, copy=True)
    s = np.zeros((rows, I // 128), np.float32) if s_init is None else np.array(s_init, np.float32, copy=True)
    ids = None if row_expert_ids is None else as_np(row_expert_ids, np.int32)
    emap = None if expert_map is None else as_np(expert_map, np.int32)
    lib().oracle_silu_and_mul_quant_fp8(_p(x), rows, I, _p(ids), _p(emap), E, clamp, fmt, _p(q), _p(s))
    return q, s


def max_blocks(R: int, L: int, block_m: int) -> int:
    return lib().oracle_max_blocks(R, L, block_m)


def apply_expert_map(topk_ids, expert_map, L: int):
    """Local expert ids under an expert map (vLLM PR "[Kernel][Perf] Fuse
    clamped MoE activation and UE8M0 FP8 block quantization", Purpose: rows
    of experts the map marks non-local are filtered out).  Reading: global id
    i selects local expert expert_map[i]; an id outside [0, E) or an entry
    outside [0, L) leaves the route masked (-1).  The result feeds every
    other oracle function with expert_offset 0 and L local experts, so the
    map form of each step is that step on the mapped ids."""
    ids = as_np(topk_ids, np.int32)
    emap = as_np(expert_map, np.int32).reshape(-1)
    out = np.full(ids.shape, -1, np.int32)
    for idx in np.ndindex(ids.shape):
        g = int(ids[idx])
        if 0 <= g < emap.size:
            e = int(emap[g])
            if 0 <= e < L:
                out[idx] = e
    return out


def route_prepare(topk_ids, expert_offset: int, L: int, block_m: int, with_blocks: bool = True):
    ids = as_np(topk_ids, np.int32).reshape(-1)
    R = ids.size
    mb = max_blocks(R, L, block_m)
    sorted_routes = np.zeros(R, np.int32)
    offsets = np.zeros(L + 1, np.int32)
    be = np.zeros(mb, np.int32) if with_blocks else None
    bs = np.zeros(mb, np.int32) if with_blocks else None
    nb = np.zeros(1, np.int32)
    lib().oracle_route_prepare(_p(ids), R, expert_offset, L, block_m, _p(sorted_routes), _p(offsets),
                               _p(be), _p(bs), mb, _p(nb))
    return dict(sorted_routes=sorted_routes, expert_offsets=offsets, block_expert=be, block_start=bs,
                num_blocks=int(nb[0]), max_blocks=mb)


def grouped_gemm(A, A_s, a_row_div: int, B, B_s, topk_ids, expert_offset: int, L: int, C_init=None):
    A = as_np(A, np.uint8); A_s = as_np(A_s, np.float32)
    B = as_np(B, np.uint8); B_s = as_np(B_s, np.float32)
    ids = as_np(topk_ids, np.int32).reshape(-1)
    N, K = B.shape[1], B.shape[2]
    R = ids.size
    C = np.zeros((R, N), np.uint16) if C_init is None else np.array(C_init, np.uint16, copy=True)
    lib().oracle_grouped_gemm(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R,
                              expert_offset, L, _p(C))
    return C


def grouped_gemm_f64(A, A_s, a_row_div: int, B, B_s, topk_ids, expert_offset: int, L: int):
    """The grouped GEMM before its BF16 rounding: ([R, N] fp64 values, [R, N]
    fp64 magnitude bounds sum |scale products| * |code products|).  Rows of
    dropped routes are NaN."""
    A = as_np(A, np.uint8); A_s = as_np(A_s, np.float32)
    B = as_np(B, np.uint8); B_s = as_np(B_s, np.float32)
    ids = as_np(topk_ids, np.int32).reshape(-1)
    N, K = B.shape[1], B.shape[2]
    R = ids.size
    acc = np.full((R, N), np.nan)
    mag = np.full((R, N), np.nan)
    lib().oracle_grouped_gemm_f64(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R,
                                  expert_offset, L, _p(acc), _p(mag))
    return acc, mag


def moe_reduce(y_bf16, topk_w, topk_ids=None, expert_offset: int = 0, L: int = 1 << 30):
    y = as_np(y_bf16, np.uint16)
    w = as_np(topk_w, np.float32)
    M, k = w.shape
    H = y.shape[1]
    ids = None if topk_ids is None else as_np(topk_ids, np.int32)
    out = np.zeros((M, H), np.uint16)
    lib().oracle_moe_reduce(_p(y), _p(w), _p(ids), expert_offset, L, M, k, H, _p(out))
    return out


SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


def router_topk(logits, k: int, score_fn: int = SCORE_SOFTMAX, bias=None, renormalize: bool = True,
                scale: float = 1.0):
    """Top-k experts per token from [M, E] fp32 router logits: ([M, k] int32
    ids, largest first, and [M, k] fp32 weights)."""
    lg = as_np(logits, np.float32)
    M, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError(f"k={k} must be in [1, E={E}]")
    b = None if bias is None else as_np(bias, np.float32)
    if b is not None and b.size != E:
        raise ValueError("the selection bias needs one value per expert")
    ids = np.zeros((M, k), np.int32)
    w = np.zeros((M, k), np.float32)
    lib().oracle_router_topk(_p(lg), M, E, k, score_fn, _p(b), int(bool(renormalize)), float(scale), _p(ids), _p(w))
    return ids, w


def router_noaux_tc(logits, k: int, n_group: int, topk_group: int, bias=None, renormalize: bool = True,
                    scale: float = 1.0):
    """Group-limited noaux-TC routing of [M, E] fp32 logits: ([M, k] int32 ids,
    largest key first, [M, k] fp32 weights)."""
    lg = as_np(logits, np.float32)
    M, E = lg.shape
    if n_group < 1 or E % n_group or not 1 <= topk_group <= n_group or not 1 <= k <= topk_group * (E // n_group):
        raise ValueError(f"bad grouping: E={E} n_group={n_group} topk_group={topk_group} k={k}")
    b = None if bias is None else as_np(bias, np.float32)
    if b is not None and b.size != E:
        raise ValueError("the selection bias needs one value per expert")
    ids = np.zeros((M, k), np.int32)
    w = np.zeros((M, k), np.float32)
    lib().oracle_router_noaux_tc(_p(lg), M, E, k, n_group, topk_group, _p(b), int(bool(renormalize)), float(scale),
                                 _p(ids), _p(w))
    return ids, w


def sigmoid_rn(x: float) -> float:
    return lib().oracle_sigmoid_rn(x)


def fused_moe(hidden, topk_ids, topk_w, w13, w13_s, w2, w2_s, expert_offset: int = 0, L: int = None,
              scale_fmt: int = SCALE_FP32, clamp: float = float("inf"), tokens=None,
              want_intermediates: bool = False):
    """Whole layer for all tokens, or for the listed token subset.  Returns the
    [M, H] BF16 output (rows of unlisted tokens are zero) and, optionally, the
    intermediates keyed by route id."""
    h = as_np(hidden, np.uint16)
    ids = as_np(topk_ids, np.int32)
    w = as_np(topk_w, np.float32)
    w13 = as_np(w13, np.uint8); w13_s = as_np(w13_s, np.float32)
    w2 = as_np(w2, np.uint8); w2_s = as_np(w2_s, np.float32)
    M, H = h.shape
    k = ids.shape[1]
    Lw = w13.shape[0]
    if L is None:
        L = Lw
    I = w2.shape[2]
    out = np.zeros((M, H), np.uint16)
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int64))
    nt = M if tok is None else tok.size
    inter = None
    if want_intermediates:
        inter = dict(h13=np.zeros((M * k, 2 * I), np.uint16), q=np.zeros((M * k, I), np.uint8),
                     s=np.zeros((M * k, I // 128), np.float32), y=np.zeros((M * k, H), np.uint16))
    lib().oracle_fused_moe(_p(h), M, H, _p(ids), _p(w), k, _p(w13), _p(w13_s), _p(w2), _p(w2_s),
                           expert_offset, L, I, scale_fmt, clamp, _p(tok), nt, _p(out),
                           _p(inter["h13"]) if inter else None, _p(inter["q"]) if inter else None,
                           _p(inter["s"]) if inter else None, _p(inter["y"]) if inter else None)
    return (out, inter) if want_intermediates else out


# ---------------------------------------------------------------- W8A8 variant

def quant_fp8_rows(x_bf16, fmt: int = SCALE_FP32, static_scale: float = 0.0):
    """One scale per row (static when > 0, else the row's amax / 448): ([rows, K]
    codes, [rows] scales)."""
    x = as_np(x_bf16, np.uint16)
    rows, K = x.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros(rows, np.float32)
    lib().oracle_quant_fp8_rows(_p(x), rows, K, fmt, static_scale, _p(q), _p(s))
    return q, s


def silu_and_mul_quant_fp8_rows(gate_up_bf16, row_expert_ids=None, expert_map=None, E: int = 0,
                                clamp: float = float("inf"), fmt: int = SCALE_FP32, static_scale: float = 0.0,
                                q_init=None, s_init=None):
    x = as_np(gate_up_bf16, np.uint16)
    rows, I2 = x.shape
    I = I2 // 2
    q = np.zeros((rows, I), np.uint8) if q_init is None else np.array(q_init, np.uint8, copy=True)
    s = np.zeros(rows, np.float32) if s_init is None else np.array(s_init, np.float32, copy=True)
    ids = None if row_expert_ids is None else as_np(row_expert_ids, np.int32)
    emap = None if expert_map is None else as_np(expert_map, np.int32)
    lib().oracle_silu_and_mul_quant_fp8_rows(_p(x), rows, I, _p(ids), _p(emap), E, clamp, fmt, static_scale, _p(q),
                                            _p(s))
    return q, s


def grouped_gemm_channel(A, A_s, a_row_div: int, B, B_s, topk_ids, expert_offset: int, L: int, exact=False):
    """Per-row activation scales A_s [rows], per-channel weight scales B_s [L, N].
    exact: ([R, N] fp64 values, magnitudes) instead of [R, N] BF16 bits."""
    A = as_np(A, np.uint8); A_s = as_np(A_s, np.float32)
    B = as_np(B, np.uint8); B_s = as_np(B_s, np.float32)
    ids = as_np(topk_ids, np.int32).reshape(-1)
    N, K = B.shape[1], B.shape[2]
    R = ids.size
    if exact:
        acc = np.full((R, N), np.nan)
        mag = np.full((R, N), np.nan)
        lib().oracle_grouped_gemm_channel(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R,
                                          expert_offset, L, None, _p(acc), _p(mag))
        return acc, mag
    C = np.zeros((R, N), np.uint16)
    lib().oracle_grouped_gemm_channel(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R, expert_offset, L,
                                      _p(C), None, None)
    return C


def fused_moe_w8a8(hidden, topk_ids, topk_w, w13, w13_s, w2, w2_s, expert_offset: int = 0, L: int = None,
                   scale_fmt: int = SCALE_FP32, a1_static: float = 0.0, a2_static: float = 0.0,
                   clamp: float = float("inf"), want_intermediates: bool = False):
    """The W8A8 layer (w13_s [L, 2I], w2_s [L, H]): [M, H] BF16 output and
    optionally the intermediates keyed by route id (s is [M*k])."""
    h = as_np(hidden, np.uint16)
    ids = as_np(topk_ids, np.int32)
    w = as_np(topk_w, np.float32)
    w13 = as_np(w13, np.uint8); w13_s = as_np(w13_s, np.float32)
    w2 = as_np(w2, np.uint8); w2_s = as_np(w2_s, np.float32)
    M, H = h.shape
    k = ids.shape[1]
    L = w13.shape[0] if L is None else L
    I = w2.shape[2]
    out = np.zeros((M, H), np.uint16)
    inter = None
    if want_intermediates:
        inter = dict(h13=np.zeros((M * k, 2 * I), np.uint16), q=np.zeros((M * k, I), np.uint8),
                     s=np.zeros(M * k, np.float32), y=np.zeros((M * k, H), np.uint16))
    lib().oracle_fused_moe_w8a8(_p(h), M, H, _p(ids), _p(w), k, _p(w13), _p(w13_s), _p(w2), _p(w2_s), expert_offset,
                                L, I, scale_fmt, a1_static, a2_static, clamp, _p(out),
                                _p(inter["h13"]) if inter else None, _p(inter["q"]) if inter else None,
                                _p(inter["s"]) if inter else None, _p(inter["y"]) if inter else None)
    return (out, inter) if want_intermediates else out


def e2m1_decode(c: int) -> float:
    return lib().oracle_e2m1_decode(c)


def e8m0_decode(e: int) -> float:
    return lib().oracle_e8m0_decode(e)


def grouped_gemm_mxfp4(A, A_s, a_row_div: int, B, B_s, topk_ids, expert_offset: int, L: int, exact=False):
    """MXFP4 weights B [L, N, K/2] (packed E2M1, even element in the low
    nibble) with E8M0 scale bytes B_s [L, N, K/32]; E4M3 activations with
    group-128 scales.  exact: ([R, N] fp64 values, magnitudes) instead of
    [R, N] BF16 bits."""
    A = as_np(A, np.uint8); A_s = as_np(A_s, np.float32)
    B = as_np(B, np.uint8); B_s = as_np(B_s, np.uint8)
    ids = as_np(topk_ids, np.int32).reshape(-1)
    N, K = B.shape[1], 2 * B.shape[2]
    R = ids.size
    if exact:
        acc = np.full((R, N), np.nan)
        mag = np.full((R, N), np.nan)
        lib().oracle_grouped_gemm_mxfp4(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R, expert_offset,
                                        L, None, _p(acc), _p(mag))
        return acc, mag
    C = np.zeros((R, N), np.uint16)
    lib().oracle_grouped_gemm_mxfp4(_p(A), _p(A_s), a_row_div, _p(B), _p(B_s), N, K, _p(ids), R, expert_offset, L,
                                    _p(C), None, None)
    return C


def fused_moe_mxfp4(hidden, topk_ids, topk_w, w13, w13_s, w2, w2_s, expert_offset: int = 0, L: int = None,
                    scale_fmt: int = SCALE_FP32, clamp: float = float("inf"), want_intermediates: bool = False):
    """The layer with MXFP4 weights (w13 [L, 2I, H/2], w13_s [L, 2I, H/32],
    w2 [L, H, I/2], w2_s [L, H, I/32]): [M, H] BF16 output and optionally
    the intermediates keyed by route id."""
    h = as_np(hidden, np.uint16)
    ids = as_np(topk_ids, np.int32)
    w = as_np(topk_w, np.float32)
    w13 = as_np(w13, np.uint8); w13_s = as_np(w13_s, np.uint8)
    w2 = as_np(w2, np.uint8); w2_s = as_np(w2_s, np.uint8)
    M, H = h.shape
    k = ids.shape[1]
    L = w13.shape[0] if L is None else L
    I = 2 * w2.shape[2]
    out = np.zeros((M, H), np.uint16)
    inter = None
    if want_intermediates:
        inter = dict(h13=np.zeros((M * k, 2 * I), np.uint16), q=np.zeros((M * k, I), np.uint8),
                     s=np.zeros((M * k, I // 128), np.float32), y=np.zeros((M * k, H), np.uint16))
    lib().oracle_fused_moe_mxfp4(_p(h), M, H, _p(ids), _p(w), k, _p(w13), _p(w13_s), _p(w2), _p(w2_s), expert_offset,
                                 L, I, scale_fmt, clamp, _p(out), _p(inter["h13"]) if inter else None,
                                 _p(inter["q"]) if inter else None, _p(inter["s"]) if inter else None,
                                 _p(inter["y"]) if inter else None)
    return (out, inter) if want_intermediates else out


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on (timing runs)."""
    lib().oracle_set_threads(n)
