"""ctypes binding of libbfp8moe.so (the C ABI in include/bfp8moe.h).

Argument marshalling only: torch tensors are turned into raw device pointers,
the current HIP stream is passed through, and a non-zero status raises.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback of any kind.  The library must have been built first
(``python -m block_fp8_mixture_route_amd.build``); importing this module
without it raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# BFP8MOE_LIB names another build of the same library (the host-sanitized one
# of tests/run_sanitized.py); by default the in-tree build
LIB_PATH = os.environ.get("BFP8MOE_LIB") or os.path.join(PKG, "libbfp8moe.so")

SCALE_FP32 = 0
SCALE_UE8M0 = 1

FLAG_ROUTE_SINGLE_WG = 1 << 0
FLAG_ROUTE_MULTI_WG = 1 << 1
FLAG_LAYER_GENERAL = 1 << 2
FLAG_LAYER_DECODE = 1 << 3
FLAG_LAYER_TOKEN = 1 << 4
FLAG_ROUTER_IN_ROUTE_PREP = 1 << 5


def FLAG_ONLY_STAGE(s):
    """Launch only stage s of the fused layer (tests and profiling)."""
    return (s + 1) << 8

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip"}


class Opts(ctypes.Structure):
    _fields_ = [
        ("block_m", ctypes.c_int32),
        ("scale_fmt", ctypes.c_int32),
        ("clamp_limit", ctypes.c_float),
        ("expert_offset", ctypes.c_int32),
        ("local_num_experts", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
        ("weight_scale_mode", ctypes.c_int32),
        ("act_static_scale", ctypes.c_float),
        ("inter_static_scale", ctypes.c_float),
        ("expert_map", ctypes.c_void_p),
    ]


WEIGHT_SCALE_BLOCK = 0
WEIGHT_SCALE_CHANNEL = 1
WEIGHT_MXFP4 = 2


class BFP8MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_i32, _i64, _u32, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "bfp8moe_opts_init": (None, [ctypes.POINTER(Opts)]),
    "bfp8moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bfp8moe_last_error": (ctypes.c_char_p, []),
    "bfp8moe_wait_faults": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]),
    "bfp8moe_stream_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p]),
    "bfp8moe_max_blocks": (_i64, [_i64, _i32, _i32]),
    "moe_route_prepare_workspace_size": (_sz, [_i64, _i32, _u32]),
    "moe_route_prepare": (ctypes.c_int, [_P, _i64, _i32, _i32, _i32, _P, _P, _P, _P, _i64, _P, _P, _sz, _u32, _P]),
    "moe_route_prepare_map": (ctypes.c_int, [_P, _i64, _P, _i32, _i32, _i32, _P, _P, _P, _P, _i64, _P, _P, _sz, _u32,
                                             _P]),
    "quant_fp8": (ctypes.c_int, [_P, _i64, _i32, _i32, _P, _P, _P]),
    "silu_and_mul": (ctypes.c_int, [_P, _i64, _i32, _f32, _P, _P]),
    "silu_and_mul_quant_fp8": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _f32, _i32, _P, _P, _P]),
    "moe_fp8_grouped_gemm": (ctypes.c_int, [_P, _P, _i32, _P, _P, _i32, _i32, _i32, _P, _P, _P, _P, _P, _i64, _i32,
                                            _i64, _P, _P]),
    "quant_fp8_rows": (ctypes.c_int, [_P, _i64, _i32, _i32, _f32, _P, _P, _P]),
    "silu_and_mul_quant_fp8_rows": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _f32, _i32, _f32, _P, _P, _P]),
    "moe_fp8_grouped_gemm_channel": (ctypes.c_int, [_P, _P, _i32, _P, _P, _i32, _i32, _i32, _P, _P, _P, _P, _P,
                                                    _i64, _i32, _i64, _P, _P]),
    "moe_mxfp4_grouped_gemm": (ctypes.c_int, [_P, _P, _i32, _P, _P, _i32, _i32, _i32, _P, _P, _P, _P, _P, _i64, _i32,
                                              _i64, _P, _P]),
    "moe_reduce": (ctypes.c_int, [_P, _P, _P, _i32, _i32, _i64, _i32, _i32, _P, _P]),
    "moe_reduce_map": (ctypes.c_int, [_P, _P, _P, _P, _i32, _i32, _i64, _i32, _i32, _P, _P]),
    "moe_router_topk": (ctypes.c_int, [_P, _i64, _i32, _i32, _i32, _P, _i32, ctypes.c_double, _P, _P, _P]),
    "moe_router_noaux_tc": (ctypes.c_int, [_P, _i64, _i32, _i32, _i32, _i32, _P, _i32, ctypes.c_double, _P, _P,
                                           _P]),
    "fused_moe_block_fp8_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(Opts)]),
    "fused_moe_block_fp8_stages": (_i32, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(Opts),
                                          ctypes.POINTER(ctypes.c_char_p), _i32]),
    "fused_moe_block_fp8": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _P, _P, _P, _P, _i32, _i32,
                                           ctypes.POINTER(Opts), _P, _P, _sz, _P]),
    "fused_moe_mxfp4": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _P, _P, _P, _P, _i32, _i32,
                                       ctypes.POINTER(Opts), _P, _P, _sz, _P]),
    "fused_moe_block_fp8_noalloc": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _P, _P, _P, _P, _i32, _i32,
                                                   ctypes.POINTER(Opts), _P, _P]),
    "fused_moe_block_fp8_routed": (ctypes.c_int, [_P, _i64, _i32, _P, _P, _i32, _i32, ctypes.c_double, _i32, _i32,
                                                  _i32, _P, _P,
                                                  _P, _P, _P, _P, _i32, _i32, ctypes.POINTER(Opts), _P, _P, _sz, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_fp8_mixture_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int):
    if status != 0:
        raise BFP8MoEError(status, lib().bfp8moe_last_error().decode())


def ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def stream_of(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_device(*ts):
    for t in ts:
        if t is not None and t.device.type != "cuda":
            raise ValueError("library entry points take device tensors")


def _u16(t):
    return t.view(torch.uint16) if t.dtype == torch.bfloat16 else t


def _u8(t):
    return t.view(torch.uint8) if t is not None and t.dtype == torch.float8_e4m3fn else t


def _expect(t, name, dtypes, shape=None):
    """Raise ValueError unless t has one of `dtypes` and, where given, the shape
    (None entries match any size).  The library reads raw memory: a wrong
    dtype or shape would silently be misread or read out of bounds."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and a != s for a, s in zip(t.shape, shape)):
            raise ValueError(f"{name} must have shape {tuple('*' if s is None else s for s in shape)}, "
                             f"got {tuple(t.shape)}")


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def stream_probe(buf: torch.Tensor, pattern: int, sink: torch.Tensor, row_bytes=0, piece=128, lds_bytes=0):
    """One read of the uint8 device buffer `buf` in the probe's shape (pattern
    0 contiguous, 1 GEMM-shaped tiles of rows of row_bytes); measurement only.
    sink: int32 device tensor of at least one word per workgroup."""
    _expect(buf, "buf", torch.uint8, (None,))
    _expect(sink, "sink", torch.int32, (None,))
    _require_device(buf, sink)
    check(lib().bfp8moe_stream_probe(ptr(buf), buf.numel(), pattern, row_bytes, piece, lds_bytes, ptr(sink),
                                     sink.numel(), stream_of(buf.device)))


def wait_faults(clear=True) -> int:
    """Fault bits of the kernels' bounded waits on the current device since the
    last clear (0: none).  Synchronises with the device; for tests and
    debugging."""
    f = ctypes.c_uint32(0)
    check(lib().bfp8moe_wait_faults(ctypes.byref(f), int(bool(clear))))
    return f.value


def opts(block_m=0, scale_fmt=SCALE_FP32, clamp_limit=math.inf, expert_offset=0, local_num_experts=0, flags=0,
         weight_scale_mode=WEIGHT_SCALE_BLOCK, act_static_scale=0.0, inter_static_scale=0.0, expert_map=None):
    """Layer options.  expert_map: device int32 [E] (global expert -> local
    expert, outside [0, local_num_experts) = held elsewhere), kept alive by
    the returned object."""
    o = Opts()
    lib().bfp8moe_opts_init(ctypes.byref(o))
    o.block_m, o.scale_fmt, o.clamp_limit = block_m, scale_fmt, clamp_limit
    o.expert_offset, o.local_num_experts, o.flags = expert_offset, local_num_experts, flags
    o.weight_scale_mode, o.act_static_scale, o.inter_static_scale = weight_scale_mode, act_static_scale, \
        inter_static_scale
    if expert_map is not None:
        _expect(expert_map, "expert_map", torch.int32, (None,))
        _require_device(expert_map)
        o.expert_map = ptr(expert_map).value
        o._expert_map = expert_map  # the pointer's owner
    return o


# ------------------------------------------------------------------ entry points

def max_blocks(R: int, L: int, block_m: int) -> int:
    return lib().bfp8moe_max_blocks(R, L, block_m)


def moe_route_prepare(topk_ids: torch.Tensor, expert_offset: int, L: int, block_m: int, with_blocks=True, flags=0,
                      expert_map=None):
    """Route preparation over the slice [expert_offset, expert_offset + L),
    or, with expert_map (device int32 [E]; expert_offset must be 0), over the
    experts the map sends into [0, L)."""
    _expect(topk_ids, "topk_ids", torch.int32)
    _expect(expert_map, "expert_map", torch.int32, (None,))
    _require_device(topk_ids, expert_map)
    if expert_map is not None and expert_offset != 0:
        raise ValueError("expert_map and expert_offset are exclusive")
    ids = topk_ids.reshape(-1)
    R = ids.numel()
    dev = ids.device
    mb = max_blocks(R, L, block_m)
    out = dict(
        sorted_routes=torch.empty(max(R, 1), dtype=torch.int32, device=dev)[:R],
        expert_offsets=torch.empty(L + 1, dtype=torch.int32, device=dev),
        block_expert=torch.empty(max(mb, 1), dtype=torch.int32, device=dev) if with_blocks else None,
        block_start=torch.empty(max(mb, 1), dtype=torch.int32, device=dev) if with_blocks else None,
        num_blocks=torch.empty(1, dtype=torch.int32, device=dev),
        max_blocks=mb,
    )
    wsb = lib().moe_route_prepare_workspace_size(R, L, flags)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    outs = (ptr(out["sorted_routes"]), ptr(out["expert_offsets"]), ptr(out["block_expert"]), ptr(out["block_start"]),
            mb, ptr(out["num_blocks"]), ptr(ws), wsb, flags, stream_of(dev))
    if expert_map is None:
        check(lib().moe_route_prepare(ptr(ids), R, expert_offset, L, block_m, *outs))
    else:
        check(lib().moe_route_prepare_map(ptr(ids), R, ptr(expert_map), expert_map.numel(), L, block_m, *outs))
    out["_ws"] = ws  # keep alive until the stream has consumed it
    return out


def quant_fp8(x: torch.Tensor, scale_fmt=SCALE_FP32, q=None, scales=None):
    _expect(x, "x", torch.bfloat16, (None, None))
    rows, K = x.shape
    _expect(q, "q", _FP8, (rows, K))
    _expect(scales, "scales", torch.float32, (rows, K // 128))
    _require_device(x, q, scales)
    q = torch.empty(rows, K, dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty(rows, K // 128, dtype=torch.float32, device=x.device) if scales is None else scales
    check(lib().quant_fp8(ptr(_u16(x)), rows, K, scale_fmt, ptr(q), ptr(scales), stream_of(x.device)))
    return q, scales


def silu_and_mul(gate_up: torch.Tensor, clamp_limit=math.inf, out=None):
    _expect(gate_up, "gate_up", torch.bfloat16, (None, None))
    rows, I2 = gate_up.shape
    _expect(out, "out", torch.bfloat16, (rows, I2 // 2))
    _require_device(gate_up, out)
    out = torch.empty(rows, I2 // 2, dtype=torch.bfloat16, device=gate_up.device) if out is None else out
    check(lib().silu_and_mul(ptr(_u16(gate_up)), rows, I2 // 2, clamp_limit, ptr(_u16(out)),
                             stream_of(gate_up.device)))
    return out


def silu_and_mul_quant_fp8(gate_up: torch.Tensor, row_expert_ids=None, expert_map=None, E=0,
                           clamp_limit=math.inf, scale_fmt=SCALE_FP32, q=None, scales=None):
    _expect(gate_up, "gate_up", torch.bfloat16, (None, None))
    rows, I2 = gate_up.shape
    I = I2 // 2
    _expect(row_expert_ids, "row_expert_ids", torch.int32, (rows,))
    _expect(expert_map, "expert_map", torch.int32, (E,))
    _expect(q, "q", _FP8, (rows, I))
    _expect(scales, "scales", torch.float32, (rows, I // 128))
    _require_device(gate_up, row_expert_ids, expert_map, q, scales)
    q = torch.empty(rows, I, dtype=torch.uint8, device=gate_up.device) if q is None else q
    scales = torch.empty(rows, I // 128, dtype=torch.float32, device=gate_up.device) if scales is None else scales
    check(lib().silu_and_mul_quant_fp8(ptr(_u16(gate_up)), rows, I, ptr(row_expert_ids), ptr(expert_map), E,
                                       clamp_limit, scale_fmt, ptr(q), ptr(scales), stream_of(gate_up.device)))
    return q, scales


def moe_fp8_grouped_gemm(A, A_scale, a_row_div, B, B_scale, route, block_m, R, C=None):
    """route: the dict returned by moe_route_prepare (with blocks)."""
    _expect(B, "B", _FP8, (None, None, None))
    L, N, K = B.shape
    _expect(A, "A", _FP8, (None, K))
    _expect(A_scale, "A_scale", torch.float32, (A.shape[0], K // 128))
    _expect(B_scale, "B_scale", torch.float32, (L, N // 128, K // 128))
    if R > A.shape[0] * a_row_div:
        raise ValueError(f"R={R} routes need {-(-R // a_row_div)} rows of A, it has {A.shape[0]}")
    _expect(C, "C", torch.bfloat16, (R, N))
    _require_device(A, A_scale, B, B_scale, C)
    A, B = _u8(A), _u8(B)
    C = torch.empty(R, N, dtype=torch.bfloat16, device=A.device) if C is None else C
    check(lib().moe_fp8_grouped_gemm(ptr(A), ptr(A_scale), a_row_div, ptr(B), ptr(B_scale), L, N, K,
                                     ptr(route["sorted_routes"]), ptr(route["expert_offsets"]),
                                     ptr(route["block_expert"]), ptr(route["block_start"]),
                                     ptr(route["num_blocks"]), route["max_blocks"], block_m, R, ptr(_u16(C)),
                                     stream_of(A.device)))
    return C


def moe_mxfp4_grouped_gemm(A, A_scale, a_row_div, B, B_scale, route, block_m, R, C=None):
    """MXFP4 weights: B [L, N, K/2] packed E2M1 (uint8), B_scale [L, N, K/32]
    E8M0 bytes (uint8); A, A_scale, route as moe_fp8_grouped_gemm."""
    _expect(B, "B", torch.uint8, (None, None, None))
    L, N, K2 = B.shape
    K = 2 * K2
    _expect(A, "A", _FP8, (None, K))
    _expect(A_scale, "A_scale", torch.float32, (A.shape[0], K // 128))
    _expect(B_scale, "B_scale", torch.uint8, (L, N, K // 32))
    if R > A.shape[0] * a_row_div:
        raise ValueError(f"R={R} routes need {-(-R // a_row_div)} rows of A, it has {A.shape[0]}")
    _expect(C, "C", torch.bfloat16, (R, N))
    _require_device(A, A_scale, B, B_scale, C)
    A = _u8(A)
    C = torch.empty(R, N, dtype=torch.bfloat16, device=A.device) if C is None else C
    check(lib().moe_mxfp4_grouped_gemm(ptr(A), ptr(A_scale), a_row_div, ptr(B), ptr(B_scale), L, N, K,
                                       ptr(route["sorted_routes"]), ptr(route["expert_offsets"]),
                                       ptr(route["block_expert"]), ptr(route["block_start"]),
                                       ptr(route["num_blocks"]), route["max_blocks"], block_m, R, ptr(_u16(C)),
                                       stream_of(A.device)))
    return C


def quant_fp8_rows(x, scale_fmt=SCALE_FP32, static_scale=0.0, q=None, scales=None):
    """One scale per row (static when > 0, else the row's amax / 448)."""
    _expect(x, "x", torch.bfloat16, (None, None))
    rows, K = x.shape
    _expect(q, "q", _FP8, (rows, K))
    _expect(scales, "scales", torch.float32, (rows,))
    _require_device(x, q, scales)
    q = torch.empty(rows, K, dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty(rows, dtype=torch.float32, device=x.device) if scales is None else scales
    check(lib().quant_fp8_rows(ptr(_u16(x)), rows, K, scale_fmt, static_scale, ptr(q), ptr(scales),
                               stream_of(x.device)))
    return q, scales


def silu_and_mul_quant_fp8_rows(gate_up, row_expert_ids=None, expert_map=None, E=0, clamp_limit=math.inf,
                                scale_fmt=SCALE_FP32, static_scale=0.0, q=None, scales=None):
    _expect(gate_up, "gate_up", torch.bfloat16, (None, None))
    rows, I2 = gate_up.shape
    I = I2 // 2
    _expect(row_expert_ids, "row_expert_ids", torch.int32, (rows,))
    _expect(expert_map, "expert_map", torch.int32, (E,))
    _expect(q, "q", _FP8, (rows, I))
    _expect(scales, "scales", torch.float32, (rows,))
    _require_device(gate_up, row_expert_ids, expert_map, q, scales)
    q = torch.empty(rows, I, dtype=torch.uint8, device=gate_up.device) if q is None else q
    scales = torch.empty(rows, dtype=torch.float32, device=gate_up.device) if scales is None else scales
    check(lib().silu_and_mul_quant_fp8_rows(ptr(_u16(gate_up)), rows, I, ptr(row_expert_ids), ptr(expert_map), E,
                                            clamp_limit, scale_fmt, static_scale, ptr(q), ptr(scales),
                                            stream_of(gate_up.device)))
    return q, scales


def moe_fp8_grouped_gemm_channel(A, A_scale, a_row_div, B, B_scale, route, block_m, R, C=None):
    """Grouped GEMM with per-row activation scales A_scale [rows] and
    per-channel weight scales B_scale [L, N]; route as moe_fp8_grouped_gemm."""
    _expect(B, "B", _FP8, (None, None, None))
    L, N, K = B.shape
    _expect(A, "A", _FP8, (None, K))
    _expect(A_scale, "A_scale", torch.float32, (A.shape[0],))
    _expect(B_scale, "B_scale", torch.float32, (L, N))
    if R > A.shape[0] * a_row_div:
        raise ValueError(f"R={R} routes need {-(-R // a_row_div)} rows of A, it has {A.shape[0]}")
    _expect(C, "C", torch.bfloat16, (R, N))
    _require_device(A, A_scale, B, B_scale, C)
    A, B = _u8(A), _u8(B)
    C = torch.empty(R, N, dtype=torch.bfloat16, device=A.device) if C is None else C
    check(lib().moe_fp8_grouped_gemm_channel(ptr(A), ptr(A_scale), a_row_div, ptr(B), ptr(B_scale), L, N, K,
                                             ptr(route["sorted_routes"]), ptr(route["expert_offsets"]),
                                             ptr(route["block_expert"]), ptr(route["block_start"]),
                                             ptr(route["num_blocks"]), route["max_blocks"], block_m, R, ptr(_u16(C)),
                                             stream_of(A.device)))
    return C


def moe_reduce(y, topk_w, topk_ids=None, expert_offset=0, L=0, out=None, expert_map=None):
    """Weighted top-k reduction; live routes: all (topk_ids None), the slice
    [expert_offset, expert_offset + L), or with expert_map (device int32 [E])
    the ids the map sends into [0, L)."""
    _expect(topk_w, "topk_w", torch.float32, (None, None))
    M, k = topk_w.shape
    _expect(y, "y", torch.bfloat16, (M * k, None))
    H = y.shape[1]
    _expect(topk_ids, "topk_ids", torch.int32, (M, k))
    _expect(out, "out", torch.bfloat16, (M, H))
    _expect(expert_map, "expert_map", torch.int32, (None,))
    _require_device(y, topk_w, topk_ids, out, expert_map)
    out = torch.empty(M, H, dtype=torch.bfloat16, device=y.device) if out is None else out
    if expert_map is None:
        check(lib().moe_reduce(ptr(_u16(y)), ptr(topk_w), ptr(topk_ids), expert_offset, L, M, k, H, ptr(_u16(out)),
                               stream_of(y.device)))
    else:
        check(lib().moe_reduce_map(ptr(_u16(y)), ptr(topk_w), ptr(topk_ids), ptr(expert_map), expert_map.numel(), L,
                                   M, k, H, ptr(_u16(out)), stream_of(y.device)))
    return out


SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


def _check_router_buffers(E, k, M, bias, topk_ids, topk_w):
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != E):
        raise ValueError("the selection bias must be float32 with one value per expert")
    if topk_ids is not None and (topk_ids.dtype != torch.int32 or tuple(topk_ids.shape) != (M, k)):
        raise ValueError("topk_ids must be int32 of shape [M, k]")
    if topk_w is not None and (topk_w.dtype != torch.float32 or tuple(topk_w.shape) != (M, k)):
        raise ValueError("topk_w must be float32 of shape [M, k]")


def router_topk(logits, k, score_fn=SCORE_SOFTMAX, bias=None, renormalize=True, scale=1.0, topk_ids=None,
                topk_w=None):
    """[M, E] fp32 router logits -> ([M, k] int32 expert ids, largest first,
    [M, k] fp32 weights)."""
    _require_device(logits, bias, topk_ids, topk_w)
    if logits.dtype != torch.float32:
        raise ValueError("router logits must be float32")
    M, E = logits.shape
    _check_router_buffers(E, k, M, bias, topk_ids, topk_w)
    ids = torch.empty(M, k, dtype=torch.int32, device=logits.device) if topk_ids is None else topk_ids
    w = torch.empty(M, k, dtype=torch.float32, device=logits.device) if topk_w is None else topk_w
    check(lib().moe_router_topk(ptr(logits), M, E, k, score_fn, ptr(bias), int(bool(renormalize)), float(scale),
                                ptr(ids), ptr(w), stream_of(logits.device)))
    return ids, w


def router_noaux_tc(logits, k, n_group, topk_group, bias=None, renormalize=True, scale=1.0, topk_ids=None,
                    topk_w=None):
    """Group-limited noaux-TC routing of [M, E] fp32 logits -> ([M, k] int32
    ids, largest key first, [M, k] fp32 weights)."""
    _expect(logits, "logits", torch.float32, (None, None))
    M, E = logits.shape
    _check_router_buffers(E, k, M, bias, topk_ids, topk_w)
    _require_device(logits, bias, topk_ids, topk_w)
    ids = torch.empty(M, k, dtype=torch.int32, device=logits.device) if topk_ids is None else topk_ids
    w = torch.empty(M, k, dtype=torch.float32, device=logits.device) if topk_w is None else topk_w
    check(lib().moe_router_noaux_tc(ptr(logits), M, E, k, n_group, topk_group, ptr(bias), int(bool(renormalize)),
                                    float(scale), ptr(ids), ptr(w), stream_of(logits.device)))
    return ids, w


def fused_moe_workspace_size(M, H, k, E, I, o: Opts) -> int:
    return lib().fused_moe_block_fp8_workspace_size(M, H, k, E, I, ctypes.byref(o))


def fused_moe_stages(M, H, k, E, I, o: Opts):
    """Names of the kernel stages a fused_moe_block_fp8 call with these sizes
    and options launches, in order."""
    names = (ctypes.c_char_p * 16)()
    n = lib().fused_moe_block_fp8_stages(M, H, k, E, I, ctypes.byref(o), names, 16)
    if n < 0:
        raise BFP8MoEError(1, lib().bfp8moe_last_error().decode())
    return [names[i].decode() for i in range(n)]


def _check_layer_buffers(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E, o, out, ws, need=None):
    """dtypes and shapes of the layer's buffers, so that no pointer handed to
    the library is misread or read past its end: hidden [M, H] bf16, routing
    [M, k] int32 / fp32, w13 [L', 2I, H] and w2 [L', H, I] E4M3 bytes with
    L' >= the local expert count, their fp32 block scales, out [M, H] bf16."""
    _expect(hidden, "hidden", torch.bfloat16, (None, None))
    M, H = hidden.shape
    _expect(topk_ids, "topk_ids", torch.int32, (M, None))
    k = topk_ids.shape[1]
    _expect(topk_w, "topk_w", torch.float32, (M, k))
    _expect(w2, "w2", _FP8, (None, H, None))
    Lw, _, I = w2.shape
    _expect(w13, "w13", _FP8, (Lw, 2 * I, H))
    if o.weight_scale_mode == WEIGHT_SCALE_CHANNEL:
        _expect(w13_scale, "w13_scale", torch.float32, (Lw, 2 * I))
        _expect(w2_scale, "w2_scale", torch.float32, (Lw, H))
    else:
        _expect(w13_scale, "w13_scale", torch.float32, (Lw, 2 * I // 128, H // 128))
        _expect(w2_scale, "w2_scale", torch.float32, (Lw, H // 128, I // 128))
    L = o.local_num_experts if o.local_num_experts > 0 else E
    if o.expert_map and getattr(o, "_expert_map", None) is not None and o._expert_map.numel() != E:
        raise ValueError(f"the expert map has {o._expert_map.numel()} entries, E is {E}")
    if Lw < L:
        raise ValueError(f"the weights hold {Lw} experts, the call addresses {L}")
    _expect(out, "out", torch.bfloat16, (M, H))
    if ws is not None:
        _expect(ws, "ws", torch.uint8, (None,))
        if need is not None and ws.numel() < need:
            raise ValueError(f"workspace of {ws.numel()} bytes, {need} needed")
    return M, H, k, I


def fused_moe_block_fp8(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E=None, o: Opts = None,
                        out=None, ws=None):
    E = w13.shape[0] if E is None else E
    o = opts() if o is None else o
    M, H, k, I = _check_layer_buffers(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E, o, out, ws)
    _require_device(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out, ws)
    w13, w2 = _u8(w13), _u8(w2)
    need = fused_moe_workspace_size(M, H, k, E, I, o)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    out = torch.empty(M, H, dtype=torch.bfloat16, device=hidden.device) if out is None else out
    check(lib().fused_moe_block_fp8(ptr(_u16(hidden)), M, H, ptr(topk_ids), ptr(topk_w), k, ptr(w13),
                                    ptr(w13_scale), ptr(w2), ptr(w2_scale), E, I, ctypes.byref(o),
                                    ptr(_u16(out)), ptr(ws), ws.numel(), stream_of(hidden.device)))
    return out


def fused_moe_mxfp4(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E=None, o: Opts = None, out=None,
                    ws=None):
    """The layer with MXFP4 weights: w13 [L, 2I, H/2] and w2 [L, H, I/2]
    packed E2M1 (uint8), w13_scale [L, 2I, H/32] and w2_scale [L, H, I/32]
    E8M0 bytes (uint8).  o: opts(weight_scale_mode=WEIGHT_MXFP4, ...) (the
    default when None)."""
    E = w13.shape[0] if E is None else E
    o = opts(weight_scale_mode=WEIGHT_MXFP4) if o is None else o
    if o.weight_scale_mode != WEIGHT_MXFP4:
        raise ValueError("fused_moe_mxfp4 takes options with weight_scale_mode=WEIGHT_MXFP4")
    _expect(hidden, "hidden", torch.bfloat16, (None, None))
    M, H = hidden.shape
    _expect(topk_ids, "topk_ids", torch.int32, (M, None))
    k = topk_ids.shape[1]
    _expect(topk_w, "topk_w", torch.float32, (M, k))
    _expect(w2, "w2", torch.uint8, (None, H, None))
    Lw, _, I2 = w2.shape
    I = 2 * I2
    _expect(w13, "w13", torch.uint8, (Lw, 2 * I, H // 2))
    _expect(w13_scale, "w13_scale", torch.uint8, (Lw, 2 * I, H // 32))
    _expect(w2_scale, "w2_scale", torch.uint8, (Lw, H, I // 32))
    L = o.local_num_experts if o.local_num_experts > 0 else E
    if Lw < L:
        raise ValueError(f"the weights hold {Lw} experts, the call addresses {L}")
    if o.expert_map and getattr(o, "_expert_map", None) is not None and o._expert_map.numel() != E:
        raise ValueError(f"the expert map has {o._expert_map.numel()} entries, E is {E}")
    _expect(out, "out", torch.bfloat16, (M, H))
    _expect(ws, "ws", torch.uint8, (None,))
    _require_device(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out, ws)
    need = fused_moe_workspace_size(M, H, k, E, I, o)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    out = torch.empty(M, H, dtype=torch.bfloat16, device=hidden.device) if out is None else out
    check(lib().fused_moe_mxfp4(ptr(_u16(hidden)), M, H, ptr(topk_ids), ptr(topk_w), k, ptr(w13), ptr(w13_scale),
                                ptr(w2), ptr(w2_scale), E, I, ctypes.byref(o), ptr(_u16(out)), ptr(ws), ws.numel(),
                                stream_of(hidden.device)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def fused_moe_block_fp8_noalloc(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E=None, o: Opts = None,
                                out=None):
    """fused_moe_block_fp8 on the library's own per-device scratch array (the
    C entry point allocates nothing; pass `out` to allocate nothing here
    either).  Calls that overlap on one GPU race."""
    E = w13.shape[0] if E is None else E
    o = opts() if o is None else o
    M, H, k, I = _check_layer_buffers(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, E, o, out, None)
    _require_device(hidden, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out)
    w13, w2 = _u8(w13), _u8(w2)
    out = torch.empty(M, H, dtype=torch.bfloat16, device=hidden.device) if out is None else out
    check(lib().fused_moe_block_fp8_noalloc(ptr(_u16(hidden)), M, H, ptr(topk_ids), ptr(topk_w), k, ptr(w13),
                                            ptr(w13_scale), ptr(w2), ptr(w2_scale), E, I, ctypes.byref(o),
                                            ptr(_u16(out)), stream_of(hidden.device)))
    return out


def fused_moe_block_fp8_routed(hidden, router_logits, k, w13, w13_scale, w2, w2_scale, score_fn=SCORE_SOFTMAX,
                               bias=None, renormalize=True, scale=1.0, o: Opts = None, out=None, ws=None,
                               topk_ids=None, topk_w=None, n_group=1, topk_group=1):
    """Router and layer in one call: returns (out [M, H] BF16, topk_ids [M, k]
    int32, topk_w [M, k] fp32)."""
    _expect(hidden, "hidden", torch.bfloat16, (None, None))
    M, H = hidden.shape
    if router_logits.dtype != torch.float32 or router_logits.dim() != 2 or router_logits.shape[0] != M:
        raise ValueError("router logits must be float32 of shape [M, E]")
    E = router_logits.shape[1]
    _check_router_buffers(E, k, M, bias, topk_ids, topk_w)
    o = opts() if o is None else o
    _check_layer_buffers(hidden, torch.empty(M, k, dtype=torch.int32, device="meta"),
                         torch.empty(M, k, dtype=torch.float32, device="meta"), w13, w13_scale, w2, w2_scale, E, o,
                         out, ws)
    _require_device(hidden, router_logits, bias, w13, w13_scale, w2, w2_scale, topk_ids, topk_w, out, ws)
    w13, w2 = _u8(w13), _u8(w2)
    I = w2.shape[2]
    need = fused_moe_workspace_size(M, H, k, E, I, o)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    out = torch.empty(M, H, dtype=torch.bfloat16, device=hidden.device) if out is None else out
    ids = torch.empty(M, k, dtype=torch.int32, device=hidden.device) if topk_ids is None else topk_ids
    w = torch.empty(M, k, dtype=torch.float32, device=hidden.device) if topk_w is None else topk_w
    check(lib().fused_moe_block_fp8_routed(ptr(_u16(hidden)), M, H, ptr(router_logits), ptr(bias), score_fn,
                                           int(bool(renormalize)), float(scale), n_group, topk_group, k, ptr(ids), ptr(w), ptr(w13),
                                           ptr(w13_scale), ptr(w2), ptr(w2_scale), E, I, ctypes.byref(o),
                                           ptr(_u16(out)), ptr(ws), ws.numel(), stream_of(hidden.device)))
    return out, ids, w
