"""Benchmark of the block-FP8 fused MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config decode_m1] [--instances N]
    python bench.py --suite out.json   # every config + act/quant + route prep + copy

A step is one fused_moe_block_fp8 call (route preparation, gate/up GEMM,
SwiGLU + quantisation, down GEMM, moe_reduce) on one batch.  The workload is
the M=1, E=256, top-k=8 decode layer (H=7168, I=256) by default.  Inputs are
seeded synthetic tensors already resident in HBM.  Steps rotate over
independent layer instances (own weights, routing and hidden states) whose
combined weight bytes exceed the 256 MB Infinity Cache several times, so the
weights stream from HBM as in a real multi-layer decode.  The K steps are
replayed from a HIP graph that holds one rotation, and timed with HIP events
between a device synchronisation on both sides.

Printed: one JSON line with the metric (achieved HBM GB/s of the whole layer
from its compulsory bytes), microseconds per layer, the roofline of the
dominant kernel (its algorithmic bytes over its average duration, that
kernel launched alone back to back from a HIP graph, timed with HIP events on
its stream), the kernel's HBM traffic from the hardware-counter
summary in profiles/ while the kernel's sources match it, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused block-FP8 MoE layer µs + achieved HBM GB/s at M=1, E=256, top-k=8"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ HIP runtime via ctypes

class Hip:
    """The few HIP runtime calls the benchmark needs: a stream, graph capture
    and replay, and events."""

    def __init__(self):
        # bind to the HIP runtime already mapped into the process (torch's),
        # never a second copy
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        self.h = ctypes.CDLL(path or "libamdhip64.so.7")
        P, PP = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "hipStreamCreateWithFlags": [PP, ctypes.c_uint],
            "hipStreamSynchronize": [P],
            "hipStreamDestroy": [P],
            "hipStreamBeginCapture": [P, ctypes.c_int],
            "hipStreamEndCapture": [P, PP],
            "hipGraphInstantiate": [PP, P, P, P, ctypes.c_size_t],
            "hipGraphLaunch": [P, P],
            "hipGraphExecDestroy": [P],
            "hipGraphDestroy": [P],
            "hipEventCreate": [PP],
            "hipEventDestroy": [P],
            "hipEventRecord": [P, P],
            "hipEventSynchronize": [P],
            "hipEventElapsedTime": [ctypes.POINTER(ctypes.c_float), P, P],
            "hipDeviceSynchronize": [],
            "hipGetErrorString": [ctypes.c_int],
        }
        for n, a in sig.items():
            f = getattr(self.h, n)
            f.argtypes = a
            f.restype = ctypes.c_char_p if n == "hipGetErrorString" else ctypes.c_int

    def ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {self.h.hipGetErrorString(rc).decode()}")

    def stream(self):
        s = ctypes.c_void_p()
        self.ok(self.h.hipStreamCreateWithFlags(ctypes.byref(s), 1), "hipStreamCreateWithFlags")
        return s

    def event(self):
        e = ctypes.c_void_p()
        self.ok(self.h.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e

    def capture(self, stream, body):
        self.ok(self.h.hipStreamBeginCapture(stream, 0), "hipStreamBeginCapture")  # global mode
        try:
            body()
        finally:
            g = ctypes.c_void_p()
            rc = self.h.hipStreamEndCapture(stream, ctypes.byref(g))
        self.ok(rc, "hipStreamEndCapture")
        ex = ctypes.c_void_p()
        self.ok(self.h.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0), "hipGraphInstantiate")
        return g, ex

    def launch(self, ex, stream):
        self.ok(self.h.hipGraphLaunch(ex, stream), "hipGraphLaunch")

    def sync(self, stream=None):
        if stream is None:
            self.ok(self.h.hipDeviceSynchronize(), "hipDeviceSynchronize")
        else:
            self.ok(self.h.hipStreamSynchronize(stream), "hipStreamSynchronize")

    def record(self, ev, stream):
        self.ok(self.h.hipEventRecord(ev, stream), "hipEventRecord")

    def elapsed_ms(self, a, b):
        self.ok(self.h.hipEventSynchronize(b), "hipEventSynchronize")
        ms = ctypes.c_float()
        self.ok(self.h.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)


# ------------------------------------------------------------------ bytes

def layer_bytes(case, ids):
    """Compulsory HBM bytes of one layer: every distinct active expert's W13 and
    W2 with their block scales, hidden states in, output out, routing in."""
    import torch
    d = int(torch.unique(ids[ids >= 0]).numel())
    H, I = case.H, case.I
    per_expert = 2 * I * H + H * I + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))
    io = case.M * H * 2 * 2 + case.M * case.k * 8
    return d * per_expert + io, d


def stage_bytes(case, ids, stage):
    """Algorithmic bytes of the dominant stage.
    token_gate_up_swiglu / decode_gate_up_swiglu / gate_up_gemm: W13 + its
    scales of every active expert, the hidden states (BF16 in, or E4M3 codes +
    scales for the general GEMM), routing in, the stage's output rows out."""
    import torch
    d = int(torch.unique(ids[ids >= 0]).numel())
    H, I, R = case.H, case.I, case.M * case.k
    w = d * (2 * I * H + 4 * (2 * I // 128) * (H // 128))
    if stage in ("token_gate_up_swiglu", "decode_gate_up_swiglu"):
        return w + case.M * H * 2 + R * 4 + R * I * 2
    return w + case.M * H + case.M * (H // 128) * 4 + R * 4 + R * 2 * I * 2


# ------------------------------------------------------------------ one layer config

FP8_PEAK_TFLOPS = 5000.0  # dense FP8 MFMA


def layer_flops(case):
    """Multiply-add flops of the two projections over all routes."""
    return 2 * case.M * case.k * (2 * case.I * case.H + case.H * case.I)


def time_graph(hip, stream, body, reps):
    """Capture body() into a HIP graph, replay it once untimed, then time
    `reps` replays with HIP events on `stream`; milliseconds per replay."""
    _, g = hip.capture(stream, body)
    hip.launch(g, stream)
    hip.sync(stream)
    ev0, ev1 = hip.event(), hip.event()
    hip.sync()
    hip.record(ev0, stream)
    for _ in range(reps):
        hip.launch(g, stream)
    hip.record(ev1, stream)
    hip.sync()
    return hip.elapsed_ms(ev0, ev1) / reps


PATH_FLAGS = {"auto": 0, "token": 1 << 4, "decode": 1 << 3, "general": 1 << 2}


def measure_layer(case, steps, warmup, instances, hip, stream, dev, per_stage=True, flags=0, block_m=0):
    """Graph-timed fused_moe_block_fp8 on `case`, rotating over independent
    instances; optionally each stage alone.  Returns a dict of figures and the
    instances (for the CPU leg)."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    # one instance first, to size the rotation
    t0 = time.time()
    first = synth.layer_inputs(case, 0, device=dev)
    b0, d0 = layer_bytes(case, first[1])
    n_inst = instances or max(1, min(64, math.ceil(4 * MALL_BYTES / b0)))
    insts = [first] + [synth.layer_inputs(case, i, device=dev) for i in range(1, n_inst)]
    torch.cuda.synchronize()
    log(f"{case.name}: {n_inst} instances generated in {time.time() - t0:.1f}s, "
        f"{b0 / 1e6:.2f} MB compulsory per layer (instance 0, {d0} active experts)")

    o = bfp8.opts(scale_fmt=case.scale_fmt, clamp_limit=case.clamp, flags=flags, block_m=block_m)
    stages = bfp8.fused_moe_stages(case.M, case.H, case.k, case.E, case.I, o)
    ws_bytes = bfp8.fused_moe_workspace_size(case.M, case.H, case.k, case.E, case.I, o)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    outs = [torch.empty(case.M, case.H, dtype=torch.bfloat16, device=dev) for _ in range(n_inst)]
    bytes_per = [layer_bytes(case, x[1])[0] for x in insts]
    torch.cuda.synchronize()
    L = bfp8.lib()
    P = ctypes.c_void_p

    def call(i, opts_obj):
        hidden, ids, w, W = insts[i]
        bfp8._lib.check(L.fused_moe_block_fp8(P(hidden.data_ptr()), case.M, case.H, P(ids.data_ptr()),
                                              P(w.data_ptr()), case.k, P(W.w13.data_ptr()), P(W.w13_s.data_ptr()),
                                              P(W.w2.data_ptr()), P(W.w2_s.data_ptr()), case.E, case.I,
                                              ctypes.byref(opts_obj), P(outs[i].data_ptr()), P(ws.data_ptr()),
                                              ws_bytes, stream))

    # warm-up: W eager steps
    for s_ in range(warmup):
        call(s_ % n_inst, o)
    hip.sync(stream)
    log(f"warm-up {warmup} steps done; stages: {stages}")

    # graph of one rotation (+ a partial rotation so that exactly K steps run)
    full, rem = divmod(steps, n_inst)
    _, g_rot = hip.capture(stream, lambda: [call(i, o) for i in range(n_inst)])
    g_rem = hip.capture(stream, lambda: [call(i, o) for i in range(rem)])[1] if rem else None
    hip.launch(g_rot, stream)  # one untimed replay to settle the graph
    hip.sync(stream)
    ev0, ev1 = hip.event(), hip.event()
    hip.sync()
    hip.record(ev0, stream)
    for _ in range(full):
        hip.launch(g_rot, stream)
    if g_rem is not None:
        hip.launch(g_rem, stream)
    hip.record(ev1, stream)
    hip.sync()
    total_ms = hip.elapsed_ms(ev0, ev1)
    steps = full * n_inst + rem
    ms_per_step = total_ms / steps
    total_bytes = full * sum(bytes_per) + sum(bytes_per[:rem])
    gbs = total_bytes / (total_ms * 1e-3) / 1e9
    log(f"timed {steps} steps: {ms_per_step * 1e3:.2f} us/layer, {gbs:.0f} GB/s")

    # per-stage durations: each stage alone (BFP8MOE_FLAG_ONLY_STAGE), at
    # least 32 calls (whole rotations) captured in a graph and replayed, HIP
    # events on the stream the kernels run on around the replays:
    # launch-to-launch time of the stage's kernel, back to back as in the
    # layer graph (a graph of one short kernel would time the host's graph
    # launches instead).  A stage past the first reads what the whole calls
    # above left in the workspace (same code path and traffic; the values are
    # not checked here).
    stage_us = {}
    if per_stage:
        per_graph = n_inst * max(1, math.ceil(32 / n_inst))
        reps = max(1, math.ceil(steps / per_graph))
        for s_, name in enumerate(stages):
            os_ = bfp8.opts(scale_fmt=case.scale_fmt, clamp_limit=case.clamp, flags=flags | bfp8.FLAG_ONLY_STAGE(s_),
                            block_m=block_m)
            stage_us[name] = time_graph(hip, stream, lambda: [call(i % n_inst, os_) for i in range(per_graph)],
                                        reps) * 1e3 / per_graph
        log("stage us (each stage alone, graph-timed): " + ", ".join(f"{k}={v:.2f}" for k, v in stage_us.items()))
    mean_bytes = sum(bytes_per) / n_inst
    roof_us = max(mean_bytes / (HBM_PEAK_GBS * 1e3), layer_flops(case) / (FP8_PEAK_TFLOPS * 1e6))
    return {"us_per_layer": ms_per_step * 1e3, "ms_per_step": ms_per_step, "gbs": gbs, "steps": steps,
            "n_inst": n_inst, "bytes_per_layer": mean_bytes, "flops_per_layer": layer_flops(case),
            "roofline_us": roof_us, "roofline_frac": roof_us / (ms_per_step * 1e3), "stages": stages,
            "stage_us": stage_us, "insts": insts, "active_experts_inst0": d0}


# ------------------------------------------------------------------ launch floor

def launch_floor(hip, stream, dev):
    """Launch-to-launch time of a kernel that does (almost) nothing, replayed
    back to back from a HIP graph: the fixed cost every kernel of a layer pays
    on top of its own work.  Uses torch's fill kernel on one element, 64
    launches per graph."""
    import torch

    ext = torch.cuda.ExternalStream(stream.value, device=dev)
    x = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def body():
        with torch.cuda.stream(ext):
            for i in range(64):
                x.fill_(i)

    us = time_graph(hip, stream, body, 20) * 1e3 / 64
    print(f"graph launch floor: {us:.2f} µs per kernel (one-element fill, 64 launches per graph)", flush=True)
    return us


def router_table(hip, stream, dev):
    """Top-k routers, graph-timed: single-group softmax (renormalised) and
    biased sigmoid (renormalised), and group-limited noaux-TC (biased sigmoid,
    8 groups keeping 4), each one launch, beside torch's softmax -> topk ->
    renormalise for context."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    L_ = bfp8.lib()
    P = ctypes.c_void_p
    ext = torch.cuda.ExternalStream(stream.value, device=dev)
    print()
    print("| tokens M | experts E | k | softmax µs | sigmoid + bias µs | noaux-TC 8 groups keep 4 µs "
          "| torch softmax/topk/renorm µs |")
    print("|---|---|---|---|---|---|---|")
    out = {}
    for (M, E) in [(1, 256), (16, 256), (256, 256), (2048, 512), (4096, 256), (16384, 256)]:
        lg = synth.router_logits(M, E, "bench_router", device=dev)
        bias = synth.router_bias(E, "bench_router", device=dev)
        rid = torch.empty(M, 8, dtype=torch.int32, device=dev)
        rw = torch.empty(M, 8, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def rt(score_fn, b):
            bfp8._lib.check(L_.moe_router_topk(P(lg.data_ptr()), M, E, 8, score_fn,
                                               None if b is None else P(b.data_ptr()), 1, 1.0, P(rid.data_ptr()),
                                               P(rw.data_ptr()), stream))

        def torch_router():
            with torch.cuda.stream(ext):
                for _ in range(20):
                    v, _i = torch.topk(torch.softmax(lg, -1), 8, -1)
                    v / v.sum(-1, keepdim=True)

        ts = time_graph(hip, stream, lambda: [rt(bfp8.SCORE_SOFTMAX, None) for _ in range(20)], 20) * 1e3 / 20
        tg = time_graph(hip, stream, lambda: [rt(bfp8.SCORE_SIGMOID, bias) for _ in range(20)], 20) * 1e3 / 20

        def rt_grouped():
            bfp8._lib.check(L_.moe_router_noaux_tc(P(lg.data_ptr()), M, E, 8, 8, 4, P(bias.data_ptr()), 1, 1.0,
                                                   P(rid.data_ptr()), P(rw.data_ptr()), stream))

        tn = time_graph(hip, stream, lambda: [rt_grouped() for _ in range(20)], 20) * 1e3 / 20
        tt = time_graph(hip, stream, torch_router, 20) * 1e3 / 20
        out[f"{M}x{E}"] = {"softmax_us": ts, "sigmoid_bias_us": tg, "noaux_tc_8x4_us": tn, "torch_us": tt}
        print(f"| {M} | {E} | 8 | {ts:.2f} | {tg:.2f} | {tn:.2f} | {tt:.2f} |", flush=True)

    return out


def routed_table(hip, stream, dev):
    """The decode layers with their router, graph-timed over 8 instances
    (more weight bytes than the Infinity Cache holds): the router's launch
    followed by the layer, against the routed layer (the router folded into
    the few-token gate/up kernel up to 4 tokens, its own launch from 8), the
    routed layer with the router inside route preparation's workgroup on the
    general path (16 to 64 tokens, BFP8MOE_FLAG_ROUTER_IN_ROUTE_PREP), and
    the layer alone on given routing."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    L_ = bfp8.lib()
    P = ctypes.c_void_p
    print()
    print("| config | router + layer µs (2 calls) | routed layer µs | routed, router in route prep µs | "
          "layer alone µs |")
    print("|---|---|---|---|---|")
    out = {}
    for M in (1, 2, 4, 8, 16, 32, 64):
        name = f"decode_m{M}"
        c = dataclasses.replace(synth.LAYER_CASES["decode_m1"], name=name, M=M)
        o = bfp8.opts()
        need = bfp8.fused_moe_workspace_size(c.M, c.H, c.k, c.E, c.I, o)
        insts = []
        for i in range(8):
            lg = synth.router_logits(c.M, c.E, "bench_routed", name, i, device=dev)
            ids, w = bfp8.router_topk(lg, c.k)
            mw = synth.moe_weights(c.E, c.H, c.I, "bench_routed", name, i,
                                   experts=ids.unique().cpu().tolist(), device=dev)
            hid = synth.hidden_states(c.M, c.H, "bench_routed", name, i, device=dev)
            insts.append(dict(lg=lg, ids=ids, w=w, mw=mw, hid=hid,
                              out=torch.empty(c.M, c.H, dtype=torch.bfloat16, device=dev),
                              ws=torch.empty(max(need, 1), dtype=torch.uint8, device=dev)))
        torch.cuda.synchronize()

        def layer(x):
            m = x["mw"]
            bfp8._lib.check(L_.fused_moe_block_fp8(P(x["hid"].data_ptr()), c.M, c.H, P(x["ids"].data_ptr()),
                                                   P(x["w"].data_ptr()), c.k, P(m.w13.data_ptr()),
                                                   P(m.w13_s.data_ptr()), P(m.w2.data_ptr()), P(m.w2_s.data_ptr()),
                                                   c.E, c.I, ctypes.byref(o), P(x["out"].data_ptr()),
                                                   P(x["ws"].data_ptr()), x["ws"].numel(), stream))

        def router(x):
            bfp8._lib.check(L_.moe_router_topk(P(x["lg"].data_ptr()), c.M, c.E, c.k, bfp8.SCORE_SOFTMAX, None, 1,
                                               1.0, P(x["ids"].data_ptr()), P(x["w"].data_ptr()), stream))

        o_rp = bfp8.opts(flags=bfp8.FLAG_ROUTER_IN_ROUTE_PREP)

        def routed(x, ro=o):
            m = x["mw"]
            bfp8._lib.check(L_.fused_moe_block_fp8_routed(
                P(x["hid"].data_ptr()), c.M, c.H, P(x["lg"].data_ptr()), None, bfp8.SCORE_SOFTMAX, 1, 1.0, 1, 1, c.k,
                P(x["ids"].data_ptr()), P(x["w"].data_ptr()), P(m.w13.data_ptr()), P(m.w13_s.data_ptr()),
                P(m.w2.data_ptr()), P(m.w2_s.data_ptr()), c.E, c.I, ctypes.byref(ro), P(x["out"].data_ptr()),
                P(x["ws"].data_ptr()), x["ws"].numel(), stream))

        reps = 40
        t2 = time_graph(hip, stream, lambda: [(router(x), layer(x)) for x in insts * 4], reps) * 1e3 / 32
        tf = time_graph(hip, stream, lambda: [routed(x) for x in insts * 4], reps) * 1e3 / 32
        trp = (time_graph(hip, stream, lambda: [routed(x, o_rp) for x in insts * 4], reps) * 1e3 / 32
               if M >= 16 else None)
        tl = time_graph(hip, stream, lambda: [layer(x) for x in insts * 4], reps) * 1e3 / 32
        out[name] = {"router_plus_layer_us": t2, "routed_us": tf, "routed_in_route_prep_us": trp, "layer_us": tl}
        rps = "—" if trp is None else f"{trp:.2f}"
        print(f"| {name} | {t2:.2f} | {tf:.2f} | {rps} | {tl:.2f} |", flush=True)
        del insts
        torch.cuda.empty_cache()
    out["shared"] = shared_table(hip, stream, dev)
    return out


def shared_table(hip, stream, dev):
    """The decode layer with a shared expert of width 2048 split into 8
    pseudo-experts of width 256 (experts 256..263, weight 1 for every token):
    one call with 16 routes per token, against the routed layer (8 routes)
    and the shared expert (8 routes) as two calls (their sum left out, which
    favours the two calls).  8 instances rotated."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    L_ = bfp8.lib()
    P = ctypes.c_void_p
    print()
    print("| tokens M | one call, 16 routes µs | routed + shared, 2 calls µs | routed layer alone µs |")
    print("|---|---|---|---|")
    out = {}
    H, I, E = 7168, 256, 264
    o = bfp8.opts()
    for M in (1, 2, 4):
        insts = []
        for i in range(8):
            rid, rw = synth.uniform_routing(M, 256, 8, "bench_shared", M, i, device=dev)
            sid = torch.arange(256, 264, dtype=torch.int32, device=dev).expand(M, 8)
            ids16 = torch.cat([rid, sid], dim=1).contiguous()
            w16 = torch.cat([rw, torch.ones(M, 8, device=dev)], dim=1).contiguous()
            experts = torch.unique(ids16).cpu().tolist()
            mw = synth.moe_weights(E, H, I, "bench_shared", M, i, experts=experts, device=dev)
            hid = synth.hidden_states(M, H, "bench_shared", M, i, device=dev)
            x = dict(ids16=ids16, w16=w16, ids8=rid.contiguous(), w8=rw.contiguous(),
                     sid=(sid - 256).contiguous(), sw=torch.ones(M, 8, device=dev), mw=mw, hid=hid,
                     out=torch.empty(M, H, dtype=torch.bfloat16, device=dev))
            need = max(bfp8.fused_moe_workspace_size(M, H, k, E, I, o) for k in (8, 16))
            x["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            insts.append(x)
        torch.cuda.synchronize()

        def call(x, ids, w, k, e0, ne):
            m = x["mw"]
            w13 = m.w13[e0:e0 + ne]
            bfp8._lib.check(L_.fused_moe_block_fp8(
                P(x["hid"].data_ptr()), M, H, P(ids.data_ptr()), P(w.data_ptr()), k, P(w13.data_ptr()),
                P(m.w13_s[e0:e0 + ne].data_ptr()), P(m.w2[e0:e0 + ne].data_ptr()), P(m.w2_s[e0:e0 + ne].data_ptr()),
                ne, I, ctypes.byref(o), P(x["out"].data_ptr()), P(x["ws"].data_ptr()), x["ws"].numel(), stream))

        one = lambda: [call(x, x["ids16"], x["w16"], 16, 0, E) for x in insts * 4]
        two = lambda: [(call(x, x["ids8"], x["w8"], 8, 0, 256), call(x, x["sid"], x["sw"], 8, 256, 8))
                       for x in insts * 4]
        routed = lambda: [call(x, x["ids8"], x["w8"], 8, 0, 256) for x in insts * 4]
        t1 = time_graph(hip, stream, one, 40) * 1e3 / 32
        t2 = time_graph(hip, stream, two, 40) * 1e3 / 32
        t0 = time_graph(hip, stream, routed, 40) * 1e3 / 32
        out[M] = {"one_call_us": t1, "two_calls_us": t2, "routed_us": t0}
        print(f"| {M} | {t1:.2f} | {t2:.2f} | {t0:.2f} |", flush=True)
        del insts
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ suite

SUITE_STEPS = {"tiny": 200, "decode_m1": 480, "decode_m4": 200, "decode_m16": 100, "decode_m32": 100,
               "small_m128": 20, "small_m512": 20, "large_m2048": 10}


def variants_table(hip, stream, dev, block_m=0, configs=("small_m128", "small_m512", "large_m2048"), formats=None):
    """The layer with each weight format on the general-path configs, one
    instance each (its weights exceed the Infinity Cache several times over),
    graph-timed over 8 calls: block FP8, the W8A8 variant (random E4M3 codes,
    per-channel scales, dynamic per-token activation scales) and MXFP4 weights
    (random E2M1 codes, E8M0 scales per 32).  Compulsory bytes: the active
    experts' weights and scales in each format, hidden states in, output out,
    routing in."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    print()
    print("| config | format | µs / layer | compulsory MB | GB/s | HBM roofline µs | fraction |")
    print("|---|---|---|---|---|---|---|")
    res = {}
    for name in configs:
        case = synth.LAYER_CASES[name]
        M, E, k, H, I = case.M, case.E, case.k, case.H, case.I
        hidden, ids, w, W = synth.layer_inputs(case, 0, device=dev)
        d = int(torch.unique(ids[ids >= 0]).numel())
        io = M * H * 2 * 2 + M * k * 8
        g = torch.Generator(device=dev).manual_seed(synth.seed_of("variants", name))

        def e4m3(shape):
            # random E4M3 codes but the NaN ones, drawn one expert at a time
            # (no single random tensor grows with E)
            t = torch.empty(shape, dtype=torch.uint8, device=dev)
            for e in range(shape[0]):
                mag = torch.randint(0, 0x7F, shape[1:], generator=g, device=dev, dtype=torch.uint8)
                t[e].copy_(mag | (torch.randint(0, 2, shape[1:], generator=g, device=dev, dtype=torch.uint8) << 7))
            return t

        c13, c2 = e4m3((E, 2 * I, H)), e4m3((E, H, I))
        s13 = torch.rand(E, 2 * I, generator=g, device=dev) * 1e-3 + 1e-4
        s2 = torch.rand(E, H, generator=g, device=dev) * 1e-3 + 1e-4
        MX = synth.mxfp4_weights(E, H, I, "variants", name, device=dev)
        out = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
        forms = {
            "block FP8": (lambda: bfp8.fused_moe_block_fp8(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, E=E, out=out,
                                                          ws=ws["block FP8"], o=opts["block FP8"]),
                          bfp8.opts(block_m=block_m),
                          d * (3 * I * H + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)))),
            "W8A8": (lambda: bfp8.fused_moe_block_fp8(hidden, ids, w, c13, s13, c2, s2, E=E, out=out, ws=ws["W8A8"],
                                                     o=opts["W8A8"]),
                     bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL, block_m=block_m),
                     d * (3 * I * H + 4 * (2 * I + H))),
            "MXFP4": (lambda: bfp8.fused_moe_mxfp4(hidden, ids, w, MX.w13, MX.w13_s, MX.w2, MX.w2_s, E=E, out=out,
                                                  ws=ws["MXFP4"], o=opts["MXFP4"]),
                      bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4, block_m=block_m),
                      d * (3 * I * H // 2 + 3 * I * H // 32)),
        }
        opts = {f: v[1] for f, v in forms.items()}
        ws = {f: torch.empty(max(bfp8.fused_moe_workspace_size(M, H, k, E, I, v[1]), 1), dtype=torch.uint8,
                             device=dev) for f, v in forms.items()}
        res[name] = {}
        ext = torch.cuda.ExternalStream(stream.value, device=dev)
        for f, (fn, _, wbytes) in forms.items():
            if formats is not None and f not in formats:
                continue
            with torch.cuda.stream(ext):  # the binding launches on torch's current stream: the timed one
                fn()
                hip.sync(stream)
                us = time_graph(hip, stream, lambda: [fn() for _ in range(8)], 5) * 1e3 / 8
            nbytes = wbytes + io
            roof = nbytes / 8e12 * 1e6
            res[name][f] = {"us": us, "bytes": nbytes, "roofline_us": roof}
            print(f"| {name} | {f} | {us:.2f} | {nbytes / 1e6:.1f} | {nbytes / (us * 1e3):.0f} | {roof:.2f} | "
                  f"{roof / us:.3f} |", flush=True)
        del c13, c2, MX, W
        torch.cuda.empty_cache()
    return res


def variants_decode_table(hip, stream, dev, token_counts=(1, 4), both_paths=False, formats=None):
    """The decode layer (E=256, top-k 8, H=7168, I=256) at a few token counts
    with each weight format: block FP8, W8A8 (random E4M3 codes, per-channel
    scales, dynamic per-token activation scales) and MXFP4 (random E2M1
    codes, E8M0 scales per 32).  One set of 256 experts per format; instance
    i routes to experts disjoint from its neighbours' (8 M consecutive ones),
    and the rotation of instances reads every expert once, more bytes than the
    Infinity Cache holds.  Graph-timed; compulsory bytes as variants_table.
    both_paths: the few-token and general paths forced in turn, else the
    library's choice.  formats: the weight formats to run (default all)."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    E, k, H, I = 256, 8, 7168, 256
    g = torch.Generator(device=dev).manual_seed(synth.seed_of("variants_decode"))

    def e4m3(shape):
        t = torch.empty(shape, dtype=torch.uint8, device=dev)
        for e in range(shape[0]):
            mag = torch.randint(0, 0x7F, shape[1:], generator=g, device=dev, dtype=torch.uint8)
            t[e].copy_(mag | (torch.randint(0, 2, shape[1:], generator=g, device=dev, dtype=torch.uint8) << 7))
        return t

    W = synth.moe_weights(E, H, I, "variants_decode", device=dev)
    C = synth.MoEWeights(e4m3((E, 2 * I, H)), torch.rand(E, 2 * I, generator=g, device=dev) * 1e-3 + 1e-4,
                         e4m3((E, H, I)), torch.rand(E, H, generator=g, device=dev) * 1e-3 + 1e-4)
    MX = synth.mxfp4_weights(E, H, I, "variants_decode", device=dev)
    print()
    print("| tokens | format | path | µs / layer | compulsory MB | GB/s | HBM roofline µs | fraction | "
          "stages µs (each alone) |")
    print("|---|---|---|---|---|---|---|---|---|")
    res = {}
    ext = torch.cuda.ExternalStream(stream.value, device=dev)
    for M in token_counts:
        n_inst = E // (M * k)
        insts = []
        for i in range(n_inst):
            ids = (torch.arange(M * k, dtype=torch.int32, device=dev) + i * M * k).reshape(M, k) % E
            w = torch.rand(M, k, generator=g, device=dev) + 0.1
            insts.append((synth.hidden_states(M, H, "variants_decode", M, i, device=dev), ids.contiguous(),
                          (w / w.sum(dim=1, keepdim=True)).contiguous(),
                          torch.empty(M, H, dtype=torch.bfloat16, device=dev)))
        d = M * k
        io = M * H * 2 * 2 + M * k * 8
        forms = {
            "block FP8": (bfp8.opts(), d * (3 * I * H + 4 * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128))),
                          lambda x, o, ws: bfp8.fused_moe_block_fp8(x[0], x[1], x[2], W.w13, W.w13_s, W.w2, W.w2_s,
                                                                    E=E, out=x[3], ws=ws, o=o)),
            "W8A8": (bfp8.opts(weight_scale_mode=bfp8.WEIGHT_SCALE_CHANNEL), d * (3 * I * H + 4 * (2 * I + H)),
                     lambda x, o, ws: bfp8.fused_moe_block_fp8(x[0], x[1], x[2], C.w13, C.w13_s, C.w2, C.w2_s, E=E,
                                                               out=x[3], ws=ws, o=o)),
            "MXFP4": (bfp8.opts(weight_scale_mode=bfp8.WEIGHT_MXFP4), d * (3 * I * H // 2 + 3 * I * H // 32),
                      lambda x, o, ws: bfp8.fused_moe_mxfp4(x[0], x[1], x[2], MX.w13, MX.w13_s, MX.w2, MX.w2_s, E=E,
                                                            out=x[3], ws=ws, o=o)),
        }
        res[M] = {}
        runs = []
        for f, (o, wbytes, fn) in forms.items():
            if formats is not None and f not in formats:
                continue
            flag_list = [PATH_FLAGS["token"], PATH_FLAGS["general"]] if both_paths else [0]
            for fl in flag_list:
                runs.append((f, bfp8.opts(weight_scale_mode=o.weight_scale_mode, flags=fl), wbytes, fn))
        for f, o, wbytes, fn in runs:
            ws = torch.empty(max(bfp8.fused_moe_workspace_size(M, H, k, E, I, o), 1), dtype=torch.uint8, device=dev)
            path = bfp8.fused_moe_stages(M, H, k, E, I, o)[0]
            with torch.cuda.stream(ext):  # the bindings launch on torch's current stream: the timed one
                for x in insts:
                    fn(x, o, ws)
                hip.sync(stream)
                us = time_graph(hip, stream, lambda: [fn(x, o, ws) for x in insts], 20) * 1e3 / n_inst
                # each stage alone (BFP8MOE_FLAG_ONLY_STAGE), after the whole calls above
                stages = bfp8.fused_moe_stages(M, H, k, E, I, o)
                st_us = {}
                for si, sn in enumerate(stages):
                    os_ = bfp8.opts(weight_scale_mode=o.weight_scale_mode, flags=o.flags | bfp8.FLAG_ONLY_STAGE(si))
                    st_us[sn] = time_graph(hip, stream, lambda: [fn(x, os_, ws) for x in insts], 20) * 1e3 / n_inst
            nbytes = wbytes + io
            roof = nbytes / 8e12 * 1e6
            res[M][f + ("" if not both_paths else f" ({path})")] = {
                "us": us, "bytes": nbytes, "roofline_us": roof, "first_stage": path, "stage_us": st_us}
            stx = ", ".join(f"{a} {b:.2f}" for a, b in st_us.items())
            print(f"| {M} | {f} | {path} | {us:.2f} | {nbytes / 1e6:.1f} | {nbytes / (us * 1e3):.0f} | {roof:.2f} | "
                  f"{roof / us:.3f} | {stx} |", flush=True)
            del ws
    return res


def phase_table(hip, stream, dev, steps):
    """Where the decode layer's time goes.  The M=1, E=256, top-k 8, I=256
    layer at hidden widths 1024..7168: each of its two kernels alone and the
    whole layer, graph-timed over instances whose weights exceed the Infinity
    Cache (measure_layer).  A least-squares line per kernel, time = fixed +
    bytes / rate over the widths, gives its fixed cost (launch, the first
    loads' latency, the tail after the last weight byte) and the rate at which
    it streams; the H=7168 layer is then split into those parts and the time
    between the kernels (the layer minus the two kernels alone)."""
    import numpy as np

    from block_fp8_mixture_route_amd import synth

    base = synth.LAYER_CASES["decode_m1"]
    rows = []
    print()
    print("| H | gate/up MB | gate/up µs | down MB | down µs | layer µs |")
    print("|---|---|---|---|---|---|")
    for H in (1024, 2048, 3584, 5120, 7168):
        case = dataclasses.replace(base, name=f"decode_m1_h{H}", H=H)
        r = measure_layer(case, steps, 8, 0, hip, stream, dev)
        ids = r["insts"][0][1]
        d = int(torch_unique_count(ids))
        b_up = d * (2 * case.I * H + 4 * (2 * case.I // 128) * (H // 128)) + H * 2 + case.k * 8 + case.k * case.I * 2
        b_dn = d * (H * case.I + 4 * (H // 128) * (case.I // 128)) + case.k * case.I * 2 + case.k * 8 + H * 2
        st = r["stage_us"]
        rows.append((H, b_up, st["token_gate_up_swiglu"], b_dn, st["token_down_reduce"], r["us_per_layer"]))
        print(f"| {H} | {b_up / 1e6:.2f} | {rows[-1][2]:.2f} | {b_dn / 1e6:.2f} | {rows[-1][4]:.2f} | "
              f"{rows[-1][5]:.2f} |", flush=True)
        del r
    a = np.array(rows, dtype=np.float64)
    fit = {}
    for name, bcol, tcol in (("gate/up", 1, 2), ("down", 3, 4)):
        slope, icpt = np.polyfit(a[:, bcol], a[:, tcol], 1)  # µs per byte, µs
        fit[name] = (icpt, 1.0 / slope / 1e3)                  # fixed µs, GB/s
    H, b_up, t_up, b_dn, t_dn, t_layer = rows[-1]
    between = t_layer - t_up - t_dn
    print()
    print("| kernel | fixed µs (intercept) | streaming GB/s (slope) |")
    print("|---|---|---|")
    for name, (f0, gbs) in fit.items():
        print(f"| {name} | {f0:.2f} | {gbs:.0f} |")
    print()
    print(f"H = {H} layer, {t_layer:.2f} µs:")
    print()
    print("| part | µs |")
    print("|---|---|")
    parts = [("gate/up: fixed cost", fit["gate/up"][0]),
             (f"gate/up: {b_up / 1e6:.1f} MB at {fit['gate/up'][1]:.0f} GB/s", b_up / (fit["gate/up"][1] * 1e3)),
             ("gate/up: fitted minus measured", t_up - fit["gate/up"][0] - b_up / (fit["gate/up"][1] * 1e3)),
             ("down: fixed cost", fit["down"][0]),
             (f"down: {b_dn / 1e6:.1f} MB at {fit['down'][1]:.0f} GB/s", b_dn / (fit["down"][1] * 1e3)),
             ("down: fitted minus measured", t_dn - fit["down"][0] - b_dn / (fit["down"][1] * 1e3)),
             ("between the kernels (layer minus both alone)", between)]
    for name, v in parts:
        print(f"| {name} | {v:.2f} |")
    print(f"| total | {sum(v for _, v in parts):.2f} |")
    print()
    print(f"All {(b_up + b_dn) / 1e6:.1f} MB at 8 TB/s: {(b_up + b_dn) / 8e6:.2f} µs; at the gate/up kernel's own "
          f"streaming rate: {(b_up + b_dn) / (fit['gate/up'][1] * 1e3):.2f} µs.", flush=True)


def torch_unique_count(ids):
    import torch
    return torch.unique(ids[ids >= 0]).numel()


def act_quant_tables(hip, stream, dev, res=None):
    """The fused activation + quantisation on the pages' act+quant workload
    (rows = tokens x 8, I = 512, clamp 7, UE8M0, ~10 % masked) and under
    8-way expert parallelism (top-k 6, width 2048, 32 of 256 experts local),
    graph-timed over 20 calls, against SwiGLU then quant_fp8 as two launches."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    res = {} if res is None else res
    res.setdefault("act_quant", {})
    L_ = bfp8.lib()
    P = ctypes.c_void_p

    # activation + quant (warm, like the pages): fused kernel against SwiGLU
    # then quant_fp8 as two launches
    print()
    print("| tokens | rows | fused µs | two kernels µs | speedup | fused GB/s (unmasked rows) |")
    print("|---|---|---|---|---|---|")
    I = synth.ACT_I
    for tok in synth.ACT_TOKENS:
        rows = tok * 8
        gu, rid = synth.act_rows(rows, I, synth.ACT_E, "bench", tok, device=dev)
        q = torch.empty(rows, I, dtype=torch.uint8, device=dev)
        sc = torch.empty(rows, I // 128, dtype=torch.float32, device=dev)
        h = torch.empty(rows, I, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

        def fused():
            bfp8._lib.check(L_.silu_and_mul_quant_fp8(P(gu.data_ptr()), rows, I, P(rid.data_ptr()), None,
                                                      synth.ACT_E, synth.ACT_CLAMP, bfp8.SCALE_UE8M0,
                                                      P(q.data_ptr()), P(sc.data_ptr()), stream))

        def two():
            bfp8._lib.check(L_.silu_and_mul(P(gu.data_ptr()), rows, I, synth.ACT_CLAMP, P(h.data_ptr()), stream))
            bfp8._lib.check(L_.quant_fp8(P(h.data_ptr()), rows, I, bfp8.SCALE_UE8M0, P(q.data_ptr()),
                                         P(sc.data_ptr()), stream))

        tf = time_graph(hip, stream, lambda: [fused() for _ in range(20)], 20) * 1e3 / 20
        t2 = time_graph(hip, stream, lambda: [two() for _ in range(20)], 20) * 1e3 / 20
        live = int(((rid >= 0) & (rid < synth.ACT_E)).sum().item())
        nbytes = live * (4 * I + I + 4 * (I // 128))
        res["act_quant"][tok] = {"rows": rows, "fused_us": tf, "two_kernel_us": t2}
        print(f"| {tok} | {rows} | {tf:.2f} | {t2:.2f} | {t2 / tf:.2f} | {nbytes / (tf * 1e3):.0f} |", flush=True)

    # activation + quant under 8-way expert parallelism (top-k 6, width 2048,
    # 32 of 256 experts local): the fused kernel skips the non-local rows
    # through the expert map; the two-kernel arm has no row filter
    print()
    print("| tokens | rows | local rows | fused µs (expert-map filter) | two kernels µs (all rows) | "
          "fused GB/s (local rows) |")
    print("|---|---|---|---|---|---|")
    res["act_quant_ep8"] = {}
    I = synth.EP_I
    for tok in synth.EP_TOKENS:
        gu, rid, emap = (t.to(dev) for t in synth.ep_act_inputs(tok, "bench"))
        rows = gu.shape[0]
        q = torch.empty(rows, I, dtype=torch.uint8, device=dev)
        sc = torch.empty(rows, I // 128, dtype=torch.float32, device=dev)
        h = torch.empty(rows, I, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

        def fused():
            bfp8._lib.check(L_.silu_and_mul_quant_fp8(P(gu.data_ptr()), rows, I, P(rid.data_ptr()),
                                                      P(emap.data_ptr()), synth.EP_E, synth.ACT_CLAMP,
                                                      bfp8.SCALE_UE8M0, P(q.data_ptr()), P(sc.data_ptr()), stream))

        def two():
            bfp8._lib.check(L_.silu_and_mul(P(gu.data_ptr()), rows, I, synth.ACT_CLAMP, P(h.data_ptr()), stream))
            bfp8._lib.check(L_.quant_fp8(P(h.data_ptr()), rows, I, bfp8.SCALE_UE8M0, P(q.data_ptr()),
                                         P(sc.data_ptr()), stream))

        tf = time_graph(hip, stream, lambda: [fused() for _ in range(20)], 20) * 1e3 / 20
        t2 = time_graph(hip, stream, lambda: [two() for _ in range(20)], 20) * 1e3 / 20
        live = int((emap[rid.long()] >= 0).sum().item())
        nbytes = live * (4 * I + I + 4 * (I // 128))
        res["act_quant_ep8"][tok] = {"rows": rows, "local_rows": live, "fused_us": tf, "two_kernel_us": t2}
        print(f"| {tok} | {rows} | {live} | {tf:.2f} | {t2:.2f} | {nbytes / (tf * 1e3):.0f} |", flush=True)
    return res


def stream_probe_table(hip, stream, dev):
    """What this memory system gives a read shape: 4 GiB read once per launch
    by bfp8moe_stream_probe, contiguous slabs and the grouped GEMM's tile
    shape (128 rows per workgroup, 8 rows x 128 bytes per load instruction, or
    1,024 bytes of a row per load), its walk along K in order or rotated per
    workgroup, at the GEMMs' row lengths, with 2, 3 or 8 workgroups per
    compute unit (unused LDS); graph-timed over 5 reads."""
    import torch

    import block_fp8_mixture_route_amd as bfp8

    L_ = bfp8.lib()
    P = ctypes.c_void_p
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print("| shape | row bytes | bytes of a row per load | workgroups per CU | TB/s |")
    print("|---|---|---|---|---|")
    res = []
    for occ in (2, 3, 8):
        lds = 0 if occ >= 8 else 160 * 1024 // occ - 1024
        for pattern, K, piece in ([(0, 0, 128)] + [(pt, K, pc) for K in (4096, 1024, 7168) for pc in (128, 1024)
                                                    for pt in (1, 2)]):
            def body():
                bfp8._lib.check(L_.bfp8moe_stream_probe(P(buf.data_ptr()), nbytes, pattern, K, piece, lds,
                                                        P(sink.data_ptr()), sink.numel(), stream))

            used = nbytes if pattern == 0 else nbytes // (128 * K) * 128 * K
            ms = time_graph(hip, stream, body, 5)
            tbs = used / (ms * 1e-3) / 1e12
            shape = ["contiguous", "tile", "tile, K walk rotated per workgroup"][pattern]
            res.append({"shape": shape, "row_bytes": K, "piece": piece, "wg_per_cu": occ, "tbs": tbs})
            print(f"| {shape} | {K or '—'} | {piece if pattern else '—'} | {occ} | {tbs:.2f} |", flush=True)
    return res


def suite(hip, stream, dev):
    """Every layer config, the activation+quant workload (fused against two
    kernels), route preparation (one workgroup against many) and a plain copy
    as the practical bandwidth ceiling.  Prints markdown tables; returns the
    figures."""
    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    L_ = bfp8.lib()
    P = ctypes.c_void_p
    ext = torch.cuda.ExternalStream(stream.value, device=dev)
    res = {"layers": {}, "act_quant": {}, "route_prep": {}, "copy": {}}

    print("| config | M | E | k | H | I | path | µs / layer | GB/s | roofline µs | fraction | stages µs (each alone) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    runs = [(name, case, 0) for name, case in synth.LAYER_CASES.items()]
    # the other paths where they apply, forced (the default picks one by M)
    runs += [(f"{n} (forced)", synth.LAYER_CASES[n], f) for n, f in
             [("decode_m4", PATH_FLAGS["decode"]), ("decode_m4", PATH_FLAGS["general"]),
              ("decode_m16", PATH_FLAGS["token"]), ("decode_m32", PATH_FLAGS["token"])]]
    oracle_insts = {}
    for name, case, flags in runs:
        r = measure_layer(case, SUITE_STEPS.get(name.split()[0], 50), 4, 0, hip, stream, dev, flags=flags)
        insts = r.pop("insts")
        if not flags:
            oracle_insts[name] = (case, insts[0], r["us_per_layer"])
        del insts
        res["layers"][name + (f" flags {flags}" if flags else "")] = r
        st = ", ".join(f"{k} {v:.2f}" for k, v in r["stage_us"].items())
        path = "few tokens" if r["stages"][0].startswith("token") else (
            "small batch" if r["stages"][0].startswith("decode") else "general")
        print(f"| {name} | {case.M} | {case.E} | {case.k} | {case.H} | {case.I} | {path} | {r['us_per_layer']:.2f} | "
              f"{r['gbs']:.0f} | {r['roofline_us']:.2f} | {r['roofline_frac']:.3f} | {st} |", flush=True)
        torch.cuda.empty_cache()

    # the CPU oracle on instance 0 of every config: one thread and every host
    # core for the small ones (mean of at least 5 runs and 2 s), every core only for the
    # configs that take minutes on one (one run)
    from oracle import oracle as O

    cores = O.num_threads()
    print()
    print(f"CPU oracle (host threads available: {cores}), whole layer, instance 0:")
    print()
    print("| config | 1 thread s / layer | all threads s / layer (threads) | GPU µs / layer | GPU speedup over all threads |")
    print("|---|---|---|---|---|")
    res["oracle"] = {"cores": cores}
    for name, (case, inst, gpu_us) in oracle_insts.items():
        big = case.M >= 512
        t1 = None if big else oracle_layer_seconds(case, inst, 2.0, threads=1, min_runs=1)[0]
        tn, n, thr = oracle_layer_seconds(case, inst, 0.0 if big else 2.0, threads=cores, min_runs=1 if big else 5)
        res["oracle"][name] = {"one_thread_s": t1, "all_threads_s": tn, "threads": thr}
        t1s = "—" if t1 is None else f"{t1:.3f}"
        print(f"| {name} | {t1s} | {tn:.3f} ({thr}) | {gpu_us:.2f} | {tn * 1e6 / gpu_us:.0f} |", flush=True)
    oracle_insts.clear()
    torch.cuda.empty_cache()

    act_quant_tables(hip, stream, dev, res)

    # route preparation: single workgroup against count + scan/scatter
    print()
    print("| routes R | local experts L | block_m | one workgroup µs | many workgroups µs |")
    print("|---|---|---|---|---|")
    for (R, L, bm, routing) in [(8, 256, 16, "uniform"), (1024, 256, 16, "mixed"), (4096, 256, 32, "mixed"),
                                (16384, 512, 64, "zipf")]:
        M = R // 8
        c = synth.LayerCase("rp", M=M, E=L, k=8, H=128, I=128, routing=routing, zipf_s=1.0 if routing == "zipf" else 1.2)
        ids, _ = synth.routing_for(c, "bench_rp", device=dev)
        ids = ids.reshape(-1).contiguous()
        mb = bfp8.max_blocks(R, L, bm)
        outs = [torch.empty(max(n, 1), dtype=torch.int32, device=dev) for n in (R, L + 1, mb, mb, 1)]
        row = []
        for flags in (bfp8.FLAG_ROUTE_SINGLE_WG, bfp8.FLAG_ROUTE_MULTI_WG):
            wsb = L_.moe_route_prepare_workspace_size(R, L, flags)
            wsr = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()

            def rp(flags=flags, wsr=wsr, wsb=wsb):
                bfp8._lib.check(L_.moe_route_prepare(P(ids.data_ptr()), R, 0, L, bm, *[P(t.data_ptr()) for t in outs[:4]],
                                                     mb, P(outs[4].data_ptr()), P(wsr.data_ptr()), wsb, flags, stream))

            try:
                row.append(time_graph(hip, stream, lambda: [rp() for _ in range(20)], 20) * 1e3 / 20)
            except bfp8.BFP8MoEError:
                row.append(float("nan"))  # outside that variant's limits
        res["route_prep"][R] = {"L": L, "block_m": bm, "single_us": row[0], "multi_us": row[1]}
        print(f"| {R} | {L} | {bm} | {row[0]:.2f} | {row[1]:.2f} |", flush=True)

    res["variants"] = variants_table(hip, stream, dev)
    res["router"] = router_table(hip, stream, dev)
    res["routed"] = routed_table(hip, stream, dev)

    # a plain device copy of the decode layer's size, rotating over buffers
    # that together exceed the Infinity Cache: the practical HBM ceiling
    nbytes = 44 << 20
    nbuf = 12
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2 * nbuf)]
    for b_ in bufs:
        b_.fill_(1)
    torch.cuda.synchronize()

    def copies():
        with torch.cuda.stream(ext):
            for i in range(nbuf):
                bufs[2 * i + 1].copy_(bufs[2 * i])

    res["launch_floor_us"] = launch_floor(hip, stream, dev)
    tc = time_graph(hip, stream, copies, 10) / nbuf
    res["copy"] = {"bytes": nbytes, "us": tc * 1e3, "gbs_read_plus_write": 2 * nbytes / (tc * 1e-3) / 1e9}
    print()
    print(f"plain copy of {nbytes >> 20} MiB: {tc * 1e3:.2f} µs, {2 * nbytes / (tc * 1e-3) / 1e9:.0f} GB/s "
          f"(read + write)", flush=True)
    return res


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--config", default="decode_m1")
    ap.add_argument("--instances", type=int, default=0, help="layer instances to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run 4 plain device copies of this many MiB (a known-size reference for "
                         "hardware traffic counters)")
    ap.add_argument("--path", choices=sorted(PATH_FLAGS), default="auto",
                    help="force one implementation of the layer (default: the library's choice by shape)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="the config's layer at this many tokens instead (same shape and routing kind)")
    ap.add_argument("--block-m", type=int, default=0, help="routes per compact block of the general path (0 = auto)")
    ap.add_argument("--floor", action="store_true", help="only the graph launch floor of one kernel")
    ap.add_argument("--router", action="store_true", help="only the router timing table")
    ap.add_argument("--variants-decode", action="store_true",
                    help="only the decode layer (1 and 4 tokens) with block-FP8, W8A8 and MXFP4 weights")
    ap.add_argument("--variants-crossover", action="store_true",
                    help="only the decode layer at 4 to 16 tokens per weight format on the few-token and the "
                         "general path (where the automatic choice switches)")
    ap.add_argument("--variants-general", action="store_true",
                    help="each weight format on the general-path configs (with --block-m: that block size)")
    ap.add_argument("--variants-configs", default="small_m128,small_m512,large_m2048",
                    help="configs of --variants-general, comma-separated")
    ap.add_argument("--variants-formats", default="block FP8,W8A8,MXFP4",
                    help="weight formats of --variants-general and --variants-crossover, comma-separated")
    ap.add_argument("--crossover-tokens", default="4,8,12,16",
                    help="token counts of --variants-crossover, comma-separated (each at most 32)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only the read-bandwidth probe: contiguous and GEMM-tile read shapes over 4 GiB")
    ap.add_argument("--act-quant", action="store_true",
                    help="only the activation + quantisation tables (the pages' workload and expert parallelism)")
    ap.add_argument("--phases", action="store_true",
                    help="only the decode layer's phase table: each kernel alone and the layer at five hidden widths, "
                         "fixed cost and streaming rate per kernel fitted, the H=7168 layer split into them")
    ap.add_argument("--suite", metavar="JSON", default=None,
                    help="instead of the metric line: every layer config, activation+quant, route preparation "
                         "and a plain copy, as markdown tables on stdout and figures in JSON")
    args = ap.parse_args()

    if args.suite and os.environ.get("BFP8MOE_SUITE_ENABLE") != "1":
        print("bench.py --suite is disabled: its last run ended in a GPU memory fault whose cause has not been found "
              "(the single-table modes --config, --phases, --floor and --router are unaffected; "
              "BFP8MOE_SUITE_ENABLE=1 runs it anyway)", file=sys.stderr)
        sys.exit(3)
    if args.variants_general and args.block_m not in (32, 64):
        print("bench.py --variants-general takes --block-m 32 or 64: its run with the automatic block size "
              "(16 routes per block at small M=128) ended in a GPU memory fault whose cause has not been found",
              file=sys.stderr)
        sys.exit(3)
    if args.variants_crossover:
        toks = args.crossover_tokens.split(",")
        if not all(t.isdigit() and 1 <= int(t) <= 32 for t in toks):
            print(f"--crossover-tokens takes token counts from 1 to 32 (got {args.crossover_tokens})", file=sys.stderr)
            sys.exit(2)
    if args.tokens < 0:
        print(f"--tokens takes a positive token count (got {args.tokens})", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_fp8_mixture_route_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = hip.stream()

    if args.floor:
        launch_floor(hip, stream, dev)
        return
    if args.router:
        router_table(hip, stream, dev)
        routed_table(hip, stream, dev)
        return
    if args.variants_decode:
        variants_decode_table(hip, stream, dev)
        return
    if args.variants_crossover:
        variants_decode_table(hip, stream, dev, token_counts=tuple(int(t) for t in args.crossover_tokens.split(",")),
                              both_paths=True, formats=args.variants_formats.split(","))
        return
    if args.phases:
        phase_table(hip, stream, dev, args.steps)
        return
    if args.act_quant:
        act_quant_tables(hip, stream, dev)
        return
    if args.stream_probe:
        stream_probe_table(hip, stream, dev)
        return
    if args.variants_general:
        variants_table(hip, stream, dev, block_m=args.block_m, configs=args.variants_configs.split(","),
                       formats=args.variants_formats.split(","))
        return
    if args.suite:
        res = suite(hip, stream, dev)
        with open(args.suite, "w") as f:
            json.dump(res, f, indent=1, default=str)
        return

    case = synth.LAYER_CASES[args.config]
    if args.tokens:
        case = dataclasses.replace(case, name=f"{case.name}_tokens{args.tokens}", M=args.tokens)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 4 copies of {args.calibrate_copy_mib} MiB")

    r = measure_layer(case, args.steps, args.warmup, args.instances, hip, stream, dev, flags=PATH_FLAGS[args.path],
                      block_m=args.block_m)
    insts, stage_us, n_inst = r["insts"], r["stage_us"], r["n_inst"]
    dom = next(s_ for s_ in ("token_gate_up_swiglu", "decode_gate_up_swiglu", "gate_up_gemm") if s_ in stage_us)
    dom_bytes = sum(stage_bytes(case, x[1], dom) for x in insts) / n_inst
    dom_us = stage_us[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = None if args.tokens else measured_traffic(dom, args.config)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": int(dom_bytes), "avg_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, insts[0], args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "us_per_layer": round(r["us_per_layer"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: M={case.M} E={case.E} top-k={case.k} H={case.H} I={case.I} "
                        f"{case.routing} routing, {'UE8M0' if case.scale_fmt else 'fp32'} activation scales",
            "M": case.M, "E": case.E, "top_k": case.k, "hidden": case.H, "intermediate": case.I,
            "instances": n_inst, "bytes_per_layer": int(r["bytes_per_layer"]),
            "hbm_roofline_us": round(r["bytes_per_layer"] / (HBM_PEAK_GBS * 1e3), 3),
        },
        "stages_us": {k: round(v, 3) for k, v in stage_us.items()},
        "roofline": roofline,
        # the whole layer against the same peak (roofline above: its dominant kernel alone)
        "layer_roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(r["gbs"] / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


KERNEL_SOURCES = {
    "token_gate_up_swiglu": ["block_fp8_mixture_route_amd/csrc/token.hip",
                             "block_fp8_mixture_route_amd/csrc/device.h",
                             "block_fp8_mixture_route_amd/csrc/router.h",
                             "block_fp8_mixture_route_amd/csrc/internal.h"],
}


def kernel_source_hash(kernel):
    """SHA-256 of the kernel's sources with comments and blank lines removed,
    so that a comment edit does not count as a kernel change."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()


def measured_traffic(kernel, config):
    """HBM bytes per launch of `kernel` from the hardware-counter summary in
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by the counters' reading for a
    plain copy of known size), or None when there is none or the kernel's
    sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def oracle_layer_seconds(case, inst, seconds, threads=None, min_runs=1):
    """The CPU oracle on one layer instance, repeated for about `seconds` (at
    least min_runs times); seconds per layer, runs, threads used."""
    import torch
    from oracle import oracle as O

    hidden, ids, w, W = inst
    used = torch.unique(ids[ids >= 0]).cpu()
    remap = torch.full((case.E,), -1, dtype=torch.int32)
    remap[used.long()] = torch.arange(used.numel(), dtype=torch.int32)
    ids_c = ids.cpu()
    ids_l = torch.where(ids_c >= 0, remap[ids_c.clamp(min=0).long()], ids_c).to(torch.int32)
    sel = used.to(W.w13.device).long()
    args = (hidden.cpu(), ids_l, w.cpu(), W.w13[sel].cpu(), W.w13_s[sel].cpu(), W.w2[sel].cpu(), W.w2_s[sel].cpu())
    np_args = [O.as_np(a) for a in args]
    full = O.num_threads()
    if threads is not None:
        O.set_threads(threads)
    try:
        used_threads = O.num_threads()  # the oracle's GEMMs spread their output rows over the threads
        t0 = time.time()
        n = 0
        while True:
            O.fused_moe(*np_args, scale_fmt=case.scale_fmt, clamp=case.clamp)
            n += 1
            if n >= min_runs and time.time() - t0 >= seconds:
                break
        return (time.time() - t0) / n, n, used_threads
    finally:
        O.set_threads(full)


def cpu_baseline(case, inst, seconds):
    """The CPU oracle on the same layer (instance 0), repeated for about
    `seconds`; throughput in the metric's unit (GB/s of compulsory bytes).

    Where one oracle run of the whole layer would take longer than `seconds`,
    the sample is the routes of the first n experts the layer uses (the rest
    dropped), n sized from a one-expert probe so a run takes about a tenth of
    `seconds`; the oracle's work is per route, so the layer's time is the
    sample's scaled by all routes over the sample's routes."""
    import torch
    from oracle import oracle as O

    hidden, ids, w, W = inst
    O.fused_moe  # the library is built and loaded before timing
    nbytes, _ = layer_bytes(case, ids)
    used = torch.unique(ids[ids >= 0])
    n_routes = int((ids >= 0).sum())

    def first_experts(n):
        keep = torch.isin(ids, used[:n])
        return (hidden, torch.where(keep, ids, torch.full_like(ids, -1)), w, W), int(keep.sum())

    probe, probe_routes = first_experts(1)
    log(f"cpu oracle: probe on the {probe_routes} routes of one expert of {used.numel()}")
    dt1, _, _ = oracle_layer_seconds(case, probe, 0.0)  # also warms
    n = used.numel()
    if dt1 * n > seconds:
        n = max(1, min(n, int(seconds / 10 / dt1)))
    sample, sample_routes = first_experts(n)
    log(f"cpu oracle: timing {sample_routes} of {n_routes} routes ({n} of {used.numel()} experts) "
        f"for about {seconds:.0f} s")
    dt, runs, threads = oracle_layer_seconds(case, sample, seconds)
    dt_layer = dt * n_routes / sample_routes
    log(f"cpu oracle: {dt * 1e3:.1f} ms per sample run over {runs} runs, {threads} thread(s); "
        f"{dt_layer * 1e3:.1f} ms/layer")
    what = ("whole layer" if n == used.numel() else
            f"routes of {n} of {used.numel()} experts ({sample_routes} of {n_routes} routes), time scaled "
            f"by routes to the whole layer")
    return {"value": round(nbytes / dt_layer / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{case.name} instance 0, {what}, {runs} runs ({dt * 1e3:.1f} ms each)",
            "us_per_layer": round(dt_layer * 1e6, 1)}


if __name__ == "__main__":
    main()
