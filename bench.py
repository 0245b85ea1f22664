"""Benchmark of the block-FP8 fused MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config decode_m1] [--instances N]

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
dominant kernel (its algorithmic bytes over its average duration: the
graph-timed step when the layer is that one kernel, otherwise HIP events the
library records between its launches, in eager calls queued back to back
behind a GPU spin), the kernel's HBM traffic from the hardware-counter
summary in profiles/ while the kernel's sources match it, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
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
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_fp8_mixture_route_amd as bfp8
    from block_fp8_mixture_route_amd import synth

    case = synth.LAYER_CASES[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 4 copies of {args.calibrate_copy_mib} MiB")

    # one instance first, to size the rotation
    t0 = time.time()
    first = synth.layer_inputs(case, 0, device=dev)
    b0, d0 = layer_bytes(case, first[1])
    n_inst = args.instances or max(1, min(64, math.ceil(4 * MALL_BYTES / b0)))
    insts = [first] + [synth.layer_inputs(case, i, device=dev) for i in range(1, n_inst)]
    torch.cuda.synchronize()
    log(f"{args.config}: {n_inst} instances generated in {time.time() - t0:.1f}s, "
        f"{b0 / 1e6:.2f} MB compulsory per layer (instance 0, {d0} active experts)")

    o = bfp8.opts(scale_fmt=case.scale_fmt, clamp_limit=case.clamp)
    stages = bfp8.fused_moe_stages(case.M, case.H, case.k, case.E, case.I, o)
    ws_bytes = bfp8.fused_moe_workspace_size(case.M, case.H, case.k, case.E, case.I, o)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    outs = [torch.empty(case.M, case.H, dtype=torch.bfloat16, device=dev) for _ in range(n_inst)]
    bytes_per = [layer_bytes(case, x[1])[0] for x in insts]
    torch.cuda.synchronize()

    hip = Hip()
    stream = hip.stream()
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
    for s in range(args.warmup):
        call(s % n_inst, o)
    hip.sync(stream)
    log(f"warm-up {args.warmup} steps done; stages: {stages}")

    # graph of one rotation (+ a partial rotation so that exactly K steps run)
    full, rem = divmod(args.steps, n_inst)
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

    # per-stage durations: each stage alone (BFP8MOE_FLAG_ONLY_STAGE), one
    # rotation captured in a graph and replayed, HIP events on the stream the
    # kernels run on around the replays: launch-to-launch time of the stage's
    # kernel, back to back as in the layer graph.  A stage past the first
    # reads what the whole calls above left in the workspace (same code path
    # and traffic; the values are not checked here).
    stage_us = {}
    reps = max(1, math.ceil(args.steps / n_inst))
    for s_, name in enumerate(stages):
        os_ = bfp8.opts(scale_fmt=case.scale_fmt, clamp_limit=case.clamp, flags=bfp8.FLAG_ONLY_STAGE(s_))
        _, g_s = hip.capture(stream, lambda: [call(i, os_) for i in range(n_inst)])
        hip.launch(g_s, stream)  # untimed replay
        hip.sync(stream)
        hip.record(ev0, stream)
        for _ in range(reps):
            hip.launch(g_s, stream)
        hip.record(ev1, stream)
        hip.sync()
        stage_us[name] = hip.elapsed_ms(ev0, ev1) * 1e3 / (reps * n_inst)
    log("stage us (each stage alone, graph-timed): " + ", ".join(f"{k}={v:.2f}" for k, v in stage_us.items()))

    dom = next(s_ for s_ in ("token_gate_up_swiglu", "decode_gate_up_swiglu", "gate_up_gemm") if s_ in stage_us)
    dom_bytes = sum(stage_bytes(case, x[1], dom) for x in insts) / n_inst
    dom_us = stage_us[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dom, args.config)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": int(dom_bytes), "avg_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, insts[0], args.cpu_seconds)

    hidden0, ids0 = insts[0][0], insts[0][1]
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: M={case.M} E={case.E} top-k={case.k} H={case.H} I={case.I} "
                        f"{case.routing} routing, {'UE8M0' if case.scale_fmt else 'fp32'} activation scales",
            "M": case.M, "E": case.E, "top_k": case.k, "hidden": case.H, "intermediate": case.I,
            "instances": n_inst, "bytes_per_layer": int(sum(bytes_per) / n_inst),
            "hbm_roofline_us": round(sum(bytes_per) / n_inst / (HBM_PEAK_GBS * 1e3), 3),
        },
        "stages_us": {k: round(v, 3) for k, v in stage_us.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


KERNEL_SOURCES = {
    "token_gate_up_swiglu": ["block_fp8_mixture_route_amd/csrc/token.hip",
                             "block_fp8_mixture_route_amd/csrc/device.h"],
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


def cpu_baseline(case, inst, seconds):
    """The CPU oracle on the same layer (instance 0), repeated for about
    `seconds`; throughput in the metric's unit (GB/s of compulsory bytes)."""
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
    nbytes, _ = layer_bytes(case, ids)
    O.fused_moe(*np_args, scale_fmt=case.scale_fmt, clamp=case.clamp)  # warm
    t0 = time.time()
    n = 0
    while True:
        O.fused_moe(*np_args, scale_fmt=case.scale_fmt, clamp=case.clamp)
        n += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / n
    threads = min(O.num_threads(), case.M)  # the oracle parallelises over tokens
    log(f"cpu oracle: {dt * 1e3:.1f} ms/layer over {n} runs, {threads} thread(s)")
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{case.name} instance 0, whole layer, {n} runs ({dt * 1e3:.1f} ms each)",
            "us_per_layer": round(dt * 1e6, 1)}


if __name__ == "__main__":
    main()
