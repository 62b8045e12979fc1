#!/usr/bin/env python3
"""Benchmark of the MoE W4A16 layer on one MI355X.

One step = the whole layer (route -> permute -> gate_up grouped GEMM with SiLU*mul -> down grouped
GEMM -> combine) over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the 800-token / 256-expert prefill shape (top-8, hidden 2048, intermediate 512, E2M1
group-32 bf16 scales).  Weights are rotated over L distinct copies (L * bytes of the experts the
routing touches >= 1 GiB) so that no step finds its weights in L2 or the Infinity Cache.  The K
timed steps run as eager launches with a HIP event between consecutive steps, after a warm-up that
brings clocks and caches to their steady state (by default at least 0.25 s of steps); the events are
created without the system-scope fence that torch's events add at every record (an L2 write-back and
invalidate that slows the next step).  `value` is the median per-step time (p10, p90, the mean and a
median from one-layer HIP graphs are under `timing`).  The
dominant kernel's roofline uses its mean HIP-event launch time from a per-kernel pass.  `workloads`
times the decode, 4096-token and skewed shapes the same way (timing only); `block` adds the whole MoE
block around the layer (router gate GEMM, shared expert); `cpu_baseline` times the CPU oracle on the
host cores (all of them, and one thread) on token samples and compares the GPU output on them.

Prints ONE JSON line on stdout; progress and the per-kernel table go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

import moe_inputs as mi

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 (and fp16) MFMA
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
RIDGE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
PAGES_US_800 = 5580.0  # Atlas page, GB10: W4A16 grouped-GEMM MoE layer at 800 tokens / 256 experts
METRIC = "MoE layer µs, TFLOP/s and weight GB/s (% roofline) at 800 tok/256 experts"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


WARMUP_SECONDS = 0.25  # default warm-up before each timed region: at least this long, and >= 10 steps

_hip_rt = None


def hip_runtime():
    """The HIP runtime that torch has loaded (the same instance, so that torch's streams are valid)."""
    global _hip_rt
    if _hip_rt is None:
        import ctypes

        path = "libamdhip64.so.7"
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        rt = ctypes.CDLL(path)
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip_rt = rt
    return _hip_rt


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence, used like torch.cuda.Event
    (record(), elapsed_time() in ms, read after a device synchronisation).  torch's timing events
    release to system scope when recorded, which writes back and invalidates the L2 caches and delays
    the work that follows (measured on MI355X: about 2 us per record between 800-token layers, 1.6 us
    between 1-token layers); these time the work between them without adding that."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = hip_runtime().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed (status {rc})")

    def record(self, stream=None):
        s = (stream or torch.cuda.current_stream()).cuda_stream
        rc = hip_runtime().hipEventRecord(self.h, self._ct.c_void_p(s))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed (status {rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = self._ct.c_float()
        rc = hip_runtime().hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed (status {rc})")
        return ms.value

    def __del__(self):
        try:
            if self.h:
                _hip_rt.hipEventDestroy(self.h)
        except Exception:
            pass


def warm_up(step, W: int) -> int:
    """Untimed steps before a timed region: W of them, or by default (W < 0) at least 10 and as many as
    fill WARMUP_SECONDS of wall time, so that clocks and caches are in their steady state (measured on
    MI355X: the first ~200 800-token layers after an idle period run up to 12 % slower).  Returns the
    count."""
    n = 0
    t0 = time.perf_counter()
    while (n < W) if W >= 0 else (n < 10 or time.perf_counter() - t0 < WARMUP_SECONDS):
        step(n)
        n += 1
        if W < 0 and n % 10 == 0:
            torch.cuda.synchronize()  # keep the wall clock on the GPU's work, not the launch queue
    torch.cuda.synchronize()
    return n


def warm_text(args) -> str:
    return str(args.warmup) if args.warmup >= 0 else f">= {WARMUP_SECONDS} s"


def warmup_count(W: int, step_ms: float) -> int:
    """Untimed steps before a further timed pass over steps of about step_ms: W, or by default enough
    to fill WARMUP_SECONDS (at least 10)."""
    return W if W >= 0 else max(10, math.ceil(WARMUP_SECONDS * 1e3 / max(step_ms, 1e-3)))


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


KERNEL_SOURCES = ["moe_w4a16_grouped_amd/csrc/grouped_gemm.hip", "moe_w4a16_grouped_amd/csrc/moe_common.h",
                  "moe_w4a16_grouped_amd/csrc/launch.h", "moe_w4a16_grouped_amd/build.py"]


def kernel_hash() -> str:
    """Hash of the sources that define the grouped-GEMM kernel (counter data is valid only for it)."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate_up launch from the committed counter runs, if taken on the current kernel."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d.get("gate_up_bytes") if d.get("kernel_hash") == kernel_hash() else None


def copy_probe():
    """Plain device copy of known size: the reference for scaling FETCH_SIZE / WRITE_SIZE counters."""
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}), flush=True)


def calibrate():
    """Measured ceilings of this machine beside the spec peaks: a timed device copy (read + write bytes
    per second) and a large bf16 GEMM from the vendor library (sustained matrix-core rate)."""
    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ev0, ev1 = TimingEvent(), TimingEvent()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(10):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    out["copy_gbps"] = round(2 * n * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9, 1)
    del src, dst
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        c = a @ b
    torch.cuda.synchronize()
    reps = 50
    ev0.record()
    for _ in range(reps):
        c = a @ b
    ev1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_tflops"] = round(2.0 * m ** 3 * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e12, 1)
    out["gemm_shape"] = f"{m}x{m}x{m} bf16, {reps} back-to-back launches"
    out["spec"] = {"hbm_gbps": HBM_PEAK_GBPS, "bf16_mfma_tflops": MFMA_BF16_PEAK_TFLOPS}
    print(json.dumps(out), flush=True)


def time_block(moe, wl, inp, x, copies, layout, args):
    """The whole MoE block from the hidden states: router gate GEMM, shared expert (a dense W4A16
    SwiGLU of intermediate size I) and the routed layer with the shared output added in the combine.
    Each weight copy gets its own router and shared-expert weights, rotated with the routed ones.
    Timed like the layer (median of per-step eager times, and from one-step graphs), plus per-stage
    events for the two extra stages."""
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    Is = I
    blk = mi.make_block_inputs(wl, Is)
    wr0 = dev_bf16(blk.w_router)
    sh0 = (dev(blk.w13s_q), dev(blk.w13s_s.view(np.int16)), dev(blk.w2s_q), dev(blk.w2s_s.view(np.int16)))
    if layout == moe.MOE_LAYOUT_PACKED:
        a, b = moe.moe_w4_prepack(sh0[0][None], sh0[1][None])
        c, d = moe.moe_w4_prepack(sh0[2][None], sh0[3][None])
        sh0 = (a[0], b[0], c[0], d[0])
    L = len(copies)
    extra = [(wr0, sh0)] + [(wr0.clone(), tuple(t.clone() for t in sh0)) for _ in range(L - 1)]
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_ffn_block_workspace_bytes(T, H, I, E, k, Is), dtype=torch.uint8, device="cuda")

    def step(i):
        q13, s13, q2, s2 = copies[i % L]
        wr, sh = extra[i % L]
        moe.moe_ffn_block_forward(x, wr, q13, s13, q2, s2, k, shared=sh, y=y, workspace=ws, weight_layout=layout)

    eager_ms = pctl(per_step_times(step, args.steps, args.warmup)[0])[0]
    graph_ms = None if args.no_graph else pctl(per_step_graph_times(step, L, args.steps, args.warmup))[0]
    # per-stage events for the two stages the block adds
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    so = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dws = torch.empty(max(moe.moe_dense_ffn_workspace_bytes(T, H, Is), 256), dtype=torch.uint8, device="cuda")
    evs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    nw = warmup_count(args.warmup, eager_ms)
    for i in range(nw + args.steps):
        wr, sh = extra[i % L]
        e = evs[i - nw] if i >= nw else None
        if e: e[0].record()
        moe.moe_router_logits(x, wr, logits=lg)
        if e: e[1].record()
        moe.moe_dense_ffn_w4a16(x, *sh, out=so, workspace=dws, weight_layout=layout)
        if e: e[2].record()
    torch.cuda.synchronize()
    router_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)
    shared_us = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e3)
    router_bytes = T * H * 2 + E * H * 2 + T * E * 4
    shared_bytes = mi.weight_bytes_per_expert(H, Is) + T * H * 2 + 2 * T * Is * 2 + T * H * 4
    out = {"us": round(eager_ms * 1e3, 2), "timing": "median of per-step eager times; graph_us from one-layer graphs",
           "graph_us": None if graph_ms is None else round(graph_ms * 1e3, 2), "shared_intermediate": Is,
           "router_us": round(router_us, 2), "router_gbps": round(router_bytes / (router_us * 1e-6) / 1e9, 1),
           "router_tflops": round(2.0 * T * H * E / (router_us * 1e-6) / 1e12, 3),
           "shared_us": round(shared_us, 2), "shared_gbps": round(shared_bytes / (shared_us * 1e-6) / 1e9, 1),
           "shared_tflops": round(6.0 * T * H * Is / (shared_us * 1e-6) / 1e12, 3)}
    log(f"bench: whole block {out['us']:.1f} us (router {router_us:.1f} us, shared expert {shared_us:.1f} us)")
    return out


def time_steps(step, L, args):
    """K steps: the median per-step eager time, the median from one-layer HIP graphs (ms) and the
    eager warm-up step count."""
    per, _, nw = per_step_times(step, args.steps, args.warmup)
    graph_ms = None if args.no_graph else pctl(per_step_graph_times(step, L, args.steps, args.warmup))[0]
    return pctl(per)[0], graph_ms, nw


def cpu_baseline_mx(inp, target_s: float, fn=None):
    """The MXFP4 oracle (or another variant's oracle function fn) timed like cpu_baseline."""
    import oracle

    fn = fn or oracle.moe_ffn_mx
    wl = inp.wl
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1)
    n = min(wl.T, cores)
    tok = np.sort(rng.choice(wl.T, n, replace=False))
    t0 = time.perf_counter()
    fn(inp, tokens=tok)
    dt = time.perf_counter() - t0
    if dt < target_s / 2 and n < wl.T:
        n2 = int(min(wl.T, max(n, n * (target_s / max(dt, 1e-3)))))
        tok = np.sort(rng.choice(wl.T, n2, replace=False))
        t0 = time.perf_counter()
        fn(inp, tokens=tok)
        dt = time.perf_counter() - t0
        n = n2
    return {"value": round(dt / n * wl.T * 1e6, 1), "unit": "us/layer", "cores": min(cores, n), "kind": "oracle",
            "sample": f"{n} of {wl.T} tokens of the same workload ({dt:.1f} s wall), scaled to {wl.T} tokens"}


def run_mxfp4(args):
    """The MXFP4 (W4A4) layer: x and h quantized per 1x32 on the fly, E2M1 x E2M1 products on the
    scaled FP4 matrix instruction.  Same workload shapes, rotation and timing as the W4A16 layer."""
    import moe_w4a16_grouped_amd as moe

    wl = mi.WORKLOADS[args.workload]
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    R = T * k
    log(f"bench: MXFP4 workload {wl.name} T={T} E={E} k={k} H={H} I={I}; generating inputs")
    inp = mi.make_mx_inputs(wl)
    x, logits = dev_bf16(inp.x), dev(inp.logits)
    ids0, _ = moe.moe_route_topk(logits, k)
    touched = int(torch.unique(ids0).numel())
    bpe = mi.mx_weight_bytes_per_expert(H, I)
    L = args.copies or max(1, math.ceil((1 << 30) / (touched * bpe)))
    w0 = (dev(inp.w13_q), dev(inp.w13_e), dev(inp.w2_q), dev(inp.w2_e))
    copies = [w0] + [tuple(t.clone() for t in w0) for _ in range(L - 1)]
    layout = moe.MOE_LAYOUT_PACKED if args.layout == "packed" else moe.MOE_LAYOUT_CANONICAL
    if layout == moe.MOE_LAYOUT_PACKED:
        copies = [moe.moe_mx_prepack(a, b) + moe.moe_mx_prepack(c, d) for (a, b, c, d) in copies]
        torch.cuda.synchronize()
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_ffn_mxfp4_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
    log(f"bench: {L} weight copies ({touched} of {E} experts touched); warmup {warm_text(args)}, steps {args.steps}")

    def step(i):
        q13, e13, q2, e2 = copies[i % L]
        moe.moe_ffn_forward_mxfp4(x, logits, q13, e13, q2, e2, k, y=y, workspace=ws, weight_layout=layout)

    eager_ms, graph_ms, nwarm = time_steps(step, L, args)
    ms = eager_ms  # the value: median per-step eager time
    log(f"bench: MXFP4 layer eager {eager_ms * 1e3:.1f} us, graph {graph_ms * 1e3 if graph_ms else 0:.1f} us")

    # per-kernel pass through the separate entry points
    bm = moe.moe_ffn_mxfp4_block_m(T, H, I, E, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    tiled = layout == moe.MOE_LAYOUT_PACKED and bm != 128  # the 128-row kernel reads row-major activations
    act = moe.MOE_ACT_TILED if tiled else moe.MOE_ACT_ROWS
    rows_cap = max(T, R, moe.moe_max_tiles(T, k, E, bm) * bm)
    xq = torch.empty((rows_cap, H // 2), dtype=torch.uint8, device="cuda")
    xs = torch.empty((rows_cap, H // 32), dtype=torch.uint8, device="cuda")
    hq = torch.empty((rows_cap, I // 2), dtype=torch.uint8, device="cuda")
    hs = torch.empty((rows_cap, I // 32), dtype=torch.uint8, device="cuda")
    O = torch.empty((R, H), dtype=torch.float32, device="cuda")
    names = ["route", "align", "quant_x", "gate_up", "down", "combine"]
    evs = [[TimingEvent() for _ in range(7)] for _ in range(args.steps)]
    al = None
    nw = warmup_count(args.warmup, eager_ms)
    for i in range(nw + args.steps):
        q13, e13, q2, e2 = copies[i % L]
        e = evs[i - nw] if i >= nw else None
        if e: e[0].record()
        moe.moe_route_topk(logits, k, ids, wts)
        if e: e[1].record()
        al = moe.moe_align(ids, E, bm)
        if e: e[2].record()
        if tiled:
            moe.moe_mx_quantize_tiles(x, al["sorted_ids"], k, al["tiles"], al["max_tiles"], al["num_tiles"], bm, xq, xs)
        else:
            moe.moe_mx_quantize(x, xq[:T], xs[:T])
        if e: e[3].record()
        moe.moe_grouped_gemm_mxfp4(xq, xs, al["sorted_ids"], k, q13, e13, al["tiles"], al["max_tiles"],
                                   al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, C=hq, Cs=hs, weight_layout=layout,
                                   act_layout=act)
        if e: e[4].record()
        moe.moe_grouped_gemm_mxfp4(hq, hs, None, 1, q2, e2, al["tiles"], al["max_tiles"], al["num_tiles"], bm,
                                   moe.MOE_EPI_NONE, R, moe.MOE_OUT_F32, C=O, weight_layout=layout, act_layout=act)
        if e: e[5].record()
        moe.moe_combine(O, al["inv_perm"], wts, y=y)
        if e: e[6].record()
    torch.cuda.synchronize()
    kern_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]) * 1e3) for j, n in enumerate(names)}
    log("bench: per-kernel us (events): " + ", ".join(f"{n}={v:.1f}" for n, v in kern_us.items()))

    us = ms * 1e3
    flops = 6.0 * R * H * I
    weight_bytes = touched * bpe
    g13 = 2 * I * H // 2 + 2 * I * (H // 32)
    gu_bytes = touched * g13 + T * H // 2 + T * H // 32 + R * I // 2 + R * I // 32
    gu_flops = 4.0 * R * H * I
    gu_us = kern_us["gate_up"]
    ridge = MFMA_FP4_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if gu_flops / gu_bytes < ridge:
        bound, achieved, peak, unit = "hbm", gu_bytes / (gu_us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", gu_flops / (gu_us * 1e-6) / 1e12, MFMA_FP4_PEAK_TFLOPS, "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 (E2M1 x E2M1, E8M0 per-32 scales; fp32 accumulation)",
        "data": "synthetic (seeded; E2M1 codes uniform, E8M0 scales 2^-8..2^-6, x and logits N(0,1))",
        "config": {"workload": f"{wl.name} MXFP4 (W4A4): {T} tokens, {E} experts top-{k}, hidden {H}, "
                               f"intermediate {I}", "method": "mxfp4", "tokens": T, "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "weight_copies": L, "touched_experts": touched,
                   "weight_layout": args.layout},
        "tflops": round(flops / (us * 1e-6) / 1e12, 3),
        "weight_gbps": round(weight_bytes / (us * 1e-6) / 1e9, 1),
        "timing": {"method": "median of per-step eager times (HIP event without system-scope fence between consecutive steps, after a warm-up of >= 0.25 s)",
                   "eager_us": round(eager_ms * 1e3, 2),
                   "graph_median_us": None if graph_ms is None else round(graph_ms * 1e3, 2)},
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "kernels_note": "per-kernel pass through the stand-alone entry points, whose down projection writes fp32 O for the combine; the layer keeps O as fp16 with in-band exponents (MXFP4 layer: from 256 rows)",
        "roofline": {"kernel": "gemm_mx_kernel (gate_up + SiLU*mul + h quantization)", "bound": bound,
                     "achieved": round(achieved, 2), "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None, "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops},
    }
    if not args.no_cpu_baseline:
        log(f"bench: timing the MXFP4 CPU oracle on a token sample (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline_mx(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_w4a8(args):
    """The W4A8 layer: x and h quantized to MXFP8 (E4M3, E8M0 per 32) on the fly, E4M3 x E2M1 products on
    the scaled matrix instruction against the MXFP4 weights.  Same workload shapes, rotation and timing
    as the W4A16 layer."""
    import moe_w4a16_grouped_amd as moe

    wl = mi.WORKLOADS[args.workload]
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    R = T * k
    log(f"bench: W4A8 workload {wl.name} T={T} E={E} k={k} H={H} I={I}; generating inputs")
    inp = mi.make_mx_inputs(wl)
    x, logits = dev_bf16(inp.x), dev(inp.logits)
    ids0, _ = moe.moe_route_topk(logits, k)
    touched = int(torch.unique(ids0).numel())
    bpe = mi.mx_weight_bytes_per_expert(H, I)
    L = args.copies or max(1, math.ceil((1 << 30) / (touched * bpe)))
    w0 = (dev(inp.w13_q), dev(inp.w13_e), dev(inp.w2_q), dev(inp.w2_e))
    copies = [w0] + [tuple(t.clone() for t in w0) for _ in range(L - 1)]
    layout = moe.MOE_LAYOUT_PACKED if args.layout == "packed" else moe.MOE_LAYOUT_CANONICAL
    if layout == moe.MOE_LAYOUT_PACKED:
        copies = [moe.moe_mx_prepack(a, b) + moe.moe_mx_prepack(c, d) for (a, b, c, d) in copies]
        torch.cuda.synchronize()
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_ffn_w4a8_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
    log(f"bench: {L} weight copies ({touched} of {E} experts touched); warmup {warm_text(args)}, steps {args.steps}")

    def step(i):
        q13, e13, q2, e2 = copies[i % L]
        moe.moe_ffn_forward_w4a8(x, logits, q13, e13, q2, e2, k, y=y, workspace=ws, weight_layout=layout)

    eager_ms, graph_ms, nwarm = time_steps(step, L, args)
    ms = eager_ms  # the value: median per-step eager time
    log(f"bench: W4A8 layer eager {eager_ms * 1e3:.1f} us, graph {graph_ms * 1e3 if graph_ms else 0:.1f} us")

    # per-kernel pass through the separate entry points
    bm = moe.moe_ffn_w4a8_block_m(T, H, I, E, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    tiled = layout == moe.MOE_LAYOUT_PACKED and bm != 128  # the 128-row kernel reads row-major activations
    act = moe.MOE_ACT_TILED if tiled else moe.MOE_ACT_ROWS
    rows_cap = max(T, R, moe.moe_max_tiles(T, k, E, bm) * bm)
    xq = torch.empty((rows_cap, H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((rows_cap, H // 32), dtype=torch.uint8, device="cuda")
    hq = torch.empty((rows_cap, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((rows_cap, I // 32), dtype=torch.uint8, device="cuda")
    O = torch.empty((R, H), dtype=torch.float32, device="cuda")
    names = ["route", "align", "quant_x", "gate_up", "down", "combine"]
    evs = [[TimingEvent() for _ in range(7)] for _ in range(args.steps)]
    nw = warmup_count(args.warmup, eager_ms)
    for i in range(nw + args.steps):
        q13, e13, q2, e2 = copies[i % L]
        e = evs[i - nw] if i >= nw else None
        if e: e[0].record()
        moe.moe_route_topk(logits, k, ids, wts)
        if e: e[1].record()
        al = moe.moe_align(ids, E, bm)
        if e: e[2].record()
        if tiled:
            moe.moe_mx8_quantize_tiles(x, al["sorted_ids"], k, al["tiles"], al["max_tiles"], al["num_tiles"], bm, xq,
                                       xs)
        else:
            moe.moe_mx8_quantize(x, xq[:T], xs[:T])
        if e: e[3].record()
        moe.moe_grouped_gemm_w4a8(xq, xs, al["sorted_ids"], k, q13, e13, al["tiles"], al["max_tiles"],
                                  al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, C=hq, Cs=hs, weight_layout=layout,
                                  act_layout=act)
        if e: e[4].record()
        moe.moe_grouped_gemm_w4a8(hq, hs, None, 1, q2, e2, al["tiles"], al["max_tiles"], al["num_tiles"], bm,
                                  moe.MOE_EPI_NONE, R, moe.MOE_OUT_F32, C=O, weight_layout=layout, act_layout=act)
        if e: e[5].record()
        moe.moe_combine(O, al["inv_perm"], wts, y=y)
        if e: e[6].record()
    torch.cuda.synchronize()
    kern_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]) * 1e3) for j, n in enumerate(names)}
    log("bench: per-kernel us (events): " + ", ".join(f"{n}={v:.1f}" for n, v in kern_us.items()))

    us = ms * 1e3
    flops = 6.0 * R * H * I
    weight_bytes = touched * bpe
    g13 = 2 * I * H // 2 + 2 * I * (H // 32)
    gu_bytes = touched * g13 + T * H + T * H // 32 + R * I + R * I // 32
    gu_flops = 4.0 * R * H * I
    gu_us = kern_us["gate_up"]
    # an 8-bit operand runs the scaled instruction at the fp8 rate
    ridge = MFMA_FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if gu_flops / gu_bytes < ridge:
        bound, achieved, peak, unit = "hbm", gu_bytes / (gu_us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", gu_flops / (gu_us * 1e-6) / 1e12, MFMA_FP8_PEAK_TFLOPS, "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 x fp4 (E4M3 x E2M1, E8M0 per-32 scales; fp32 accumulation)",
        "data": "synthetic (seeded; E2M1 codes uniform, E8M0 scales 2^-8..2^-6, x and logits N(0,1))",
        "config": {"workload": f"{wl.name} W4A8 (MXFP8 activations): {T} tokens, {E} experts top-{k}, hidden {H}, "
                               f"intermediate {I}", "method": "w4a8", "tokens": T, "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "weight_copies": L, "touched_experts": touched,
                   "weight_layout": args.layout},
        "tflops": round(flops / (us * 1e-6) / 1e12, 3),
        "weight_gbps": round(weight_bytes / (us * 1e-6) / 1e9, 1),
        "timing": {"method": "median of per-step eager times (HIP event without system-scope fence between consecutive steps, after a warm-up of >= 0.25 s)",
                   "eager_us": round(eager_ms * 1e3, 2),
                   "graph_median_us": None if graph_ms is None else round(graph_ms * 1e3, 2)},
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "kernels_note": "per-kernel pass through the stand-alone entry points, whose down projection writes fp32 O for the combine; the layer keeps O as fp16 with in-band exponents (W4A8 layer: from 16384 rows)",
        "roofline": {"kernel": "gemm_mx_kernel, E4M3 activations (gate_up + SiLU*mul + h quantization)", "bound": bound,
                     "achieved": round(achieved, 2), "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None, "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops},
    }
    if not args.no_cpu_baseline:
        import oracle

        log(f"bench: timing the W4A8 CPU oracle on a token sample (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline_mx(inp, args.cpu_seconds, oracle.moe_ffn_w4a8)
    print(json.dumps(result), flush=True)


def run_f8(args):
    """The FP8 (W8A8, per-1x128) layer: x and h quantized per 1x128 on the fly, E4M3 x E4M3 products
    on the FP8 matrix instruction.  Same workload shapes, rotation and timing as the W4A16 layer."""
    import oracle
    import moe_w4a16_grouped_amd as moe

    wl = mi.WORKLOADS[args.workload]
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    R = T * k
    log(f"bench: FP8 workload {wl.name} T={T} E={E} k={k} H={H} I={I}; generating inputs")
    inp = mi.make_f8_inputs(wl)
    x, logits = dev_bf16(inp.x), dev(inp.logits)
    ids0, _ = moe.moe_route_topk(logits, k)
    touched = int(torch.unique(ids0).numel())
    bpe = mi.f8_weight_bytes_per_expert(H, I)
    L = args.copies or max(1, math.ceil((1 << 30) / (touched * bpe)))
    w0 = (dev(inp.w13_q), dev(inp.w13_s), dev(inp.w2_q), dev(inp.w2_s))
    copies = [w0] + [tuple(t.clone() for t in w0) for _ in range(L - 1)]
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_ffn_f8_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
    log(f"bench: {L} weight copies ({touched} of {E} experts touched); warmup {warm_text(args)}, steps {args.steps}")

    def step(i):
        q13, s13, q2, s2 = copies[i % L]
        moe.moe_ffn_forward_f8(x, logits, q13, s13, q2, s2, k, y=y, workspace=ws)

    eager_ms, graph_ms, nwarm = time_steps(step, L, args)
    ms = eager_ms  # the value: median per-step eager time
    log(f"bench: FP8 layer eager {eager_ms * 1e3:.1f} us, graph {graph_ms * 1e3 if graph_ms else 0:.1f} us")

    # per-kernel pass through the separate entry points
    bm = moe.moe_ffn_f8_block_m(T, E, k)
    fused_h = bm == 128 and I % 128 == 0
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    xq = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")
    hf = torch.empty((R, I), dtype=torch.float32, device="cuda")
    hq = torch.empty((R, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((R, I // 128), dtype=torch.float32, device="cuda")
    O = torch.empty((R, H), dtype=torch.float32, device="cuda")
    names = ["route", "align", "quant_x", "gate_up", "quant_h", "down", "combine"]
    evs = [[TimingEvent() for _ in range(len(names) + 1)] for _ in range(args.steps)]
    nw = warmup_count(args.warmup, eager_ms)
    for i in range(nw + args.steps):
        q13, s13, q2, s2 = copies[i % L]
        e = evs[i - nw] if i >= nw else None
        if e: e[0].record()
        moe.moe_route_topk(logits, k, ids, wts)
        if e: e[1].record()
        al = moe.moe_align(ids, E, bm)
        if e: e[2].record()
        moe.moe_f8_quantize(x, xq, xs)
        if e: e[3].record()
        if fused_h:  # the 128-row kernel quantizes h in its epilogue
            moe.moe_grouped_gemm_f8(xq, xs, al["sorted_ids"], k, q13, s13, al["tiles"], al["max_tiles"],
                                    al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, moe.MOE_OUT_F8, C=hq, Cs=hs)
        else:
            moe.moe_grouped_gemm_f8(xq, xs, al["sorted_ids"], k, q13, s13, al["tiles"], al["max_tiles"],
                                    al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, C=hf)
        if e: e[4].record()
        if not fused_h:
            moe.moe_f8_quantize(hf, hq, hs)
        if e: e[5].record()
        moe.moe_grouped_gemm_f8(hq, hs, None, 1, q2, s2, al["tiles"], al["max_tiles"], al["num_tiles"], bm,
                                moe.MOE_EPI_NONE, R, moe.MOE_OUT_F32, C=O)
        if e: e[6].record()
        moe.moe_combine(O, al["inv_perm"], wts, y=y)
        if e: e[7].record()
    torch.cuda.synchronize()
    kern_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]) * 1e3) for j, n in enumerate(names)}
    log("bench: per-kernel us (events): " + ", ".join(f"{n}={v:.1f}" for n, v in kern_us.items()))

    us = ms * 1e3
    flops = 6.0 * R * H * I
    weight_bytes = touched * bpe
    g13 = 2 * I * H + 2 * I * (H // 128) * 4
    gu_bytes = touched * g13 + T * H + T * (H // 128) * 4 + (R * I + R * (I // 128) * 4 if fused_h else R * I * 4)
    gu_flops = 4.0 * R * H * I
    gu_us = kern_us["gate_up"]
    ridge = MFMA_FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if gu_flops / gu_bytes < ridge:
        bound, achieved, peak, unit = "hbm", gu_bytes / (gu_us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", gu_flops / (gu_us * 1e-6) / 1e12, MFMA_FP8_PEAK_TFLOPS, "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (E4M3 x E4M3, fp32 per-1x128 scales; fp32 accumulation)",
        "data": "synthetic (seeded; E4M3 weight codes with a geometric exponent field, fp32 scales, "
                "x and logits N(0,1))",
        "config": {"workload": f"{wl.name} FP8 (W8A8, per-1x128): {T} tokens, {E} experts top-{k}, hidden {H}, "
                               f"intermediate {I}", "method": "f8", "tokens": T, "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "weight_copies": L, "touched_experts": touched},
        "tflops": round(flops / (us * 1e-6) / 1e12, 3),
        "weight_gbps": round(weight_bytes / (us * 1e-6) / 1e9, 1),
        "timing": {"method": "median of per-step eager times (HIP event without system-scope fence between consecutive steps, after a warm-up of >= 0.25 s)",
                   "eager_us": round(eager_ms * 1e3, 2),
                   "graph_median_us": None if graph_ms is None else round(graph_ms * 1e3, 2)},
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "kernels_note": "per-kernel pass through the stand-alone entry points, whose down projection writes fp32 O for the combine; the layer keeps O as fp16 with in-band exponents (FP8 layer: with 128-row tiles from 16384 rows)",
        "roofline": {"kernel": ("gemm_f8_mm (gate_up + SiLU*mul + h quantization)" if fused_h
                                else "gemm_f8_kernel (gate_up + SiLU*mul, fp32 h)"), "bound": bound,
                     "achieved": round(achieved, 2), "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None, "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops},
    }
    if not args.no_cpu_baseline:
        log(f"bench: timing the FP8 CPU oracle on a token sample (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline_mx(inp, args.cpu_seconds, oracle.moe_ffn_f8)
    print(json.dumps(result), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_set_threads(n: int) -> bool:
    """Thread count of the oracle's OpenMP runtime (the process-wide libgomp it links)."""
    import ctypes

    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


def cpu_baseline_w4a16(inp, y_gpu: np.ndarray, target_s: float, fn=None):
    """The CPU oracle as it stands, timed on the host cores on bounded token samples of the same
    workload and scaled to one whole layer: once with every core the process may use, once with one
    thread.  The all-core sample's outputs are also compared with the GPU's y on those tokens."""
    import oracle

    fn = fn or oracle.moe_ffn
    wl = inp.wl
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1)

    def timed(n_target, seconds):
        n = min(wl.T, n_target)
        tok = np.sort(rng.choice(wl.T, n, replace=False))
        t0 = time.perf_counter()
        ref = fn(inp, tokens=tok)
        dt = time.perf_counter() - t0
        if dt < seconds / 2 and n < wl.T:
            n = int(min(wl.T, max(n, n * (seconds / max(dt, 1e-3)))))
            tok = np.sort(rng.choice(wl.T, n, replace=False))
            t0 = time.perf_counter()
            ref = fn(inp, tokens=tok)
            dt = time.perf_counter() - t0
        return tok, ref, dt

    _omp_set_threads(cores)
    tok, ref, dt = timed(cores, target_s)
    out = {"value": round(dt / len(tok) * wl.T * 1e6, 1), "unit": "us/layer", "cores": min(cores, len(tok)),
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{len(tok)} of {wl.T} tokens of the same workload ({dt:.1f} s wall, {cores} threads), "
                     f"scaled to {wl.T} tokens"}
    if y_gpu is not None:
        d = np.abs(y_gpu[tok] - ref)
        rms = float(np.sqrt(np.mean(ref ** 2)))
        out["parity"] = {"tokens": int(len(tok)), "max_over_rms": round(float(d.max() / rms), 5),
                         "mean_rel": round(float(d.sum() / np.abs(ref).sum()), 6),
                         "bound": {"max_over_rms": 3e-2, "mean_rel": 5e-3}}
    if _omp_set_threads(1):
        tok1, _, dt1 = timed(1, target_s / 2)
        out["one_thread"] = {"value": round(dt1 / len(tok1) * wl.T * 1e6, 1), "unit": "us/layer", "cores": 1,
                             "sample": f"{len(tok1)} of {wl.T} tokens ({dt1:.1f} s wall, 1 thread), scaled to "
                                       f"{wl.T} tokens"}
        _omp_set_threads(cores)
    return out


def pctl(xs):
    a = np.asarray(xs, np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def per_step_times(step, K: int, W: int):
    """The warm-up (warm_up), then K steps with a HIP event between consecutive steps on the stream
    the layer runs on (torch's current stream), bracketed by device synchronisation.  Returns the K
    per-step durations (ms), the host wall time of the K steps (s) and the warm-up step count."""
    nw = warm_up(step, W)
    evs = [TimingEvent() for _ in range(K + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(K):
        step(nw + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(K)], wall, nw


def per_step_graph_times(step, L: int, K: int, W: int):
    """The same steps replayed from HIP graphs: one graph per weight copy, each holding one layer,
    replayed in rotation with a HIP event between consecutive replays.  Returns per-step ms."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(L):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    nw = warm_up(lambda i: graphs[i % L].replay(), W)
    evs = [TimingEvent() for _ in range(K + 1)]
    evs[0].record()
    for i in range(K):
        graphs[(nw + i) % L].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]


def measured_hbm(n_bytes: int = 1 << 30):
    """This box's measured bandwidth beside the 8 TB/s spec: a device copy (read + write bytes per
    second) and a read-only reduction of n_bytes."""
    src = torch.ones(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ev0, ev1 = TimingEvent(), TimingEvent()
    out = {}
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(10):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    out["copy_gbps"] = round(2 * n_bytes * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9, 1)
    v = src.view(torch.int64)
    for _ in range(3):
        r = v.sum()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(10):
        r = v.sum()
    ev1.record()
    torch.cuda.synchronize()
    out["read_gbps"] = round(n_bytes * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9, 1)
    del src, dst, v, r
    torch.cuda.empty_cache()
    return out


def layer_roofline(wl, touched: int):
    """Algorithmic bytes and flops of one layer (touched experts' packed weights and scales once, x,
    logits and y; intermediates excluded) and the roofline time, bound and floor."""
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    nbytes = touched * mi.weight_bytes_per_expert(H, I) + T * H * 2 + T * E * 4 + T * H * 2
    flops = 6.0 * T * k * H * I
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return nbytes, flops, ("hbm" if t_hbm >= t_mfma else "mfma"), max(t_hbm, t_mfma)


def setup_w4a16(moe, wl, layout, copies_arg=0, log_prefix="bench"):
    """Seeded inputs on the device, the touched expert count and L weight copies (prepacked when
    the layout asks), so that L x touched bytes >= 1 GiB and every step streams its weights."""
    inp = mi.make_inputs(wl)
    x, logits = dev_bf16(inp.x), dev(inp.logits)
    ids0, _ = moe.moe_route_topk(logits, wl.k)
    touched = int(torch.unique(ids0).numel())
    L = copies_arg or max(1, math.ceil((1 << 30) / (touched * mi.weight_bytes_per_expert(wl.H, wl.I))))
    w0 = (dev(inp.w13_q), dev(inp.w13_s.view(np.int16)), dev(inp.w2_q), dev(inp.w2_s.view(np.int16)))
    copies = [w0] + [tuple(t.clone() for t in w0) for _ in range(L - 1)]
    prepack_us = None
    if layout == moe.MOE_LAYOUT_PACKED:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        copies = [moe.moe_w4_prepack(a, b) + moe.moe_w4_prepack(c, d) for (a, b, c, d) in copies]
        torch.cuda.synchronize()
        prepack_us = (time.perf_counter() - t0) / L * 1e6
    return inp, x, logits, touched, L, copies, prepack_us


def time_workloads(moe, names, layout, args):
    """Timing only (no oracle) of further workloads, each in the default line's launch configuration:
    median, p10 and p90 of per-step eager times, the layer roofline and its fraction."""
    out = {}
    K = max(20, args.steps)
    for name in names:
        wl = mi.WORKLOADS[name]
        lay = layout if (wl.H % 128 == 0 and wl.I % 128 == 0) else moe.MOE_LAYOUT_CANONICAL
        inp, x, logits, touched, L, copies, _ = setup_w4a16(moe, wl, lay)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(moe.moe_ffn_workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k), 256), dtype=torch.uint8,
                         device="cuda")

        def step(i):
            q13, s13, q2, s2 = copies[i % L]
            moe.moe_ffn_forward(x, logits, q13, s13, q2, s2, wl.k, y=y, workspace=ws, weight_layout=lay)

        per, _, _ = per_step_times(step, K, args.warmup)
        med, p10, p90 = pctl(per)
        gmed = None
        if not args.no_graph:
            gmed = pctl(per_step_graph_times(step, L, K, args.warmup))[0]
        nbytes, flops, bound, t_min = layer_roofline(wl, touched)
        out[name] = {"us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
                     "graph_us": None if gmed is None else round(gmed * 1e3, 2),
                     "bound": bound, "roofline_us": round(t_min * 1e6, 2), "frac": round(t_min / (med * 1e-3), 4),
                     "tflops": round(flops / (med * 1e-3) / 1e12, 2),
                     "gbps": round(nbytes / (med * 1e-3) / 1e9, 1), "algorithmic_bytes": nbytes,
                     "algorithmic_flops": flops, "touched_experts": touched, "weight_copies": L,
                     "block_m": moe.moe_ffn_block_m(wl.T, wl.E, wl.k, lay)}
        log(f"bench: workload {name}: {out[name]['us']:.1f} us/layer (p10 {out[name]['p10_us']:.1f}, "
            f"p90 {out[name]['p90_us']:.1f}; graph {out[name]['graph_us']}), {bound} roofline frac {out[name]['frac']}")
        del inp, x, logits, copies, y, ws
        torch.cuda.empty_cache()
    return out


def run_w4a16(args):
    """The W4A16 layer (the default line)."""
    import moe_w4a16_grouped_amd as moe

    wl = mi.WORKLOADS[args.workload]
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    R = T * k
    layout = moe.MOE_LAYOUT_PACKED if args.layout == "packed" else moe.MOE_LAYOUT_CANONICAL
    log(f"bench: workload {wl.name} T={T} E={E} k={k} H={H} I={I}; generating inputs")
    inp, x, logits, touched0, L, copies, prepack_us = setup_w4a16(moe, wl, layout, args.copies)
    wbytes_all = E * mi.weight_bytes_per_expert(H, I)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_ffn_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
    log(f"bench: {L} weight copies of {wbytes_all / 1e6:.1f} MB ({touched0} of {E} experts touched); "
        f"warmup {warm_text(args)}, timed steps {args.steps}")

    def step(i):
        q13, s13, q2, s2 = copies[i % L]
        moe.moe_ffn_forward(x, logits, q13, s13, q2, s2, k, y=y, workspace=ws, weight_layout=layout)

    # The timed region: K eager steps, a HIP event between consecutive steps; value = the median.
    per, wall, nwarm = per_step_times(step, args.steps, args.warmup)
    med, p10, p90 = pctl(per)
    mean_ms = float(np.sum(per)) / args.steps
    log(f"bench: whole layer median {med * 1e3:.1f} us/step (p10 {p10 * 1e3:.1f}, p90 {p90 * 1e3:.1f}, "
        f"mean {mean_ms * 1e3:.1f}; host wall {wall / args.steps * 1e6:.1f} us/step)")
    y_host = mi.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    graph_med = None
    if not args.no_graph:
        graph_med = pctl(per_step_graph_times(step, L, args.steps, args.warmup))[0]
        log(f"bench: whole layer from HIP graphs (one layer per graph) median {graph_med * 1e3:.1f} us/step")

    # Per-kernel pass: the same layer through the individual entry points, HIP events between the
    # launches on the stream they run on (torch's current stream), K steps after W warmup steps.
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    bm = moe.moe_ffn_block_m(T, E, k, layout)
    # the layer runs its 128-row tiles (packed weights) on the exact fp16 path: x to fp16 first
    f16 = bm == 128 and layout == moe.MOE_LAYOUT_PACKED
    h = torch.empty((R, I), dtype=torch.float16 if f16 else torch.bfloat16, device="cuda")
    O = torch.empty((R, H), dtype=torch.float16, device="cuda")  # the layer's fp16 down output + side values
    Os = torch.empty((R, H // 8), dtype=torch.float32, device="cuda")
    if f16:
        x16 = torch.empty((T, H), dtype=torch.float16, device="cuda")
        xe = torch.empty((T,), dtype=torch.int32, device="cuda")
        hfl = torch.empty((max(moe.moe_max_tiles(T, k, E, bm), 1), (I + 31) // 32), dtype=torch.uint8, device="cuda")
        hex_ = torch.empty((R, (I + 31) // 32), dtype=torch.uint8, device="cuda")
    names = ["route", "align"] + (["x_to_f16"] if f16 else []) + ["gate_up", "down", "combine"]
    evs = [[TimingEvent() for _ in range(len(names) + 1)] for _ in range(args.steps)]
    al = None
    nw = warmup_count(args.warmup, med)
    for i in range(nw + args.steps):
        q13, s13, q2, s2 = copies[i % L]
        e = evs[i - nw] if i >= nw else None
        j = 0

        def mark():
            nonlocal j
            if e: e[j].record()
            j += 1
        mark()
        moe.moe_route_topk(logits, k, ids, wts)
        mark()
        al = moe.moe_align(ids, E, bm)
        mark()
        if f16:
            moe.moe_x_to_f16(x, x16=x16, x_exp=xe)
            mark()
            moe.moe_grouped_gemm_w4f16(x16, xe, None, al["sorted_ids"], k, q13, s13, al["tiles"], al["max_tiles"],
                                       al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, moe.MOE_OUT_H16, C=h,
                                       C_aux=hfl, C_aux2=hex_, weight_layout=layout)
            mark()
            moe.moe_grouped_gemm_w4f16(h, None, (hfl, hex_), None, 1, q2, s2, al["tiles"], al["max_tiles"],
                                       al["num_tiles"], bm, moe.MOE_EPI_NONE, R, moe.MOE_OUT_F16E, C=O, C_aux=Os,
                                       weight_layout=layout)
        else:
            moe.moe_grouped_gemm_w4a16(x, al["sorted_ids"], k, q13, s13, al["tiles"], al["max_tiles"],
                                       al["num_tiles"], bm, moe.MOE_EPI_SILU_MUL, R, C=h, weight_layout=layout)
            mark()
            moe.moe_grouped_gemm_w4a16(h, None, 1, q2, s2, al["tiles"], al["max_tiles"], al["num_tiles"], bm,
                                       moe.MOE_EPI_NONE, R, moe.MOE_OUT_F16E, C=O, C_side=Os, weight_layout=layout)
        mark()
        moe.moe_combine(O, al["inv_perm"], wts, y=y, O_side=Os)
        mark()
    torch.cuda.synchronize()
    kern_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]) * 1e3) for j, n in enumerate(names)}
    touched = int((al["counts"] > 0).sum().item())
    log("bench: per-kernel us (events): " + ", ".join(f"{n}={v:.1f}" for n, v in kern_us.items()))

    us = med * 1e3
    layer_bytes, flops, layer_bound, t_min = layer_roofline(wl, touched)
    weight_bytes = touched * mi.weight_bytes_per_expert(H, I)
    g13 = 2 * I * H // 2 + 2 * I * (H // 32) * 2
    # the dominant kernel (gate_up): its touched experts' weights and x, once (h excluded, an intermediate)
    gu_bytes = touched * g13 + T * H * 2
    gu_flops = 4.0 * R * H * I
    gu_us = kern_us["gate_up"]
    bound = "hbm" if gu_flops / gu_bytes < RIDGE else "mfma"
    if bound == "hbm":
        achieved, peak, unit = gu_bytes / (gu_us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        achieved, peak, unit = gu_flops / (gu_us * 1e-6) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    hbm = measured_hbm()
    log(f"bench: measured copy {hbm['copy_gbps']} GB/s (read + write), read {hbm['read_gbps']} GB/s")
    result = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(med, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(us / PAGES_US_800, 5) if wl.name == "pre800" else None,
        "dtype": "bf16",
        "data": "synthetic (seeded; E2M1 codes uniform, bf16 group-32 scales U[0.005,0.02], x and logits N(0,1))",
        "config": {"workload": f"{wl.name}: {T} tokens, {E} experts top-{k}, hidden {H}, intermediate {I}, "
                               f"W4 E2M1 group-32 bf16 scales", "tokens": T, "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "weight_copies": L, "touched_experts": touched,
                   "weight_layout": args.layout, "block_m": bm,
                   "prepack_us_per_copy": None if prepack_us is None else round(prepack_us, 1)},
        "tflops": round(flops / (us * 1e-6) / 1e12, 3),
        "weight_gbps": round(weight_bytes / (us * 1e-6) / 1e9, 1),
        "layer_gbps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
        "layer_roofline": {"bound": layer_bound, "algorithmic_bytes": layer_bytes, "algorithmic_flops": flops,
                           "roofline_us": round(t_min * 1e6, 2), "frac": round(t_min / (us * 1e-6), 4)},
        "timing": {"method": "median of per-step eager times (HIP event without system-scope fence between consecutive steps, after a warm-up of >= 0.25 s)",
                   "median_us": round(us, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
                   "mean_us": round(mean_ms * 1e3, 2),
                   # host clock around the K timed steps (launches to the final synchronisation) / K
                   "host_wall_us_per_step": round(wall / args.steps * 1e6, 2),
                   "graph_median_us": None if graph_med is None else round(graph_med * 1e3, 2)},
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "roofline": {"kernel": ("gemm_w4a16_mm, exact fp16 path" if f16 else "gemm_w4a16_tiled")
                               + " (gate_up + SiLU*mul)", "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(wl.name) if args.layout == "packed" else None,
                     "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops,
                     "duration_us": round(gu_us, 2),
                     "duration_from": "mean of K HIP-event launch durations in the per-kernel pass",
                     "measured_peak": {"read_gbps": hbm["read_gbps"], "copy_gbps": hbm["copy_gbps"],
                                       "frac_of_read": round(achieved / hbm["read_gbps"], 4) if bound == "hbm" else None}},
    }
    if not args.no_block:
        result["block"] = time_block(moe, wl, inp, x, copies, layout, args)
    del copies
    torch.cuda.empty_cache()
    if not args.no_workloads:
        others = [n for n in ("dec1", "dec8", "dec32", "dec64", "big4096", "skew8192") if n != wl.name]
        result["workloads"] = time_workloads(moe, others, layout, args)
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle on token samples (~{args.cpu_seconds:.0f} s + 1 thread)")
        result["cpu_baseline"] = cpu_baseline_w4a16(inp, y_host, args.cpu_seconds)
        pr = result["cpu_baseline"].get("parity")
        if pr:
            log(f"bench: GPU y vs oracle on {pr['tokens']} tokens: max/rms {pr['max_over_rms']}, "
                f"mean rel {pr['mean_rel']}")
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps before each timed region (default: at least 10, filling "
                         f"{WARMUP_SECONDS} s)")
    ap.add_argument("--workload", default="pre800", choices=sorted(mi.WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = enough for 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--layout", choices=["packed", "canonical"], default="packed",
                    help="weight layout the timed layer reads (packed = prepacked once, outside the timed region)")
    ap.add_argument("--copy-probe", action="store_true", help="run only the counter-calibration copy")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--calibrate", action="store_true", help="measure copy bandwidth and a vendor bf16 GEMM rate only")
    ap.add_argument("--method", choices=["w4a16", "mxfp4", "w4a8", "f8"], default="w4a16",
                    help="w4a16: bf16 activations, bf16 group scales (the default); mxfp4: W4A4 with E8M0 scales; "
                         "w4a8: MXFP8 activations on the MXFP4 weights; f8: W8A8 E4M3 with per-1x128 fp32 scales")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the timing-only lines of the other workloads (decode, 4096-token, skewed)")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the whole-block timing (router gate + shared expert + routed layer)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return
    if args.calibrate:
        calibrate()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    if args.method == "mxfp4":
        run_mxfp4(args)
        return
    if args.method == "f8":
        run_f8(args)
        return
    if args.method == "w4a8":
        run_w4a8(args)
        return

    run_w4a16(args)


if __name__ == "__main__":
    main()
