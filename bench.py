#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the fused forward
(O, LSE; its one planner launch also plans the backward) and the backward (dQ, dK, dV) of the
block-sparse workload (batch 2, 16 heads, seq 4096,
head_dim 128, 64x64 blocks kept with p = 0.25 plus the diagonal), the only measured workload that
exercises every step of the path. Inputs are resident in HBM before the timed region starts.
Before the W warm-up steps, 0.25 s of untimed steps bring the graphics clock to its steady state
under this step (`settle`), so that short and long runs measure the same rate.

Prints one JSON line. `value` is algorithmic TFLOP/s: 4*D flops per visible (query, key) pair for
the forward plus 10*D for the backward (five products); masked and skipped work is not counted.
`roofline` describes the dominant kernel, timed live with HIP events on the library's stream;
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload.
`workloads` holds every measured workload on its own, measured before the headline step: the fp32
workload (batch 1, 2 heads, seq 64, head_dim 64) in microseconds and GB/s against the 8 TB/s HBM
peak; the forward of the four bf16 workloads and the backward of the block-sparse one in TFLOP/s
and % of the bf16 MFMA peak, each with a live-timed roofline entry for its kernels.
Secondary figures, measured after the timed region: `cold_cache` (the same step with 512 MiB
written before each one, so that the inputs come from HBM) and `gfx_clock` (the graphics clock
amdsmi reports while the step runs, giving `pct_of_clock_adjusted_bf16_peak`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--all]
       python bench.py --fwd-only N | --bwd-only N [--steps K] [--warmup W]   (one workload, for traces)
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

METRIC = "attention fwd/bwd TFLOP/s (bf16) + % of MFMA peak on 1 MI355X, seq 2048-8192"
SETTLE_S = 0.25   # seconds of untimed steps before the warm-up steps (see run_gpu)
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
KERNEL_NAMES = {0: "plan", 1: "fwd", 2: "bwd_pre", 3: "bwd_dkdv", 4: "bwd_dq", 5: "fwd_merge", 6: "bwd_dq_convert",
                7: "mask_pack"}


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events from the HIP runtime itself (they are recorded by the library on its stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b) -> float:
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


def visible_pairs(w, inp) -> int:
    """Number of (query, key) pairs the mask keeps, summed over batch and query heads."""
    import torch
    b, hq, sq, sk = w.batch, w.heads_q, w.seq_q, w.seq_k
    if w.mask == "none":
        return b * hq * sq * sk
    if w.mask == "causal":
        return b * hq * sq * (sq + 1) // 2
    if w.mask == "padding":
        return hq * int(sum(int(n) ** 2 for n in inp["lengths"].tolist()))
    lay = inp["layout"].to(torch.int64)
    rows = torch.clamp(sq - torch.arange(lay.shape[-2]) * w.block, max=w.block)
    cols = torch.clamp(sk - torch.arange(lay.shape[-1]) * w.block, max=w.block)
    per = (lay * rows[:, None] * cols[None, :]).sum()
    return int(per) * (1 if lay.dim() == 4 else b * hq)


def library_sources_sha256() -> str:
    """Hash of every source the HIP library is built from (kernels, C ABI, public header)."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "attention_attn_fwd_09_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".cpp", ".h")))
    files.append(os.path.join(root, "include", "attn.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hbm_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain copy of known
    size), or None when no summary matches the sources this library is built from."""
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
    if not os.path.isdir(root):
        return None
    digest = library_sources_sha256()
    for name in sorted(os.listdir(root)):
        if not name.endswith("_hbm_traffic.md"):
            continue
        with open(os.path.join(root, name)) as fh:
            for line in fh:
                if not line.startswith("traffic-record: "):
                    continue
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("workload") == workload and rec.get("sources_sha256") == digest:
                    k = rec.get("kernels", {}).get(kernel)
                    if k is not None:
                        return int(k["bytes_per_launch"])
    return None


KERNEL_CLASS = {v: k for k, v in KERNEL_NAMES.items()}


def set_hook(clib, cls, st, sp, cap, cnt):
    rc = clib.attn_set_timing_events(cls, st, sp, cap, ctypes.byref(cnt) if cnt is not None else None)
    if rc != 0:
        raise RuntimeError(f"attn_set_timing_events({cls}) failed: {rc}")


def timed_calls(torch, fn, clib, hip, classes, n=20, warm=10, settle_s=0.2):
    """Median ms of n calls of fn (one torch event pair per call on the current stream, which is the
    library's stream), after `warm` calls and settle_s seconds of untimed calls so that the clocks
    have left their idle state; and, for each kernel class in `classes`, the median over the same
    calls of that class's kernel time per call (HIP events the library records around each launch of
    the class on its stream). Returns (call_ms, {class: (kernel_ms, launches_per_call)})."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    cap = 4 * n
    hooks = {}
    for cls in classes:
        st, sp, cnt = hip.create(cap), hip.create(cap), ctypes.c_int32(0)
        set_hook(clib, cls, st, sp, cap, cnt)
        hooks[cls] = (st, sp, cnt)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    calls = sorted(a.elapsed_time(b) for a, b in ev)
    kernels = {}
    for cls, (st, sp, cnt) in hooks.items():
        set_hook(clib, cls, None, None, 0, None)
        k = cnt.value // n
        per_call = sorted(sum(hip.elapsed_ms(st[i * k + j], sp[i * k + j]) for j in range(k)) for i in range(n)) \
            if k > 0 else [0.0]
        kernels[cls] = (per_call[len(per_call) // 2], k)
        hip.destroy(st)
        hip.destroy(sp)
    return calls[len(calls) // 2], kernels


def kernel_roofline(name, ms, flops):
    """Roofline entry of one kernel: executed algorithmic flops per launch over its median time."""
    achieved = flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    return {"kernel": name, "ms": round(ms, 5), "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}


def measure_workloads(lib, torch, dev, clib, hip):
    """Every measured workload, each timed on its own (median of 20 calls after warm-up):
    c1 (fp32, launch-bound) in microseconds and GB/s of the call's tensors against the 8 TB/s HBM
    peak; c2-c5 forward, and the c5 backward, in algorithmic TFLOP/s (4*D flops per visible pair
    forward, 10*D backward) and % of the bf16 MFMA peak, each with its kernels' live-timed
    roofline entries (forward kernel: 4*D flops per visible pair; dK/dV pass 8*D; dQ pass 6*D)."""
    from attention_attn_fwd_09_amd.inputs import WORKLOADS, workload_inputs

    out = {}
    for cfg, w in WORKLOADS.items():
        inp = workload_inputs(cfg, with_do=w.backward)
        q, k, v = (inp[x].to(dev).contiguous() for x in ("q", "k", "v"))
        m = lib.Mask(kind=w.mask, lengths=None if inp["lengths"] is None else inp["lengths"].to(dev),
                     layout=None if inp["layout"] is None else inp["layout"].to(dev))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
        pairs = visible_pairs(w, inp)
        d = w.head_dim

        def fwd():
            lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse, workspace=ws)

        ms, kern = timed_calls(torch, fwd, clib, hip, (KERNEL_CLASS["fwd"], KERNEL_CLASS["plan"]))
        fl = 4 * d * pairs
        line = {"workload": w.name, "fwd_ms": round(ms, 5), "fwd_tflops": round(fl / ms / 1e9, 2),
                "fwd_pct_of_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2), "visible_pairs": pairs}
        if w.dtype == "f32":
            nbytes = (2 * q.numel() + k.numel() + v.numel()) * q.element_size() + lse.numel() * 4
            line.update({"fwd_us": round(ms * 1e3, 2), "io_bytes": int(nbytes),
                         "io_gb_s": round(nbytes / ms / 1e6, 2),
                         "io_pct_of_hbm_peak": round(100 * nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                         "bound": "launch latency (2 work items)"})
            fk = kern[KERNEL_CLASS["fwd"]][0]
            line["kernel"] = {"kernel": "fwd_f32", "us": round(fk * 1e3, 2),
                              "gb_s": round(nbytes / fk / 1e6, 2) if fk > 0 else None}
        else:
            line["roofline"] = kernel_roofline("fwd", kern[KERNEL_CLASS["fwd"]][0], fl)
            line["plan_ms"] = round(kern[KERNEL_CLASS["plan"]][0], 5)
        if w.backward:
            do = inp["do"].to(dev).contiguous()
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            wsb = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
            fwd()

            def bwd():
                lib.attn_bwd(q, k, v, o, do, lse, mask=m, scale=inp["scale"], dq=dq, dk=dk, dv=dv, workspace=wsb)

            cls = (KERNEL_CLASS["bwd_dkdv"], KERNEL_CLASS["bwd_dq"], KERNEL_CLASS["plan"])
            bms, bk = timed_calls(torch, bwd, clib, hip, cls)
            bfl = 10 * d * pairs
            line.update({"bwd_ms": round(bms, 5), "bwd_tflops": round(bfl / bms / 1e9, 2),
                         "bwd_pct_of_bf16_peak": round(100 * bfl / bms / 1e9 / PEAK_BF16_TFLOPS, 2),
                         "bwd_roofline": [kernel_roofline("bwd_dkdv", bk[cls[0]][0], 8 * d * pairs),
                                          kernel_roofline("bwd_dq", bk[cls[1]][0], 6 * d * pairs)],
                         "bwd_plan_ms": round(bk[cls[2]][0], 5)})
        log(json.dumps(line))
        out[f"c{cfg}"] = line
    return out


def run_gpu(args):
    import torch

    from attention_attn_fwd_09_amd import binding as lib
    from attention_attn_fwd_09_amd.inputs import WORKLOADS, workload_inputs

    cfg = 5
    w = WORKLOADS[cfg]
    dev = torch.device("cuda:0")
    inp = workload_inputs(cfg, with_do=True)
    q, k, v, do = (inp[x].to(dev).contiguous() for x in ("q", "k", "v", "do"))
    layout = inp["layout"].to(dev).contiguous()
    mask = lib.Mask(kind="block", layout=layout)
    scale = inp["scale"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, mask)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, mask)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # the forward's planner launch also writes the backward's two lists into the backward's
    # workspace (attn_fwd_with_bwd_plan), and the backward then launches no planner of its own
    def step():
        lib.attn_fwd(q, k, v, mask=mask, scale=scale, out=o, lse=lse, workspace=ws_f, stream=stream, bwd_plan=ws_b)
        lib.attn_bwd(q, k, v, o, do, lse, mask=mask, scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                     stream=stream, planned=True)

    pairs = visible_pairs(w, inp)
    d = w.head_dim
    flops_fwd = 4 * d * pairs
    flops_bwd = 10 * d * pairs
    flops_step = flops_fwd + flops_bwd
    # flops each kernel class executes per launch (its own products, recomputation included)
    kernel_flops = {1: 4 * d * pairs, 3: 8 * d * pairs, 4: 6 * d * pairs}
    kernel_bytes = {2: w.batch * w.heads_q * w.seq_q * (2 * d * 2 + 4)}

    hip = HipEvents()
    clib = lib.load_library()
    clib.attn_set_timing_events.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32)]
    clib.attn_set_timing_events.restype = ctypes.c_int

    # every workload on its own, before the headline step (this also takes the clocks out of their
    # idle state, so that the short default warm-up measures the steady state)
    workloads = measure_workloads(lib, torch, dev, clib, hip)

    # The graphics clock follows sustained load: a few hundred steps (about 0.1 s) after other work,
    # the step still runs about 6% slower than in steady state. SETTLE_S seconds of untimed steps
    # come before the caller's warm-up steps, so that a short run (few warm-up and timed steps)
    # measures the same steady state as a long one.
    settle_steps = 0
    settle_end = time.perf_counter() + args.settle_s
    while time.perf_counter() < settle_end:
        step()
        settle_steps += 1
        if settle_steps % 32 == 0:
            torch.cuda.synchronize()   # keeps the host from queueing far ahead of the GPU
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # which kernel dominates the step: bracket every class for a few untimed steps
    probe_steps = 3
    cap = 4 * probe_steps
    probes = {}
    for cls in KERNEL_NAMES:
        st, sp = hip.create(cap), hip.create(cap)
        cnt = ctypes.c_int32(0)
        clib.attn_set_timing_events(cls, st, sp, cap, ctypes.byref(cnt))
        probes[cls] = (st, sp, cnt)
    for _ in range(probe_steps):
        step()
    torch.cuda.synchronize()
    per_class = {}
    for cls, (st, sp, cnt) in probes.items():
        clib.attn_set_timing_events(cls, None, None, 0, None)
        n = cnt.value
        per_class[cls] = (sum(hip.elapsed_ms(st[i], sp[i]) for i in range(n)) / probe_steps, n // probe_steps)
        hip.destroy(st)
        hip.destroy(sp)
    dominant = max(per_class, key=lambda c: per_class[c][0])
    log("untimed probe steps, kernel ms per step: " +
        ", ".join(f"{KERNEL_NAMES[c]}={per_class[c][0]:.4f}x{per_class[c][1]}" for c in per_class))

    # timed region: the dominant kernel is bracketed on the library's stream
    st, sp = hip.create(args.steps), hip.create(args.steps)
    cnt = ctypes.c_int32(0)
    clib.attn_set_timing_events(dominant, st, sp, args.steps, ctypes.byref(cnt))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    clib.attn_set_timing_events(dominant, None, None, 0, None)
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    n_dom = cnt.value
    dom_ms = sum(hip.elapsed_ms(st[i], sp[i]) for i in range(n_dom)) / max(n_dom, 1)
    hip.destroy(st)
    hip.destroy(sp)

    tflops = flops_step / (ms_step * 1e-3) / 1e12
    if dominant in kernel_flops:
        achieved = kernel_flops[dominant] / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        achieved = kernel_bytes.get(dominant, 0) / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roofline["traffic"] = hbm_traffic(KERNEL_NAMES[dominant], w.name)
    roofline["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roofline["kernel"] = KERNEL_NAMES[dominant]
    roofline["kernel_ms"] = round(dom_ms, 5)

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch, "heads": w.heads_q, "seq_len": w.seq_q, "head_dim": d,
            "mask": "block 64x64, p=0.25 + diagonal (shared by all heads)",
            "step": "attn_fwd (its planner launch also plans the backward) + attn_bwd (planned)",
            "visible_pairs": pairs,
            "flops_per_step": flops_step,
            "fwd_tflops_share": round(flops_fwd / flops_step, 4),
        },
        "pct_of_bf16_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed": round(wall, 4),
        "settle": {"seconds": args.settle_s, "steps": settle_steps, "note": "untimed steps before the warm-up steps"},
        "roofline": roofline,
        "workloads": workloads,
    }
    # secondary figures, measured after the timed region: the same step with cold caches, and the
    # graphics clock the step runs at (for the clock-adjusted peak)
    cold = cold_cache_steps(torch, step, stream)
    cold["value"] = round(flops_step / (cold["ms_per_step_median"] * 1e-3) / 1e12, 2)
    result["cold_cache"] = cold
    clk = gfx_clock_under_load(torch, step)
    result["gfx_clock"] = clk
    if clk is not None:
        adj = PEAK_BF16_TFLOPS * clk["mhz_median"] / 2400.0
        result["pct_of_clock_adjusted_bf16_peak"] = round(100 * tflops / adj, 2)
    sample = None
    if not args.no_cpu_baseline:
        sample = cpu_baseline(w, inp, pairs)
    result["cpu_baseline"] = sample

    if args.all:
        forward_all(lib, torch, dev, WORKLOADS, workload_inputs)
    if args.copy_mib:
        # a plain device copy of known size: hardware byte counters read for it calibrate the
        # counters read for the attention kernels
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
    return result


def gfx_clock_under_load(torch, step, seconds=1.5, skip_s=0.5):
    """Median graphics clock (MHz) that amdsmi reports while `step` runs back to back for
    `seconds` (samples of the first `skip_s` seconds dropped); None when amdsmi is unavailable.
    The driver refreshes the value about once a second, so this runs outside the timed region."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
    except Exception as e:  # telemetry only: the measurement itself does not depend on it
        log(f"amdsmi unavailable ({e}); no clock reading")
        return None
    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.perf_counter()
        while not stop.is_set():
            try:
                mhz = amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclk")
            except Exception:
                mhz = None
            if isinstance(mhz, (int, float)) and time.perf_counter() - t0 >= skip_s:
                samples.append(float(mhz))
            time.sleep(0.02)

    th = threading.Thread(target=sampler)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not samples:
        return None
    samples.sort()
    return {"mhz_median": samples[len(samples) // 2], "mhz_min": samples[0], "mhz_max": samples[-1],
            "samples": len(samples), "source": "amdsmi current_gfxclk, untimed run of the same step"}


def cold_cache_steps(torch, step, stream, n=20, flush_mib=512):
    """Mean ms of `n` steps, each preceded (outside its event pair) by a 512 MiB write that
    evicts the inputs from L2 and the 256 MiB Infinity Cache."""
    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    ms = []
    for i in range(n):
        buf.fill_(i & 255)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del buf
    ms.sort()
    return {"ms_per_step_median": round(ms[len(ms) // 2], 5), "ms_per_step_min": round(ms[0], 5), "steps": n,
            "flush_mib": flush_mib}


def cpu_baseline(w, inp, pairs_total):
    """fp64 oracle (as it stands) on a bounded sample: forward + backward of a few (b, h) pairs."""
    import numpy as np

    import oracle

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max((i.get("num_threads", 1) for i in pools), default=1)
        if pools:
            blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in pools}))
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    q64, k64, v64, do64 = (inp[x].to(dtype=__import__("torch").float64).numpy() for x in ("q", "k", "v", "do"))
    spec = oracle.MaskSpec(kind="block", layout=inp["layout"].numpy(), block_q=w.block, block_k=w.block)
    heads_done = 0
    t0 = time.perf_counter()
    budget = 12.0
    total_heads = w.batch * w.heads_q
    while heads_done < total_heads:
        b, h = divmod(heads_done, w.heads_q)
        qs, ks, vs, dos = (x[b:b + 1, h:h + 1] for x in (q64, k64, v64, do64))
        sub = oracle.MaskSpec(kind="block", layout=spec.layout, block_q=w.block, block_k=w.block)
        oracle.attention_fwd(qs, ks, vs, sub, inp["scale"])
        oracle.attention_bwd(qs, ks, vs, dos, sub, inp["scale"])
        heads_done += 1
        if time.perf_counter() - t0 > budget:
            break
    secs = time.perf_counter() - t0
    flops = 14 * w.head_dim * pairs_total * heads_done / total_heads
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fwd+bwd of {heads_done} of {total_heads} (batch, head) pairs of the same workload, "
                      f"{secs:.1f} s; value counts the same algorithmic flops per pair as the GPU line",
            "seconds": round(secs, 2), "blas": blas}


def time_calls(torch, fn, n=20, warm=10, settle_s=0.2):
    """Median, min and mean milliseconds of n calls of fn after warm untimed calls and at least
    settle_s seconds of untimed calls (so that the clocks have left their idle state); one event
    pair per call on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2], ms[0], sum(ms) / len(ms)


def forward_all(lib, torch, dev, workloads, workload_inputs):
    """Extra diagnostics on stderr: forward-only TFLOP/s of every measured workload (median of 20
    calls after 10 warm-up calls; min and mean alongside) with the rate at which the call's tensors
    move (GB/s against the 8 TB/s HBM peak, the figure for the small launch-bound workload), then
    the backward of every bf16 workload, then split-KV against no split on shapes with few work
    items."""
    for cfg, w in workloads.items():
        inp = workload_inputs(cfg)
        q, k, v = (inp[x].to(dev).contiguous() for x in ("q", "k", "v"))
        m = lib.Mask(kind=w.mask, lengths=None if inp["lengths"] is None else inp["lengths"].to(dev),
                     layout=None if inp["layout"] is None else inp["layout"].to(dev))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
        med, mn, mean = time_calls(torch, lambda: lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse,
                                                                 workspace=ws))
        fl = 4 * w.head_dim * visible_pairs(w, inp)
        # bytes of the call's tensors, each moved once: Q, K, V read, O and LSE (fp32) written (for
        # the padding workload this counts the padded rows too)
        nbytes = (2 * q.numel() + k.numel() + v.numel()) * q.element_size() + lse.numel() * 4
        log(json.dumps({"workload": w.name, "fwd_ms": round(med, 5), "fwd_ms_min": round(mn, 5),
                        "fwd_ms_mean": round(mean, 5), "fwd_tflops": round(fl / med / 1e9, 2),
                        "pct_peak": round(100 * fl / med / 1e9 / PEAK_BF16_TFLOPS, 2),
                        "io_bytes": int(nbytes), "io_gbps": round(nbytes / med / 1e6, 1),
                        "io_pct_of_hbm_peak": round(100 * nbytes / med / 1e6 / 8000.0, 3)}))
    bwd_all_diag(lib, torch, dev, workloads, workload_inputs)
    split_kv_diag(lib, torch, dev)
    bwd_modes_diag(lib, torch, dev, workloads, workload_inputs)
    dense_mask_diag(lib, torch, dev)
    fp8_diag(lib, torch, dev, workloads, workload_inputs)


def forward_only(cfg: int, calls: int, warmup: int) -> dict:
    """Forward of one workload only (the same inputs and launch as the bench's workloads), timed
    over `calls` calls after `warmup` calls and 0.2 s of settling: one HIP event pair per call on
    the current stream, median and mean reported, TFLOP/s on visible pairs (4*D flops each)."""
    import torch

    from attention_attn_fwd_09_amd import binding as lib
    from attention_attn_fwd_09_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[cfg]
    if w.dtype != "bf16":
        raise SystemExit(f"--fwd-only takes a bf16 workload (2-5), not {cfg}")
    dev = torch.device("cuda:0")
    inp = workload_inputs(cfg)
    q, k, v = (inp[x].to(dev).contiguous() for x in ("q", "k", "v"))
    m = lib.Mask(kind=w.mask, lengths=None if inp["lengths"] is None else inp["lengths"].to(dev),
                 layout=None if inp["layout"] is None else inp["layout"].to(dev))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
    med, mn, mean = time_calls(torch, lambda: lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse,
                                                             workspace=ws), n=calls, warm=warmup)
    fl = 4 * w.head_dim * visible_pairs(w, inp)
    return {"workload": w.name, "calls": calls, "fwd_ms": round(med, 5), "fwd_ms_min": round(mn, 5),
            "fwd_ms_mean": round(mean, 5), "visible_pairs": visible_pairs(w, inp), "flops_per_call": fl,
            "fwd_tflops": round(fl / med / 1e9, 2), "pct_peak": round(100 * fl / med / 1e9 / PEAK_BF16_TFLOPS, 2)}


def backward_only(cfg: int, calls: int, warmup: int) -> dict:
    """Backward of one bf16 workload only (two-pass default; O and LSE from one forward, dO from the
    workload's seed), timed like forward_only; TFLOP/s counts 10*D flops per visible pair."""
    import torch

    from attention_attn_fwd_09_amd import binding as lib
    from attention_attn_fwd_09_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[cfg]
    if w.dtype != "bf16":
        raise SystemExit(f"--bwd-only takes a bf16 workload (2-5), not {cfg}")
    dev = torch.device("cuda:0")
    inp = workload_inputs(cfg, with_do=True)
    q, k, v, do = (inp[x].to(dev).contiguous() for x in ("q", "k", "v", "do"))
    m = lib.Mask(kind=w.mask, lengths=None if inp["lengths"] is None else inp["lengths"].to(dev),
                 layout=None if inp["layout"] is None else inp["layout"].to(dev))
    o, lse = lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
    med, mn, mean = time_calls(torch, lambda: lib.attn_bwd(q, k, v, o, do, lse, mask=m, scale=inp["scale"], dq=dq,
                                                             dk=dk, dv=dv, workspace=ws), n=calls, warm=warmup)
    pairs = visible_pairs(w, inp)
    fl = 10 * w.head_dim * pairs
    return {"workload": w.name, "calls": calls, "bwd_ms": round(med, 5), "bwd_ms_min": round(mn, 5),
            "bwd_ms_mean": round(mean, 5), "visible_pairs": pairs, "flops_per_call": fl,
            "bwd_tflops": round(fl / med / 1e9, 2), "pct_peak": round(100 * fl / med / 1e9 / PEAK_BF16_TFLOPS, 2)}


def fp8_diag(lib, torch, dev, workloads, workload_inputs):
    """Forward with fp8 (e4m3) inputs at the causal GQA workload's shape, against the same values
    in bf16; TFLOP/s counts 4*D flops per visible pair; the fp8 line is also given against the
    5.0 PFLOP/s dense fp8 MFMA peak."""
    cfg = 4
    w = workloads[cfg]
    inp = workload_inputs(cfg)
    q8, k8, v8 = (inp[x].float().to(torch.float8_e4m3fn).to(dev).contiguous() for x in ("q", "k", "v"))
    q16, k16, v16 = (x.to(torch.bfloat16) for x in (q8, k8, v8))
    m = lib.Mask(kind=w.mask)
    fl = 4 * w.head_dim * visible_pairs(w, inp)
    line = {"workload": w.name.replace("bf16", "fp8")}
    for label, (q, k, v) in (("fp8", (q8, k8, v8)), ("bf16", (q16, k16, v16))):
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        med, _, _ = time_calls(torch, lambda: lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse))
        line[f"{label}_ms"] = round(med, 5)
        line[f"{label}_tflops"] = round(fl / med / 1e9, 2)
    line["fp8_pct_of_fp8_peak"] = round(100 * line["fp8_tflops"] / PEAK_FP8_TFLOPS, 2)
    log(json.dumps(line))


def dense_mask_diag(lib, torch, dev):
    """Forward and backward under a dense element mask at the block-sparse workload's shape (pairs
    kept with p = 0.5 inside 64x64 blocks kept with p = 0.7); the pack of the mask to bits and a
    block layout is inside every call."""
    from attention_attn_fwd_09_amd.inputs import Workload, make_inputs

    w = Workload("fwdbwd_bf16_b2_h16_s4096_d128_dense_p05", "bf16", 2, 16, 16, 4096, 4096, 128, "dense",
                 backward=True, keep_prob=0.5)
    inp = make_inputs(w, 8000)
    q, k, v, do = (inp[x].to(dev).contiguous() for x in ("q", "k", "v", "do"))
    m = lib.Mask(kind="dense", dense=inp["dense"].to(dev).contiguous())
    pairs = int(inp["dense"].to(torch.int64).sum()) * w.batch * w.heads_q
    wsf = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fmed, _, _ = time_calls(torch, lambda: lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse,
                                                         workspace=wsf))
    bmed, _, _ = time_calls(torch, lambda: lib.attn_bwd(q, k, v, o, do, lse, mask=m, scale=inp["scale"], dq=dq, dk=dk,
                                                         dv=dv, workspace=wsb))
    log(json.dumps({"workload": w.name, "visible_pairs": pairs, "fwd_ms": round(fmed, 5),
                    "fwd_tflops": round(4 * w.head_dim * pairs / fmed / 1e9, 2), "bwd_ms": round(bmed, 5),
                    "bwd_tflops": round(10 * w.head_dim * pairs / bmed / 1e9, 2)}))


def bwd_all_diag(lib, torch, dev, workloads, workload_inputs):
    """Backward (two-pass default, `attn_bwd` alone, O and LSE from one forward) of every bf16
    workload with dO ~ N(0, 1) from the workload's seed: TFLOP/s counts 10*D flops per visible pair."""
    for cfg, w in workloads.items():
        if w.dtype != "bf16":
            continue
        inp = workload_inputs(cfg, with_do=True)
        q, k, v, do = (inp[x].to(dev).contiguous() for x in ("q", "k", "v", "do"))
        m = lib.Mask(kind=w.mask, lengths=None if inp["lengths"] is None else inp["lengths"].to(dev),
                     layout=None if inp["layout"] is None else inp["layout"].to(dev))
        o, lse = lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, m)), dtype=torch.uint8, device=dev)
        med, mn, _ = time_calls(torch, lambda: lib.attn_bwd(q, k, v, o, do, lse, mask=m, scale=inp["scale"], dq=dq,
                                                             dk=dk, dv=dv, workspace=ws))
        fl = 10 * w.head_dim * visible_pairs(w, inp)
        log(json.dumps({"workload": w.name + "_bwd", "bwd_ms": round(med, 5), "bwd_ms_min": round(mn, 5),
                        "bwd_tflops": round(fl / med / 1e9, 2),
                        "pct_peak": round(100 * fl / med / 1e9 / PEAK_BF16_TFLOPS, 2)}))


def bwd_modes_diag(lib, torch, dev, workloads, workload_inputs):
    """Backward of the block-sparse workload: the two-pass default against the single pass with
    atomic dQ accumulation (10*D algorithmic flops per visible pair in both)."""
    cfg = 5
    w = workloads[cfg]
    inp = workload_inputs(cfg, with_do=True)
    q, k, v, do = (inp[x].to(dev).contiguous() for x in ("q", "k", "v", "do"))
    m = lib.Mask(kind="block", layout=inp["layout"].to(dev).contiguous())
    o, lse = lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fl = 10 * w.head_dim * visible_pairs(w, inp)
    line = {"workload": w.name + "_bwd"}
    for label, flags in (("two_pass", 0), ("single_pass_atomic_dq", lib.ATTN_BWD_ATOMIC_DQ)):
        ws = torch.empty(max(1, lib.attn_bwd_workspace_bytes(q, k, m, flags=flags)), dtype=torch.uint8, device=dev)
        med, mn, _ = time_calls(torch, lambda: lib.attn_bwd(q, k, v, o, do, lse, mask=m, scale=inp["scale"], dq=dq,
                                                             dk=dk, dv=dv, workspace=ws, flags=flags))
        line[f"{label}_ms"] = round(med, 5)
        line[f"{label}_tflops"] = round(fl / med / 1e9, 2)
    log(json.dumps(line))


def split_kv_diag(lib, torch, dev):
    """Forward TFLOP/s with the automatic split-KV choice and with no split, on two shapes whose
    items leave most workgroup slots idle: few heads with long keys, and short query blocks
    against long keys (decode-like)."""
    from attention_attn_fwd_09_amd.inputs import Workload, make_inputs

    shapes = (Workload("fwd_bf16_b1_h2_s16384_d128_none", "bf16", 1, 2, 2, 16384, 16384, 128, "none"),
              Workload("fwd_bf16_b4_hq32_hkv8_sq128_sk32768_d128_none", "bf16", 4, 32, 8, 128, 32768, 128, "none"))
    for i, w in enumerate(shapes):
        inp = make_inputs(w, 7000 + i)
        q, k, v = (inp[x].to(dev).contiguous() for x in ("q", "k", "v"))
        m = lib.Mask()
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        line = {"workload": w.name}
        fl = 4 * w.head_dim * w.batch * w.heads_q * w.seq_q * w.seq_k
        for label, splits in (("auto", 0), ("nosplit", 1)):
            ws = torch.empty(max(1, lib.attn_fwd_workspace_bytes(q, k, m, kv_splits=splits)), dtype=torch.uint8,
                             device=dev)
            med, mn, _ = time_calls(torch, lambda: lib.attn_fwd(q, k, v, mask=m, scale=inp["scale"], out=o, lse=lse,
                                                                  workspace=ws, kv_splits=splits))
            line[f"{label}_splits"] = lib.attn_fwd_kv_splits(q, k, m, splits)
            line[f"{label}_ms"] = round(med, 5)
            line[f"{label}_tflops"] = round(fl / med / 1e9, 2)
        log(json.dumps(line))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks settle within about 50 ms of sustained work (about 100 steps): the default
    # warmup covers that, and the timed steps then measure the steady-state rate (about 0.4 s).
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warm-up steps (0 for counter runs, whose "
                         "per-dispatch records the settling steps would multiply)")
    ap.add_argument("--all", action="store_true", help="also print forward timings of every workload to stderr")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--fwd-only", type=int, default=0, metavar="CONFIG",
                    help="diagnostic: time only the forward of workload CONFIG (2-5) for --steps calls after "
                         "--warmup calls, print one JSON line and exit (for per-workload kernel traces)")
    ap.add_argument("--bwd-only", type=int, default=0, metavar="CONFIG",
                    help="diagnostic: likewise for the backward of workload CONFIG (2-5)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the attention path here is built and "
              "timed on a single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if args.fwd_only:
        print(json.dumps(forward_only(args.fwd_only, args.steps, args.warmup)), flush=True)
        return
    if args.bwd_only:
        print(json.dumps(backward_only(args.bwd_only, args.steps, args.warmup)), flush=True)
        return
    res = run_gpu(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
