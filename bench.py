#!/usr/bin/env python3
"""Benchmark of the chunkwise key-only GLA forward on one MI355X.

Metric: forward tokens/s (fp16) on the 640x640-image workload (B=1, 40x40
stride-16 grid = 1,600 tokens, H=6, dk=dv=64, chunk 64, one call per scan
direction), with the other fp16 workloads reported beside it (the 1280x1280
image: 6,400 tokens; eight 640x640 images at H=12; the 12-block
direction-cycling stack over four 1280x1280 images at H=16), each with the
fraction of the HBM roofline reached by the path and by its dominant kernel,
and the counter-measured traffic where the kernel sources match it.

A step is one pass of the workload: one gla_fwd call per scan direction on
that call's own seeded inputs, already resident in device memory. Steps are
replayed from captured HIP graphs and timed with events on the launching
stream, mirroring the pages' protocol of event timing under graph replay
(GTR project page, "Accuracy-Latency Frontier"). The headline rotates
through copies of the step's inputs and outputs that together exceed twice
the 256 MB Infinity Cache, so the bytes come from HBM; the same steps on one
set of buffers (cache-warm) are reported beside it. By default the headline
times 20,000 steps (about a second of replays) and each other workload as
many steps as fill about a second, from a short timed pilot. One JSON line
is printed.

  python bench.py [--steps K] [--warmup W] [--workload I] [--no-also]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunkwise GLA fwd tokens/s (fp16) at 1600/6400 tokens; % of roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores, published
ROTATE_BYTES = 512 << 20  # rotating buffers: twice the 256 MB Infinity Cache
MAX_SETS = 64
KERNEL_SOURCES = ["gla_kernels.hip", "gla_chunk.h", "gla_tile.h", "gla_gated.hip",
                  "gla_runs.hip", "ssw_kernels.hip", "gla_device.h", "gla_launch.h"]


def source_sha() -> str:
    """Hash of the kernel sources' code: comments and blank lines are left
    out, so that counter traffic measured on a build stays attached to it
    when only its comments change."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "recurrent_vision_token_gla_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def per_unit_bytes(w):
    """Algorithmic bytes of the whole forward per (token, head): read q, k, gk
    (dk each) and v (dv), write o (dv)."""
    e = 2 if w.dtype == "f16" else 4
    return (3 * w.dk + 2 * w.dv) * e


def phase_bytes(w):
    """Algorithmic bytes each kernel must move per launch.

    single_pass: read q, k, gk, v; write o (the whole forward's own I/O; the
                 chunk summaries it publishes to its successors are not
                 counted)
    runs:        the same (one launch; its published run states not counted)
    summaries:   read k, gk, v; write per chunk-head U (f16 dk*dv) and the
                 pairs (a, row max of U) (2 f32 per key dim)
    scan:        read U and the pairs; write S (f16 dk*dv) and its row
                 scales (f32 dk)
    outputs:     read q, k, gk, v, S and its row scales; write o
    """
    e = 2 if w.dtype == "f16" else 4
    th = w.B * w.T * w.H
    ch = w.B * w.H * math.ceil(w.T / w.chunk)
    return {
        "single_pass": th * per_unit_bytes(w),
        "runs": th * per_unit_bytes(w),
        "summaries": th * (2 * w.dk + w.dv) * e + ch * (2 * w.dk * w.dv + 8 * w.dk),
        "scan": ch * (2 * w.dk * w.dv + 8 * w.dk + 2 * w.dk * w.dv + 4 * w.dk),
        "outputs": th * (3 * w.dk + 2 * w.dv) * e + ch * (2 * w.dk * w.dv + 4 * w.dk),
    }


def phase_flops(w):
    """Algorithmic matrix flops each kernel performs per launch (per
    token-head: the summary K^T V and the readout Q S, 2 dk dv each; the
    causal halves of the chunk's Q K^T and A V, C (dk + dv); the scan's
    2 dk dv / C is negligible and not counted)."""
    th = w.B * w.T * w.H
    summ = 2 * w.dk * w.dv
    outs = 2 * w.dk * w.dv + w.chunk * (w.dk + w.dv)
    return {"single_pass": th * (summ + outs), "runs": th * (summ + outs),
            "summaries": th * summ, "scan": 0, "outputs": th * outs}


def load_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch from profiles/traffic.json, or None
    if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    for r in rec.get("entries", []):
        if r.get("kernel") == kernel and r.get("workload") == workload:
            if r.get("source_sha") != source_sha():
                return None
            return r.get("hbm_bytes_per_launch")
    return None


def path_traffic(w, used):
    """Counter-measured HBM bytes of one call (the sum over the kernels its
    schedule launches) and their ratio to the path's algorithmic bytes, or
    None when any of them is missing or stale."""
    parts = [load_traffic(k, w.name) for k in used]
    if any(x is None for x in parts):
        return None
    path = w.B * w.T * w.H * per_unit_bytes(w)
    return {"bytes_per_call": sum(parts), "ratio": sum(parts) / path,
            "kernels": dict(zip(used, parts))}


def _graph(torch, stream, fn):
    """fn(s) captured once in a graph on a side stream (after one eager run)."""
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn(s)
    stream.wait_stream(s)
    torch.cuda.synchronize()
    return g


def _time_steps(torch, runs, steps, warmup):
    """Milliseconds per step over exactly `steps` steps (runs replayed in
    rotation), bracketed by synchronisations and timed with events."""
    for i in range(warmup):
        runs[i % len(runs)]()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        runs[i % len(runs)]()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, time.perf_counter() - wall0


def run_workload(w, steps, warmup, use_graph, torch, gla, W, timing_reps=30, max_seconds=None):
    dev = torch.device("cuda:0")
    calls = []
    for c in range(w.calls):
        q, k, v, g = W.workload_inputs(w, c)
        tq, tk, tv, tg = (torch.from_numpy(x).to(dev) for x in (q, k, v, g))
        calls.append(dict(q=tq, k=tk, v=tv, g=tg, dirs=w.directions(c),
                          out=torch.empty_like(tv), host=(q, k, v, g)))
    # rotating copies of every call's inputs and output (the contents do not
    # matter to the caches; set 0 holds the originals)
    step_bytes = sum(sum(c[n].numel() * c[n].element_size() for n in ("q", "k", "v", "g", "out"))
                     for c in calls)
    nsets = max(1, min(MAX_SETS, math.ceil(ROTATE_BYTES / step_bytes)))
    sets = [calls] + [[dict(c, q=c["q"].clone(), k=c["k"].clone(), v=c["v"].clone(),
                            g=c["g"].clone(), out=torch.empty_like(c["out"])) for c in calls]
                      for _ in range(nsets - 1)]
    ws = gla.alloc_workspace(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk, dev)
    stream = torch.cuda.current_stream()

    def step(cs, s=None):
        for c in cs:
            gla.fwd(c["q"], c["k"], c["v"], c["g"], w.grid_h, w.grid_w, c["dirs"], w.chunk,
                    out=c["out"], workspace=ws, stream=s)

    for cs in sets:
        step(cs)
    torch.cuda.synchronize()
    if use_graph:
        graphs = [_graph(torch, stream, lambda s, cs=cs: step(cs, s)) for cs in sets]
        runs = [g.replay for g in graphs]
    else:
        runs = [lambda cs=cs: step(cs) for cs in sets]

    # with max_seconds: as many steps (at most `steps`, at least 10) as fill
    # about that long, from a short timed pilot
    if max_seconds:
        pilot_ms, _ = _time_steps(torch, runs, 5, 2)
        steps = max(10, min(steps, int(max_seconds * 1e3 / max(pilot_ms, 1e-3))))
        warmup = min(warmup, steps)
    # headline: the sets in rotation; then the first set alone (cache-warm)
    ms_per_step, wall = _time_steps(torch, runs, steps, warmup)
    warm_ms, _ = _time_steps(torch, runs[:1], steps, warmup)

    # median single-step latency (event pair per step), rotating
    lat = []
    for i in range(min(50, max(10, steps // 4))):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        runs[i % nsets]()
        b.record()
        b.synchronize()
        lat.append(a.elapsed_time(b) * 1e3)

    # per-kernel durations: each kernel alone, `timing_reps` launches captured
    # back to back in one graph (no host gaps), cycling through every call of
    # every rotating set (the step's directions and inputs, so the inputs
    # come from HBM as in the step), timed with events on the stream the
    # kernels are launched on; and the step's first call repeated on one set
    # (cache-warm). The step's own schedule is the one gla_fwd picks; the
    # other schedules' kernels are timed for reference.
    flat = [cs[i] for cs in sets for i in range(len(cs))]
    sched = gla.auto_schedule(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk)

    def phase(name, c0, s):
        if name in ("single_pass", "runs"):
            return gla.fwd(c0["q"], c0["k"], c0["v"], c0["g"], w.grid_h, w.grid_w, c0["dirs"],
                           w.chunk, out=c0["out"], workspace=ws, stream=s,
                           schedule=gla.SCHED_SINGLE_PASS if name == "single_pass"
                           else gla.SCHED_RUNS)
        if name == "summaries":
            return gla.chunk_summaries(c0["k"], c0["v"], c0["g"], w.grid_h, w.grid_w, c0["dirs"],
                                       w.chunk, workspace=ws, stream=s)
        if name == "scan":
            return gla.state_scan(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk, ws, stream=s)
        return gla.chunk_outputs(c0["q"], c0["k"], c0["v"], c0["g"], w.grid_h, w.grid_w,
                                 c0["dirs"], w.chunk, workspace=ws, out=c0["out"], stream=s)

    def time_phase(name, rot):
        def fn(s):
            for r in range(timing_reps):
                phase(name, flat[r % len(flat)] if rot else calls[0], s)
        pg = _graph(torch, stream, fn)
        pg.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            pg.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / (3 * timing_reps)

    phase_us, phase_warm_us = {}, {}
    for name in ("single_pass", "runs", "summaries", "scan", "outputs"):
        if name in ("single_pass", "runs"):
            try:
                phase(name, calls[0], None)  # rejected on the host (nothing launched) if it does not fit
            except gla.GLAError:
                continue
        phase_us[name] = time_phase(name, True)
        phase_warm_us[name] = time_phase(name, False)
    # the kernels ran last on the workspace: re-run the step so outputs are current
    step(calls)
    torch.cuda.synchronize()
    used = ["single_pass"] if sched == gla.SCHED_SINGLE_PASS else ["summaries", "scan", "outputs"]
    return dict(calls=calls, steps=steps, ms_per_step=ms_per_step, warm_ms_per_step=warm_ms,
                wall_s=wall,
                lat_us=lat, phase_us=phase_us, phase_warm_us=phase_warm_us, ws=ws, used=used,
                sets=nsets, set_bytes=step_bytes,
                schedule="single_pass" if sched == gla.SCHED_SINGLE_PASS else "three_phase")


def launch_floor_us(torch):
    """Per-launch time of a one-element kernel, 20 captured back to back in one
    graph: the floor any single kernel launch pays in this timing protocol."""
    x = torch.zeros(1, device="cuda")
    return time_graph(torch, lambda s: x.add_(1.0))


def time_graph(torch, fn, reps=20, rounds=5):
    """Median microseconds per call of fn, from `reps` calls captured back to
    back in one graph and replayed `rounds` times (events on the launching
    stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / reps)
    return statistics.median(ts)


def token_sweep(torch, gla, W, np):
    """Self-relative scaling over the pages' token counts (16x16, 40x40, 80x80
    and 128x128 grids: 256, 1.6K, 6.4K, 16.4K tokens) for the configs' head
    shape (64/64) and the pages' operator shape (dk 32, dv 64); B 1, H 6,
    chunk 64, direction left->right, auto schedule."""
    out = []
    for dk, dv in ((64, 64), (32, 64)):
        for g in (16, 40, 80, 128):
            T = g * g
            q, k, v, gk = W.make_inputs(1, T, 6, dk, dv, np.float16, seed=7000 + g + dk)
            tq, tk, tv, tg = (torch.from_numpy(x).cuda() for x in (q, k, v, gk))
            ws = gla.alloc_workspace(1, 6, g, g, dk, dv, 64)
            o = torch.empty_like(tv)
            us = time_graph(torch, lambda s: gla.fwd(tq, tk, tv, tg, g, g, [0], 64, out=o,
                                                     workspace=ws, stream=s))
            nbytes = T * 6 * (3 * dk + 2 * dv) * 2
            out.append({"dk": dk, "dv": dv, "grid": f"{g}x{g}", "tokens": T, "us_per_call": us,
                        "tokens_per_s": T / (us * 1e-6),
                        "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "schedule": "single_pass" if gla.auto_schedule(1, 6, g, g, dk, dv, 64)
                        == gla.SCHED_SINGLE_PASS else "three_phase"})
    return out


def extra_kernels(torch, gla, W, np):
    """The fused output gate and the carried-state forward at the 640^2 shape
    and the Spatial SwiGLU core on its two workloads, each with its own HBM
    roofline fraction."""
    res = {}
    wl = W.WORKLOADS[1]
    q, k, v, gk = W.workload_inputs(wl, 0)
    z, wn = W.make_gate_inputs(wl.B, wl.T, wl.H, wl.dv, np.float16, seed=7100)
    tq, tk, tv, tg, tz = (torch.from_numpy(x).cuda() for x in (q, k, v, gk, z))
    tw = torch.from_numpy(wn).cuda()
    ws = gla.alloc_workspace(wl.B, wl.H, wl.grid_h, wl.grid_w, wl.dk, wl.dv, wl.chunk)
    y = torch.empty_like(tv)
    us = time_graph(torch, lambda s: gla.fwd_gated(tq, tk, tv, tg, tz, tw, W.GATE_EPS, wl.grid_h,
                                                   wl.grid_w, [0], wl.chunk, out=y, workspace=ws,
                                                   stream=s))
    nbytes = wl.T * wl.H * (3 * wl.dk + 3 * wl.dv) * 2  # + the gate rows
    res["gated_" + wl.name] = {"us_per_call": us, "tokens_per_s": wl.T / (us * 1e-6),
                               "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    # carried state: S_0 in, S_T out (fp32 [B][H][dk][dv] each) beside the forward
    s0 = torch.from_numpy(np.random.default_rng(7300).standard_normal(
        (wl.B, wl.H, wl.dk, wl.dv)).astype(np.float32)).cuda()
    sT = torch.empty_like(s0)
    o = torch.empty_like(tv)
    us = time_graph(torch, lambda s: gla.fwd_state(tq, tk, tv, tg, wl.grid_h, wl.grid_w, [0],
                                                   wl.chunk, s0=s0, s_final=sT, out=o,
                                                   workspace=ws, stream=s))
    nbytes = wl.T * wl.H * per_unit_bytes(wl) + 2 * wl.B * wl.H * wl.dk * wl.dv * 4
    res["state_" + wl.name] = {"us_per_call": us, "tokens_per_s": wl.T / (us * 1e-6),
                               "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    for sw in W.SSW_WORKLOADS:
        a, u, w, bias = W.make_ssw_inputs(sw.B, sw.T, sw.F, np.float16, seed=7200)
        ta, tu, tw2, tb = (torch.from_numpy(x).cuda() for x in (a, u, w, bias))
        h = torch.empty_like(tu)
        us = time_graph(torch, lambda s: gla.spatial_swiglu(ta, tu, tw2, tb, sw.grid_h, sw.grid_w,
                                                            out=h, stream=s))
        nbytes = sw.B * sw.T * sw.F * 2 * 3 + sw.F * 40  # a, u, h + weights and bias
        res[sw.name] = {"us_per_call": us, "tokens_per_s": sw.B * sw.T / (us * 1e-6),
                        "achieved_GBs": nbytes / (us * 1e-6) / 1e9,
                        "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return res


def parity_check(w, res, oracle, np, max_bh=4):
    """Max relative error of the benchmarked outputs against the oracle, on
    a sample of (batch, head) slices of every call."""
    errs = []
    for c in res["calls"]:
        q, k, v, g = c["host"]
        o = c["out"].double().cpu().numpy()
        bhs = [(b, h) for b in range(w.B) for h in range(w.H)][:max_bh]
        for b, h in bhs:
            sl = lambda x: x[b:b + 1, :, h:h + 1]
            ref = oracle.gla_forward(sl(q), sl(k), sl(v), sl(g), w.grid_h, w.grid_w,
                                     [c["dirs"][b]])
            errs.append(float(np.max(np.abs(o[b:b + 1, :, h:h + 1] - ref)) / np.max(np.abs(ref))))
    return max(errs)


def cpu_baseline(w, res, oracle, target_s=10.0):
    """The oracle, as it stands, timed on the host cores on the same inputs:
    whole steps until about target_s seconds have passed."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        for c in res["calls"]:
            q, k, v, g = c["host"]
            oracle.gla_forward(q, k, v, g, w.grid_h, w.grid_w, c["dirs"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    tokens = reps * w.calls * w.B * w.T
    return {"value": tokens / el, "unit": "tokens/s", "cores": oracle.oracle_threads(),
            "kind": "oracle",
            "sample": f"{reps} full step(s) of {w.name} ({w.calls} calls, all heads), "
                      f"{el:.2f} s wall"}


def summarize(w, res):
    tokens_step = w.calls * w.B * w.T
    value = tokens_step / (res["ms_per_step"] * 1e-3)
    th_call = w.B * w.T * w.H
    path_bytes_call = th_call * per_unit_bytes(w)
    call_us = res["ms_per_step"] * 1e3 / w.calls
    pb = phase_bytes(w)
    used = {k: res["phase_us"][k] for k in res["used"]}
    dom = max(used, key=used.get)
    ach = pb[dom] / (res["phase_us"][dom] * 1e-6) / 1e9
    fl = phase_flops(w)
    tflops = fl[dom] / (res["phase_us"][dom] * 1e-6) / 1e12
    path_flops = fl["single_pass"]
    return {
        "value": value,
        "call_us": call_us,
        "median_step_latency_us": statistics.median(res["lat_us"]),
        "path_roofline": {"bound": "hbm", "achieved": path_bytes_call / (call_us * 1e-6) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": path_bytes_call / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "bytes_per_call": path_bytes_call},
        "dominant": dom,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS,
                     "traffic": load_traffic(dom, w.name),
                     "kernel": dom, "algorithmic_bytes_per_launch": pb[dom],
                     "avg_launch_us": res["phase_us"][dom]},
        "mfma_roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": tflops / MFMA_F16_PEAK_TFLOPS,
                          "kernel": dom, "algorithmic_flops_per_launch": fl[dom],
                          "path_frac": path_flops / (call_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS},
        "path_traffic": path_traffic(w, res["used"]),
        "phase_us": res["phase_us"],
        "schedule": res["schedule"],
        "warm": {"value": tokens_step / (res["warm_ms_per_step"] * 1e-3),
                 "ms_per_step": res["warm_ms_per_step"],
                 "call_us": res["warm_ms_per_step"] * 1e3 / w.calls,
                 "kernel_us": res["phase_warm_us"]},
        "rotation": {"sets": res["sets"], "bytes_per_set": res["set_bytes"]},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=1, help="index into workloads.WORKLOADS")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-also", action="store_true", help="only the selected workload")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this implementation runs on one GPU only; there is no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from recurrent_vision_token_gla_amd import gla
    from recurrent_vision_token_gla_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gla.load()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: 3 copies of {n} bytes", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()

    w = W.WORKLOADS[args.workload]
    print(f"# bench: workload {w.index} {w.name} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    res = run_workload(w, args.steps, args.warmup, not args.no_graph, torch, gla, W)
    s = summarize(w, res)
    print(f"# {w.name}: {s['value']:.4g} tokens/s, {s['call_us']:.2f} us/call "
          f"({s['rotation']['sets']} rotating sets; warm {s['warm']['call_us']:.2f}), "
          f"path {100 * s['path_roofline']['frac']:.1f}% of HBM roofline, {s['schedule']}; kernels "
          + ", ".join(f"{k} {v:.2f} us" for k, v in s["phase_us"].items()),
          file=sys.stderr, flush=True)
    floor = launch_floor_us(torch)
    print(f"# launch floor (one-element kernel, graph-captured): {floor:.2f} us",
          file=sys.stderr, flush=True)

    import oracle
    parity = parity_check(w, res, oracle, np)
    print(f"# parity max rel err (sampled) {parity:.3e}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, res, oracle)
        print(f"# cpu oracle {cpu['value']:.4g} tokens/s on {cpu['cores']} threads",
              file=sys.stderr, flush=True)

    also = []
    # the other fp16 image workloads: 80x80 (6,400 tokens), eight 40x40 images
    # at H 12, and the 12-block stack of four 80x80 images at H 16
    extra = [i for i in (2, 3, 4) if i != args.workload] if not args.no_also else []
    for i in extra:
        wi = W.WORKLOADS[i]
        ri = run_workload(wi, max(10, args.steps // 4), max(3, args.warmup // 4),
                          not args.no_graph, torch, gla, W, max_seconds=1.0)
        si = summarize(wi, ri)
        print(f"# {wi.name}: {si['value']:.4g} tokens/s, {si['call_us']:.2f} us/call "
              f"({si['rotation']['sets']} rotating sets; warm {si['warm']['call_us']:.2f}), path "
              f"{100 * si['path_roofline']['frac']:.1f}% of HBM roofline, {si['schedule']}; kernels "
              + ", ".join(f"{k} {v:.2f} us" for k, v in si["phase_us"].items()),
              file=sys.stderr, flush=True)
        also.append({"workload": wi.name, "tokens_per_call": wi.B * wi.T, "steps": ri["steps"],
                     "value": si["value"], "unit": "tokens/s", "us_per_call": si["call_us"],
                     "path_roofline_frac": si["path_roofline"]["frac"],
                     "schedule": si["schedule"], "dominant": si["dominant"],
                     "dominant_frac": si["roofline"]["frac"],
                     "dominant_traffic": si["roofline"]["traffic"],
                     "path_traffic": si["path_traffic"], "kernel_us": si["phase_us"],
                     "warm": si["warm"], "rotation": si["rotation"]})
        del ri
        torch.cuda.empty_cache()

    sweep = extras = None
    if not args.no_also:
        sweep = token_sweep(torch, gla, W, np)
        for r in sweep:
            print(f"# sweep dk{r['dk']}/dv{r['dv']} {r['grid']}: {r['us_per_call']:.2f} us, "
                  f"{r['tokens_per_s']:.3g} tokens/s, {100 * r['hbm_frac']:.1f}% HBM, "
                  f"{r['schedule']}", file=sys.stderr, flush=True)
        extras = extra_kernels(torch, gla, W, np)
        for k2, r in extras.items():
            print(f"# {k2}: {r['us_per_call']:.2f} us, {100 * r['hbm_frac']:.1f}% HBM",
                  file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": s["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "grid": f"{w.grid_h}x{w.grid_w}",
                   "tokens_per_call": w.B * w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "calls_per_step": w.calls, "dir_mode": w.dir_mode,
                   "timing": "eager" if args.no_graph else "graph_replay"},
        "roofline": s["roofline"],
        "path_roofline": s["path_roofline"],
        "path_traffic": s["path_traffic"],
        "mfma_roofline": s["mfma_roofline"],
        "median_step_latency_us": s["median_step_latency_us"],
        "schedule": s["schedule"],
        "kernel_us": s["phase_us"],
        "warm": s["warm"],
        "rotation": s["rotation"],
        "launch_floor_us": floor,
        "parity_max_rel_err": parity,
        "cpu_baseline": cpu,
        "also": also,
        "sweep": sweep,
        "extras": extras,
        "kernel_source_sha": source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
