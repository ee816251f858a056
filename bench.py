#!/usr/bin/env python3
"""Benchmark: Monarch-factored video attention forward on one MI355X.

One step = one ``monarch_attn_fwd`` call (stage R + stage L) over the
21x30x52 token grid (32760 tokens), batch 1, 12 heads, head_dim 128, bf16,
on seeded synthetic Q/K/V (Q, K ~ N(0,1)/128^0.25, V ~ N(0,1)). The timed
region rotates over several input/output buffer sets (together larger than
the 256 MB MALL) so that every step reads its inputs from HBM.

Printed as one JSON line: tokens/s and ms/step of that step, the roofline
of the dominant kernel (timed with HIP events on the launch stream inside the
timed loop), the whole step against its two-stage roofline, side figures
(warm-cache step, tiled Monarch on structured data, the dense comparator),
and the CPU oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector), TFLOP/s
METRIC = "Monarch-attn ms/call & tokens/s at 21×30×52 grid, 12h d128; % HBM/MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_full_%s.json")
KERNEL_SOURCES = ["attn_bf16.h", "group_addr.h", "kernels_common.h", "monarch_attn.hip"]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # untimed steps before each timed loop: after an idle period the first ~20 ms of
    # launches run at lower clocks (measured: 0.245 ms/step after 10 warm-up steps,
    # 0.232 after 200), so the default warms for about 25 ms
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=3, help="rotating buffer sets in the timed loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip tiled/dense side figures")
    ap.add_argument("--profile-only", choices=["stage_l", "stage_r", "copy", "backward", "fp32", "stage_l_tiled"],
                    help="run only this kernel (or a plain device copy of one input tensor, the "
                         "calibration for byte counters; or the whole backward) --steps times on "
                         "the 21x30x52 workload (stage_l_tiled: stage L in 3x30 tiles on the "
                         "structured workload); for rocprofv3")
    ap.add_argument("--profile-warmup", type=int, default=0,
                    help="with --profile-only: launches before the --steps profiled ones (clock ramp)")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv output (kernel runs and "
                         "copy runs) into the per-launch HBM traffic of --kernel, written to "
                         "profiles/traffic_full_<kernel>.json")
    ap.add_argument("--kernel", default="stage_l", choices=["stage_l", "stage_r", "stage_l_tiled"])
    return ap.parse_args()


def kernel_source_hash():
    """Hash of the kernel sources with comments and whitespace removed (so that a
    comment edit does not void counter data taken on unchanged code)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_attention_video_attn_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def stage_work(N, d, heads, group_len):
    """(flops, compulsory bytes) of one stage over groups of `group_len` tokens (bf16)."""
    flops = 4.0 * N * d * heads * group_len
    nbytes = 8.0 * N * d * heads          # read Q, K, V-or-Y; write Y-or-O (2 B each)
    return flops, nbytes


def roofline_us(flops, nbytes):
    return max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6


# The GPU's clocks ramp up over the first tens of milliseconds of work after an
# idle period (0.245 ms/step after 10 warm-up steps against 0.232 after 200 on
# one box): every timed loop is preceded by its --warmup steps and, when those
# took less than this, by further untimed steps up to this much time of steady
# launches. The first call of a loop does not count: on a fresh process it also
# loads code objects (tens of milliseconds of host time with an idle GPU; with it
# counted, a 5-step warm-up ended with cold clocks and read 0.274 ms/step).
MIN_WARM_MS = 80.0


def time_loop(fn, steps, warmup, min_warm_ms=MIN_WARM_MS, info=None):
    """ms per call of fn(i) over `steps` calls, after `warmup` untimed calls (then more
    untimed calls until at least min_warm_ms of warm-up have run; their count goes
    to info["extra_warmup"] when info is a dict)."""
    import torch
    if warmup > 0 or min_warm_ms > 0:
        fn(0)   # may load code objects: not part of the clock warm-up
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(1, warmup):
        fn(i)
    torch.cuda.synchronize()
    extra = 0
    while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
        for _ in range(8):
            fn(warmup + extra)
            extra += 1
        torch.cuda.synchronize()
    if info is not None:
        info["extra_warmup"] = extra
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def repeat_stats(fn, steps, first_ms, repeats=5):
    """Median, p10 and p90 of ms/step over the headline loop and `repeats` more loops
    of the same `steps` calls (clocks already warm)."""
    import numpy as np
    vals = [first_ms] + [time_loop(fn, steps, 0, min_warm_ms=0.0) for _ in range(repeats)]
    return {"loops": len(vals), "steps_each": steps, "median_ms": round(float(np.median(vals)), 5),
            "p10_ms": round(float(np.percentile(vals, 10)), 5),
            "p90_ms": round(float(np.percentile(vals, 90)), 5)}


def cpu_baseline(wl, q, k, v):
    """The fp64 oracle, as it stands, on the host cores: whole 12-head calls."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    try:
        host_cores = len(os.sched_getaffinity(0))
    except Exception:
        host_cores = os.cpu_count() or 1
    grid = (wl.T, wl.H, wl.W)
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.monarch_attention(q, k, v, grid)
        calls += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or calls >= 5:
            break
    # cores: the threads the oracle ran on (its BLAS pool; the rest of it is one Python thread)
    return {"value": wl.n_tokens * calls / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "blas_threads": threads, "host_cores_available": host_cores,
            "sample": "%d whole call(s) of the fp64 NumPy oracle at 21x30x52, 12 heads, d128 "
                      "(stage R + stage L), %.1f s wall" % (calls, el)}


KERNEL_SYMBOL = {"stage_l": "group_attn_bf16", "stage_r": "block_attn_bf16", "stage_l_tiled": "group_attn_bf16"}


def _counter_rows(d, counter):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel, out_path=None):
    """Per-launch HBM bytes of one kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a device copy of one 100.6 MB tensor;
    written to out_path (default profiles/traffic_full_<kernel>.json) and returned."""
    wl_bytes = 12 * 32760 * 128 * 2
    sym = KERNEL_SYMBOL[kernel]

    def mean_for(rows, pred):
        vals = [v for name, v in rows if pred(name)]
        if not vals:
            raise SystemExit("no matching dispatches in counter output")
        return sum(vals) / len(vals)

    copy_pred = lambda name: "copyBuffer" in name   # device-to-device copies only
    fetch_scale = wl_bytes / (1024.0 * mean_for(_counter_rows(copy_fetch_dir, "FETCH_SIZE"), copy_pred))
    write_scale = wl_bytes / (1024.0 * mean_for(_counter_rows(copy_write_dir, "WRITE_SIZE"), copy_pred))
    kpred = lambda name: sym in name
    fetch = 1024.0 * mean_for(_counter_rows(fetch_dir, "FETCH_SIZE"), kpred) * fetch_scale
    write = 1024.0 * mean_for(_counter_rows(write_dir, "WRITE_SIZE"), kpred) * write_scale
    out = {"kernel": kernel, "kernel_symbol": sym, "kernel_source_hash": kernel_source_hash(),
           "fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "algorithmic_bytes": 8.0 * 32760 * 128 * 12}
    path = out_path or os.path.join(ROOT, "profiles", "traffic_full_%s.json" % kernel)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))
    return out


def measured_peaks(dev):
    """What this machine delivers to plain library calls, beside the vendor peaks: a
    device-to-device copy (read + write) and a bf16 GEMM through torch (hipBLASLt)."""
    import torch
    def timed(fn, iters):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters * 1e-3
    src = torch.empty(256 << 20, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    copy_gbps = 2.0 * src.numel() * 2 / t_copy / 1e9
    del src, dst
    n = 8192
    gen = torch.Generator(device=dev).manual_seed(11)
    x = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=gen)
    w = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=gen)
    t_mm = timed(lambda: torch.mm(x, w), 10)
    return {"device_copy_GBps": round(copy_gbps, 1),
            "torch_mm_bf16_8192_TFLOPs": round(2.0 * n ** 3 / t_mm / 1e12, 1)}


def profile_only(which, steps, warmup=0, n_sets=3):
    """Run one kernel `steps` times over rotating buffer sets (about 1.5 GB in all,
    more than the 256 MB MALL), so that every launch reads its inputs from HBM; the
    first `warmup` of them only bring the clocks up."""
    import torch
    import structured_attention_video_attn_amd as ma
    from workloads import WORKLOADS, make_qkv
    ma.load_library()
    wl = WORKLOADS["structured" if which == "stage_l_tiled" else "full"]
    T, H, W = wl.T, wl.H, wl.W
    dev = torch.device("cuda:0")
    dt = torch.float32 if which == "fp32" else torch.bfloat16
    base = [torch.from_numpy(x).to(dev).to(dt) for x in make_qkv(wl)]
    sets = []
    for _ in range(n_sets):
        q, k, v = (x.clone() for x in base)
        y = torch.empty_like(q)   # also the fp32 call's workspace
        ma.ma_stage_r_fwd(q, k, v, y, T, H, W)
        sets.append((q, k, v, y, torch.empty_like(q)))
    del base
    if which == "backward":
        gen = torch.Generator(device=dev).manual_seed(7)
        dout = torch.randn(sets[0][0].shape, generator=gen, device=dev).to(torch.bfloat16)
        grads = [torch.empty_like(dout) for _ in range(3)]
        wsb = torch.empty(ma.ma_bwd_workspace_bytes(1, 12, T, H, W) // 2, dtype=torch.bfloat16, device=dev)
        for q, k, v, y, o in sets:
            ma.ma_stage_l_fwd(q, k, y, o, T, H, W)
    torch.cuda.synchronize()
    for i in range(warmup + steps):
        q, k, v, y, o = sets[i % n_sets]
        if which == "backward":
            ma.monarch_attn_bwd(q, k, v, o, dout, *grads, wsb, T, H, W)
        elif which == "stage_l":
            ma.ma_stage_l_fwd(q, k, y, o, T, H, W)
        elif which == "stage_l_tiled":
            ma.ma_stage_l_fwd(q, k, y, o, T, H, W, 1, wl.tile[0], wl.tile[1])
        elif which == "stage_r":
            ma.ma_stage_r_fwd(q, k, v, y, T, H, W)
        elif which == "fp32":
            ma.monarch_attn_fwd(q, k, v, o, y, T, H, W)
        else:
            o.copy_(q)
    torch.cuda.synchronize()
    print("profiled %s x%d (after %d more)" % (which, steps, warmup), flush=True)


def main():
    args = parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, kernel=args.kernel)
        return
    if args.profile_only:
        profile_only(args.profile_only, args.steps, args.profile_warmup)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the method is measured on a single MI355X and "
              "the library has no multi-GPU path (asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import structured_attention_video_attn_amd as ma
    from workloads import CAUSAL_CHUNK_T, WORKLOADS, make_qkv

    ma.load_library()   # raises when the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = WORKLOADS["full"]
    T, H, W = wl.T, wl.H, wl.W
    N, d, heads = wl.n_tokens, wl.head_dim, wl.heads
    q_np, k_np, v_np = make_qkv(wl)
    up = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    base = [up(x) for x in (q_np, k_np, v_np)]
    ws_elems = ma.ma_workspace_bytes(1, heads, T, H, W, 1, 0, 0, d, ma.MA_BF16) // 2
    sets = []
    for s in range(max(1, args.sets)):
        q, k, v = (x.clone() for x in base)
        sets.append((q, k, v, torch.empty_like(q), torch.empty(ws_elems, dtype=torch.bfloat16, device=dev)))
    del base
    torch.cuda.synchronize()

    def step(i):
        q, k, v, o, ws = sets[i % len(sets)]
        ma.monarch_attn_fwd(q, k, v, o, ws, T, H, W)

    def step_r2(i):
        q, k, v, o, ws = sets[i % len(sets)]
        ma.monarch_attn_fwd(q, k, v, o, ws, T, H, W, r_axes=2)

    warm_info = {}
    ms = time_loop(step, args.steps, args.warmup, info=warm_info)
    reps = repeat_stats(step, args.steps, ms)
    ms_warm = time_loop(lambda i: step(0), args.steps, args.warmup)

    # Per-kernel durations, live, with events on the stream the kernels run on,
    # each launch bracketed inside the step it belongs to: stage L reads the Y that
    # stage R has just written, as in monarch_attn_fwd (launched back to back over
    # the rotating sets instead, stage L reads Y cold and takes ~8% longer).
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        q, k, v, o, ws = sets[i % len(sets)]
        y = ws[:q.numel()].view(q.shape)
        ev[i][0].record(stream)
        ma.ma_stage_r_fwd(q, k, v, y, T, H, W)
        ev[i][1].record(stream)
        ma.ma_stage_l_fwd(q, k, y, o, T, H, W)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    r_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    l_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    fr, br = stage_work(N, d, heads, W)
    fl, bl = stage_work(N, d, heads, T * H)
    roof_r, roof_l = roofline_us(fr, br), roofline_us(fl, bl)
    roof_min = roofline_us(fr + fl, 8.0 * N * d * heads)
    if l_us >= r_us:
        name, dur, f, b = "stage_l", l_us, fl, bl
    else:
        name, dur, f, b = "stage_r", r_us, fr, br
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma_bound = f / b >= ridge
    achieved = (f / (dur * 1e-6) / 1e12) if mfma_bound else (b / (dur * 1e-6) / 1e9)
    peak = PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS
    traffic = None
    if os.path.exists(TRAFFIC_FILE % name):
        with open(TRAFFIC_FILE % name) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("kernel") == name:
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s" if mfma_bound else "GB/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": name,
                "kernel_us": round(dur, 2), "algorithmic_flops": f, "algorithmic_bytes": b}

    extras = {}
    if not args.no_extras:
        # tiled Monarch on the structured workload, timed like the headline: rotating
        # buffer sets (3 x 503 MB) so that every call reads its inputs from HBM
        wl3 = WORKLOADS["structured"]
        base3 = [up(x) for x in make_qkv(wl3)]
        sets3 = []
        for _ in range(max(1, args.sets)):
            q3, k3, v3 = (x.clone() for x in base3)
            sets3.append((q3, k3, v3, torch.empty_like(q3), torch.empty(ws_elems, dtype=torch.bfloat16, device=dev)))
        del base3
        tt, th = wl3.tile

        def tiled_step(i):
            q3_, k3_, v3_, o3_, ws3_ = sets3[i % len(sets3)]
            ma.monarch_attn_tiled_fwd(q3_, k3_, v3_, o3_, ws3_, T, H, W, tt, th)
        ms_tiled = time_loop(tiled_step, args.steps, args.warmup)
        reps_tiled = repeat_stats(tiled_step, args.steps, ms_tiled)
        del sets3
        q, k, v, o, ws = sets[0]
        # frame-aligned blocks (r_axes = 2): b2 = H*W = 1560, b1 = T = 21
        ms_frames = time_loop(lambda i: step_r2(i), args.steps, args.warmup)
        ms_dense = time_loop(lambda i: ma.dense_attn_fwd(q, k, v, o), 3, 1)
        # chunk-causal forms (3-frame chunks): the whole sequence, and the last
        # chunk as one generation step over a cache of Y for frames 0..17
        ct = CAUSAL_CHUNK_T
        def causal(i):
            q_, k_, v_, o_, ws_ = sets[i % len(sets)]
            ma.monarch_attn_causal_fwd(q_, k_, v_, o_, ws_, T, H, W, ct)
        ms_causal = time_loop(causal, args.steps, args.warmup)
        t0 = T - ct

        def chunk_step(i):
            q_, k_, v_, o_, ws_ = sets[i % len(sets)]
            ma.monarch_attn_chunk_fwd(q_, k_, v_, ws_[:q_.numel()].view(q_.shape), o_, T, H, W, t0, ct)
        ms_step = time_loop(chunk_step, args.steps, args.warmup)
        fsz = H * W
        nq = ct * fsz                     # tokens of the chunk
        causal_l_flops = sum(4.0 * d * heads * W * (ct * H) * ((c + 1) * ct * H) for c in range(T // ct))
        roof_causal = roofline_us(*stage_work(N, d, heads, W)) + roofline_us(causal_l_flops, 8.0 * N * d * heads)
        step_bytes_r = 8.0 * nq * d * heads
        step_bytes_l = 2.0 * d * heads * (2 * nq + 2 * N)   # read Q (chunk), K and Y (all); write O (chunk)
        step_flops_l = 4.0 * d * heads * W * (ct * H) * (T * H)
        roof_step = roofline_us(4.0 * nq * d * heads * W, step_bytes_r) + roofline_us(step_flops_l, step_bytes_l)
        # backward of the headline operator (bf16): dq, dk, dv given dO
        dout = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                           dtype=torch.float32).to(torch.bfloat16)
        grads = [torch.empty_like(q) for _ in range(3)]
        wsb = torch.empty(ma.ma_bwd_workspace_bytes(1, heads, T, H, W, 1, 0, 0, d, ma.MA_BF16) // 2,
                          dtype=torch.bfloat16, device=dev)
        ma.monarch_attn_fwd(q, k, v, o, ws, T, H, W)
        ms_bwd = time_loop(lambda i: ma.monarch_attn_bwd(q, k, v, o, dout, *grads, wsb, T, H, W),
                           max(3, args.steps // 4), 2)
        y_fwd = ws[:q.numel()].view(q.shape)   # the forward's Y, kept as a training step would
        ms_bwd_y = time_loop(lambda i: ma.monarch_attn_bwd(q, k, v, o, dout, *grads, wsb, T, H, W, y=y_fwd),
                             max(3, args.steps // 4), 2)
        del grads, wsb, dout
        # the 81x30x52 workload (126360 tokens, 16 heads, Q, K, V ~ N(0, 1)): untiled and
        # in 9-frame x 30-row tiles
        wl4 = WORKLOADS["long"]
        T4, H4, W4, h4 = wl4.T, wl4.H, wl4.W, wl4.heads
        N4 = T4 * H4 * W4
        g4 = torch.Generator(device=dev).manual_seed(wl4.seed)
        q4, k4, v4 = (torch.randn(1, h4, N4, d, generator=g4, device=dev).to(torch.bfloat16) for _ in range(3))
        o4, ws4 = torch.empty_like(q4), torch.empty_like(q4)
        tt4, th4 = wl4.tile
        n4 = max(3, args.steps // 5)
        ms_long = time_loop(lambda i: ma.monarch_attn_fwd(q4, k4, v4, o4, ws4, T4, H4, W4), n4, 3)
        ms_long_tiled = time_loop(lambda i: ma.monarch_attn_tiled_fwd(q4, k4, v4, o4, ws4, T4, H4, W4, tt4, th4),
                                  n4, 3)
        del q4, k4, v4, o4, ws4
        roof_r4 = roofline_us(*stage_work(N4, d, h4, W4))
        roof_long = roof_r4 + roofline_us(*stage_work(N4, d, h4, T4 * H4))
        roof_long_tiled = roof_r4 + roofline_us(*stage_work(N4, d, h4, tt4 * th4))
        # fp32 path (fp32 matrix cores at head_dim 128): the 3x30x52 workload and the
        # full sequence; rooflines at the fp32 peak and 4-byte elements
        wl1 = WORKLOADS["chunk"]
        up32 = lambda x: torch.from_numpy(x).to(dev).to(torch.float32)
        q1, k1, v1 = (up32(x) for x in make_qkv(wl1))
        o1 = torch.empty_like(q1)
        ws1 = torch.empty_like(q1)
        ms_f32_chunk = time_loop(lambda i: ma.monarch_attn_fwd(q1, k1, v1, o1, ws1, wl1.T, wl1.H, wl1.W),
                                 args.steps, min(args.warmup, 20))
        del q1, k1, v1, o1, ws1
        q2, k2, v2 = (up32(x) for x in (q_np, k_np, v_np))
        o2 = torch.empty_like(q2)
        ws2 = torch.empty_like(q2)
        ms_f32_full = time_loop(lambda i: ma.monarch_attn_fwd(q2, k2, v2, o2, ws2, T, H, W),
                                max(3, args.steps // 10), 3)
        del q2, k2, v2, o2, ws2
        roof32 = lambda f_, b_: max(f_ / (PEAK_FP32_TFLOPS * 1e12), 2.0 * b_ / (PEAK_HBM_GBS * 1e9)) * 1e6
        N1 = wl1.T * wl1.H * wl1.W
        roof_f32_chunk = (roof32(*stage_work(N1, d, wl1.heads, wl1.W))
                          + roof32(*stage_work(N1, d, wl1.heads, wl1.T * wl1.H)))
        roof_f32_full = roof32(fr, br) + roof32(fl, bl)
        bwd_flops = 2.5 * (fr + fl)
        mp = measured_peaks(dev)
        roof_m = lambda f_, b_: max(f_ / (mp["torch_mm_bf16_8192_TFLOPs"] * 1e12),
                                    b_ / (mp["device_copy_GBps"] * 1e9)) * 1e6
        fr3, br3 = stage_work(N, d, heads, W)
        fl3, bl3 = stage_work(N, d, heads, tt * th)
        extras = {
            "tiled_structured_ms": round(ms_tiled, 4),
            "tiled_structured_repeats": reps_tiled,
            "tiled_structured_tokens_per_s": round(N / (ms_tiled * 1e-3), 1),
            "tiled_structured_roofline_frac": round(
                (roofline_us(fr3, br3) + roofline_us(fl3, bl3)) / (ms_tiled * 1e3), 4),
            "frame_blocks_ms": round(ms_frames, 4),
            "frame_blocks_roofline_frac": round(
                (roofline_us(*stage_work(N, d, heads, H * W)) + roofline_us(*stage_work(N, d, heads, T)))
                / (ms_frames * 1e3), 4),
            "causal_chunk3_ms": round(ms_causal, 4),
            "causal_chunk3_roofline_frac": round(roof_causal / (ms_causal * 1e3), 4),
            "chunk_step_t18_ms": round(ms_step, 4),
            "chunk_step_t18_roofline_frac": round(roof_step / (ms_step * 1e3), 4),
            "backward_ms": round(ms_bwd, 4),
            "backward_saved_y_ms": round(ms_bwd_y, 4),
            # algorithmic work of a backward, counted as FlashAttention does: 2.5x the forward's
            # matmul flops (five products against two); the kernels also recompute Y and P
            "backward_tflops": round(bwd_flops / (ms_bwd * 1e-3) / 1e12, 1),
            "backward_mfma_frac": round(bwd_flops / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fp32_chunk_3x30x52_ms": round(ms_f32_chunk, 4),
            "fp32_chunk_3x30x52_roofline_frac": round(roof_f32_chunk / (ms_f32_chunk * 1e3), 4),
            "fp32_full_ms": round(ms_f32_full, 4),
            "fp32_full_roofline_frac": round(roof_f32_full / (ms_f32_full * 1e3), 4),
            "dense_ms": round(ms_dense, 3),
            "dense_tflops": round(4.0 * N * N * d * heads / (ms_dense * 1e-3) / 1e12, 1),
            "monarch_speedup_vs_dense": round(ms_dense / ms, 2),
            "long_81x30x52_h16_ms": round(ms_long, 4),
            "long_81x30x52_h16_roofline_frac": round(roof_long / (ms_long * 1e3), 4),
            "long_tiled_9x30_ms": round(ms_long_tiled, 4),
            "long_tiled_9x30_roofline_frac": round(roof_long_tiled / (ms_long_tiled * 1e3), 4),
            "measured_peaks": mp,
            # the same rooflines with this box's measured copy and GEMM rates as the peaks
            "step_roofline_frac_measured_peaks": round(
                (roof_m(fr, br) + roof_m(fl, bl)) / (ms * 1e3), 4),
            "tiled_structured_roofline_frac_measured_peaks": round(
                (roof_m(fr3, br3) + roof_m(fl3, bl3)) / (ms_tiled * 1e3), 4),
        }

    out = {
        "metric": METRIC,
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q,K/128^0.25 and V; rotating buffer sets, inputs in HBM)",
        "config": {"workload": "monarch_attn_fwd 21x30x52 grid (32760 tokens), batch 1, 12 heads, "
                               "head_dim 128, blocks (b1,b2)=(630,52)",
                   "T": T, "H": H, "W": W, "batch": 1, "heads": heads, "head_dim": d,
                   "buffer_sets": len(sets)},
        "roofline": roofline,
        "step_roofline": {"roofline_us": round(roof_r + roof_l, 2), "measured_us": round(ms * 1e3, 2),
                          "frac": round((roof_r + roof_l) / (ms * 1e3), 4),
                          # the method's own minimum: Q, K, V read and O written once
                          # (Y never leaves the chip), all products at peak
                          "method_min_us": round(roof_min, 2),
                          "frac_method_min": round(roof_min / (ms * 1e3), 4),
                          "stage_r_us": round(r_us, 2), "stage_l_us": round(l_us, 2)},
        "repeats": reps,
        "extra_clock_warmup_steps": warm_info.get("extra_warmup", 0),
        "warm_ms_per_step": round(ms_warm, 5),
        # The pages' own figures, measured on NVIDIA GPUs with their Triton kernels at
        # shapes they do not give: context only, never a baseline for this line.
        "context": {
            "pages_kernel_speedup_vs_flashattention": "1.4x-11.8x (FA-2 on RTX 5090 up to 11.8x, "
                                                      "FA-3 on H100 up to 5.6x, FA-4 on B200 1.4x)",
            "pages_end_to_end": "16 FPS Self-Forcing video generation at 480p on one RTX 5090 "
                                "(FA-2: 11 FPS), with about 95% attention sparsity",
            "same_gpu_ratio_here": "monarch_speedup_vs_dense: the dense comparator over this step, "
                                   "both on this MI355X",
        },
    }
    out.update(extras)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, q_np, k_np, v_np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
