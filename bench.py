#!/usr/bin/env python3
"""Benchmark of the q8ta int8 path on one MI355X.

A step is one pass of the measured workload over resident synthetic inputs.
The default workload is the large linear:
    q8ta_linear GEMM  M=2048 K=4096 N=11008  (int8 x int8 -> int32 -> int8)
    -> dequantize_per_tensor of the int8 output to fp32
by default as one fused call (q8ta_linear_dq).  `value` is 2*M*N*K int8
operations per step divided by the wall-clock step time (TOPS).

Protocol: a fixed, time-based untimed phase (--settle-ms of back-to-back
steps, whatever --warmup says: the GPU clock needs tens of milliseconds of
load to settle), then --warmup untimed steps, then --steps timed steps, with
a HIP event every --steps/10 steps on the stream the library launches on.

The JSON line also carries
  roofline      the GEMM call's own rate (the mean launch time between the
                first and last event; median, p10 and p90 over the ten
                batches beside it) against the dense int8 matrix-core peak,
                and its HBM traffic per launch from the copy-calibrated
                rocprofv3 counters under profiles/ (null when the kernel
                source changed since they were taken);
  cpu_baseline  the CPU oracle timed on a sample of the same workload (a block
                of rows, median of 3 runs), its rows compared with the GPU's;
  extra         the other workloads of the op family (GEMV, quantize,
                dequantize, the transposed and forward convolutions, the fused
                chains), each timed in 5 batches of back-to-back launches queued
                behind a spin kernel (so that short launches are not paced by
                the host) -- HBM-bound ones rotate through enough buffer copies
                to exceed the 256 MB last-level cache -- and each output
                compared with the oracle over every element in the CPU leg of
                the same run (`oracle_bitexact`).

All oracle work happens in the CPU leg, after the GPU timing; --no-cpu-baseline
skips it (the flags are then null).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T]
                       [--no-cpu-baseline] [--no-extra] [--step fused|chain]
                       [--profile-only gemm|gemm-and-copy|deconv|deconv-and-copy]
       python bench.py --summarize-counters FETCH.csv WRITE.csv --traffic-of gemm_w8|deconv_fixed
       python bench.py --summarize-trace TRACE.{db,csv} [--kernel SUBSTRING]
                       [--window K --before SUBSTRING]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 TOPS (2·M·N·Kred) for q8ta_linear/conv_transposed; % of int8 MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix peak, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
CSRC = os.path.join(ROOT, "int8_quantized_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def valid_taps(out_size, in_size, k, s, p):
    """Number of (output, tap) pairs of one spatial axis the gather sums."""
    n = 0
    for o in range(out_size):
        for kk in range(k):
            num = o + p - kk
            if num >= 0 and num % s == 0 and num // s < in_size:
                n += 1
    return n


def deconv_ops(c):
    N, IC, H, W = c.x.shape if c.x_fp32 is None else c.x_fp32.shape
    OC = c.w.shape[0]
    th = valid_taps(c.H_out, H, c.Kh, c.stride[0], c.padding[0])
    tw = valid_taps(c.W_out, W, c.Kw, c.stride[1], c.padding[1])
    return 2 * N * OC * IC * th * tw


def conv_ops(c):
    """Exact int8 ops of the forward conv: taps inside the input only."""
    N, IC, H, W = c.x.shape
    OC = c.w.shape[0]
    th = sum(1 for oh in range(c.H_out) for k in range(c.Kh)
             if 0 <= oh * c.stride[0] - c.padding[0] + k * c.dilation[0] < H)
    tw = sum(1 for ow in range(c.W_out) for k in range(c.Kw)
             if 0 <= ow * c.stride[1] - c.padding[1] + k * c.dilation[1] < W)
    return 2 * N * OC * IC * th * tw


def file_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(name, src):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE in separate runs, scaled by what the same counters read for a
    copy kernel of known size) and stored beside the profiles; used only while
    the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != file_hash(src):
        return None
    return d.get("bytes_per_launch")


def pct(xs, q):
    """q-quantile of xs by linear interpolation between order statistics."""
    s = sorted(xs)
    if not s:
        return float("nan")
    pos = (len(s) - 1) * q
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def dist_us(ms, per_batch=1):
    """Statistics of per-launch durations in ms: the mean, and the median,
    p10, p90 and minimum over the samples given (each the mean launch time of
    a batch of `per_batch` back-to-back launches)."""
    us = [m * 1e3 for m in ms]
    return {"mean_us": round(statistics.mean(us), 2), "median_us": round(pct(us, 0.5), 2),
            "p10_us": round(pct(us, 0.1), 2), "p90_us": round(pct(us, 0.9), 2),
            "min_us": round(min(us), 2), "batches": len(us), "launches_per_batch": per_batch}


class Timer:
    """HIP events on torch's current stream (the stream libq8ta launches on)."""

    def __init__(self, torch):
        self.torch = torch
        # Calibrate the spin kernel that keeps the GPU busy while the host
        # enqueues a batch of short launches (cycles of its clock per us).
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda._sleep(1000)
        ev[0].record()
        torch.cuda._sleep(2_000_000)
        ev[1].record()
        torch.cuda.synchronize()
        rate = 2_000_000 / max(ev[0].elapsed_time(ev[1]) * 1e3, 1.0)
        self.cycles_per_us = min(max(rate, 50.0), 5000.0)

    def settle(self, fns, ms):
        """Back-to-back calls for at least `ms` milliseconds of wall time."""
        torch = self.torch
        t_end = time.perf_counter() + ms / 1e3
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                fns[i % len(fns)]()
                i += 1
            torch.cuda.synchronize()

    def batches(self, fns, n, batches=5):
        """Mean launch time (ms) of each of `batches` runs of n back-to-back
        calls cycling through `fns`, between two events per batch.  A spin
        kernel queued first (about 20 us of host time per call) lets the host
        enqueue the whole batch before the GPU reaches it, so that launches
        shorter than a Python call still run back to back: each figure is the
        GPU's own launch rate, not the host's call rate, and no event sits
        between two launches (an event costs a few microseconds of GPU time)."""
        torch = self.torch
        out = []
        for _ in range(batches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(int(self.cycles_per_us * min(20.0 * n + 200.0, 50_000.0)))
            e0.record()
            for i in range(n):
                fns[i % len(fns)]()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / n)
        return out


def summarize_trace(path, kernel=None, window=0, before=None):
    """Per-kernel duration statistics of a rocprofv3 kernel trace (the rocpd
    SQLite database or the kernel_trace CSV), as a text table.  With
    `window` and `before`: also the statistics of the last `window` launches
    of the kernels matching `kernel` that start before the first launch
    matching `before` (the timed steps of a run, which the benchmark follows
    with other kernels)."""
    rows = []
    if path.endswith(".db"):
        import sqlite3
        db = sqlite3.connect(path)
        for name, start, end in db.execute("select name, start, end from kernels"):
            rows.append((name, int(start), int(end)))
    else:
        import csv
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort(key=lambda r: r[1])
    by = {}
    for name, t0, t1 in rows:
        if kernel and kernel not in name:
            continue
        by.setdefault(name, []).append((t1 - t0) / 1e3)
    out = [f"{'calls':>6} {'mean_us':>9} {'median_us':>9} {'p10_us':>9} {'p90_us':>9} "
           f"{'min_us':>9} {'max_us':>9}  kernel"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{len(v):6d} {statistics.mean(v):9.2f} {pct(v, 0.5):9.2f} {pct(v, 0.1):9.2f} "
                   f"{pct(v, 0.9):9.2f} {min(v):9.2f} {max(v):9.2f}  {name[:160]}")
    if window and before:
        stop = next((t0 for name, t0, _ in rows if before in name), None)
        sel = [(t1 - t0) / 1e3 for name, t0, t1 in rows
               if (not kernel or kernel in name) and (stop is None or t0 < stop)][-window:]
        if sel:
            out.append(f"last {len(sel)} launches before the first '{before}': mean "
                       f"{statistics.mean(sel):.2f}, median {pct(sel, 0.5):.2f}, p10 "
                       f"{pct(sel, 0.1):.2f}, p90 {pct(sel, 0.9):.2f} us")
    return "\n".join(out)


# Kernels whose HBM traffic is taken from rocprofv3 counters: name ->
# (kernel-name substring, source file, algorithmic bytes read, written).
TRAFFIC = {
    "gemm_w8": ("k_gemm_w8", "gemm_w8.hip",
                2048 * 4096 + 11008 * 4096 + 8 * 11008, 4 * 2048 * 11008),
    "deconv_fixed": ("k_deconv_fixed", "deconv_fixed.hip",
                     8 * 256 * 64 * 64 + 128 * 9 * 256 + 8 * 128, 8 * 128 * 128 * 128),
}
COPY_BYTES = 256 * 1024 * 1024      # the calibration copy reads and writes this much


def summarize_counters(fetch_csv, write_csv, name, command):
    """HBM bytes per call of one kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the 256 MiB calibration copy (k_copy16) of the same
    run.  A call that launches several instantiations of the kernel (the
    GEMM's two tile shapes) counts the median dispatch of each once.  Writes
    profiles/traffic_<name>.json (read by the benchmark while the kernel
    source is unchanged) and returns a text summary."""
    import csv
    sub, src, alg_r, alg_w = TRAFFIC[name]

    def read(path, counter):
        by, copy = {}, []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if sub in r["Kernel_Name"]:
                    by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
                elif "k_copy16" in r["Kernel_Name"]:
                    copy.append(float(r["Counter_Value"]))
        if not by or not copy:
            raise SystemExit(f"{path}: no {counter} rows for {sub} and k_copy16")
        return by, statistics.median(copy)

    fb, fc = read(fetch_csv, "FETCH_SIZE")
    wb, wc = read(write_csv, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / (fc * 1024), COPY_BYTES / (wc * 1024)
    fetch = sum(statistics.median(v) for v in fb.values()) * 1024 * f_scale
    write = sum(statistics.median(v) for v in wb.values()) * 1024 * w_scale
    raw = []
    for label, by in (("FETCH", fb), ("WRITE", wb)):
        for kname, v in sorted(by.items()):
            raw.append(f"#   {label} {min(v):.0f} / {statistics.median(v):.0f} / {max(v):.0f} "
                       f"({len(v)})  {kname[:150]}")
    sha = file_hash(os.path.join(CSRC, src))
    d = {"kernel": sub, "source": src, "source_sha256_16": sha,
         "bytes_per_launch": int(round(fetch + write)), "fetch_bytes": int(round(fetch)),
         "write_bytes": int(round(write)), "fetch_scale": round(f_scale, 4),
         "write_scale": round(w_scale, 4), "algorithmic_read_bytes": alg_r,
         "algorithmic_write_bytes": alg_w, "command": command}
    with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json"), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    return "\n".join([
        f"# HBM traffic per call of {sub} ({src} sha256[:16] = {sha}) on one MI355X",
        f"# commands (one run per counter): {command}",
        f"# reference: 16-byte copy of 256 MiB (reads and writes {COPY_BYTES} B per launch)",
        f"#   FETCH_SIZE reads {fc:.1f} KiB for it -> scale {f_scale:.4f}",
        f"#   WRITE_SIZE reads {wc:.1f} KiB for it -> scale {w_scale:.4f}",
        "# per-dispatch raw values (KiB; min / median / max over the dispatches, per kernel):",
        *raw,
        "",
        f"{'':24}{'measured':>14}{'algorithmic':>14}{'ratio':>8}",
        f"{'read (FETCH_SIZE)':24}{fetch:14.0f}{alg_r:14d}{fetch / alg_r:8.2f}",
        f"{'write (WRITE_SIZE)':24}{write:14.0f}{alg_w:14d}{write / alg_w:8.2f}",
        f"{'total':24}{fetch + write:14.0f}{alg_r + alg_w:14d}"
        f"{(fetch + write) / (alg_r + alg_w):8.2f}"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="fixed untimed phase of back-to-back steps before --warmup (the GPU "
                         "clock settles over the first tens of milliseconds of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--step", choices=["fused", "chain"], default="fused",
                    help="fused: one q8ta_linear_dq call (the dequantize folded into the GEMM "
                         "epilogue); chain: q8ta_linear then q8ta_dequantize_per_tensor")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="target CPU time of one oracle sample run (3 runs, median)")
    ap.add_argument("--profile-only", default=None,
                    choices=["gemm", "gemm-and-copy", "deconv", "deconv-and-copy"],
                    help="for profiler runs: --steps launches of the GEMM step or of the large "
                         "transposed conv (after the settle phase), then with -and-copy the "
                         "256 MiB calibration copy 3 times; print nothing else")
    ap.add_argument("--summarize-trace", default=None,
                    help="print per-kernel duration statistics of a rocprofv3 kernel trace")
    ap.add_argument("--kernel", default=None, help="with --summarize-trace: kernel name filter")
    ap.add_argument("--window", type=int, default=0,
                    help="with --summarize-trace and --before: statistics of the last WINDOW "
                         "matching launches before the first launch matching --before")
    ap.add_argument("--before", default=None)
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    default=None, help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, "
                    "WRITE_SIZE) into profiles/traffic_<--traffic-of>.json")
    ap.add_argument("--traffic-of", choices=sorted(TRAFFIC), default="gemm_w8")
    ap.add_argument("--command", default="", help="with --summarize-counters: the profiling "
                    "command, recorded in the summary")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.kernel, args.window, args.before))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.traffic_of, args.command))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the q8ta path has no multi-GPU form in this "
              "library (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_quantized_amd as q8
    import q8ta_inputs as qi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    lib = q8.lib()
    stream = torch.cuda.current_stream().cuda_stream
    timer = Timer(torch)

    def check(rc):
        if rc != 0:
            raise RuntimeError(q8.q8ta_last_error())

    # ------------------------------------------------------------ headline: GEMM -> dequantize
    c = qi.make_gemm()
    M, K, N = c.M, c.K, c.N
    log(f"workload: q8ta_linear GEMM M={M} K={K} N={N} -> dequantize_per_tensor")
    x = torch.from_numpy(c.x).cuda()
    w = torch.from_numpy(c.w).cuda()
    ws = torch.from_numpy(c.weight_scales).cuda()
    b = torch.from_numpy(c.bias).cuda()
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    none = b"none"

    def gemm():
        check(lib.q8ta_linear(x.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(), N, None,
                              ws.data_ptr(), b.data_ptr(), c.out_scale, c.out_zp, none,
                              out.data_ptr(), stream))

    def deq():
        check(lib.q8ta_dequantize_per_tensor(out.data_ptr(), y.data_ptr(), M * N, c.out_scale,
                                             c.out_zp, stream))

    def gemm_dq():
        check(lib.q8ta_linear_dq(x.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(), N, None,
                                 ws.data_ptr(), b.data_ptr(), c.out_scale, c.out_zp, none,
                                 y.data_ptr(), stream))

    def chain_step():
        gemm()
        deq()

    step = gemm_dq if args.step == "fused" else chain_step

    if args.profile_only in ("deconv", "deconv-and-copy"):
        d = qi.make_deconv_large()
        xf = torch.from_numpy(d.x_fp32).cuda()
        xq = torch.empty(d.x_fp32.shape, dtype=torch.int8, device="cuda")
        check(lib.q8ta_quantize_per_tensor(xf.data_ptr(), xq.data_ptr(), d.x_fp32.size,
                                           d.in_scale, d.in_zp, stream))
        fn, _ = deconv_call(torch, lib, check, stream, d, xq)
        timer.settle([fn], args.settle_ms)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        if args.profile_only == "deconv-and-copy":
            profile_copy(torch, stream)
        log(f"profiled {args.steps} launches of the large transposed conv")
        return
    if args.profile_only in ("gemm", "gemm-and-copy"):
        timer.settle([step], args.settle_ms)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        if args.profile_only == "gemm-and-copy":
            profile_copy(torch, stream)
        log(f"profiled {args.steps} steps ({args.step})")
        return

    # settle the clock (fixed, time-based), then --warmup steps, then the timed steps
    timer.settle([step], args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The fused step is the one GEMM launch: events every `chunk` steps time
    # the launches in batches (an event between every two launches would add
    # a few microseconds of GPU time to each).  The chain step brackets each
    # GEMM launch with its own pair of events.
    chunk = max(1, args.steps // 10)
    if args.step == "fused":
        marks = list(range(0, args.steps, chunk)) + [args.steps]
        bounds = [torch.cuda.Event(enable_timing=True) for _ in marks]
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.step == "fused":
        j = 0
        for i in range(args.steps):
            if i == marks[j]:
                bounds[j].record()
                j += 1
            gemm_dq()
        bounds[j].record()
    else:
        for i in range(args.steps):
            ev[i][0].record()
            gemm()
            ev[i][1].record()
            deq()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    ops = 2.0 * M * N * K
    if args.step == "fused":
        gemm_ms = [bounds[j].elapsed_time(bounds[j + 1]) / (marks[j + 1] - marks[j])
                   for j in range(len(marks) - 1)]
        dist = dist_us(gemm_ms, chunk)
        # the mean over all steps (the last batch may be shorter)
        dist["mean_us"] = round(bounds[0].elapsed_time(bounds[-1]) / args.steps * 1e3, 2)
    else:
        dist = dist_us([a_.elapsed_time(b_) for a_, b_ in ev], 1)
    gemm_avg_s = dist["mean_us"] / 1e6
    achieved = ops / gemm_avg_s / 1e12
    log(f"step {step_s * 1e6:.1f} us; GEMM launches: {dist} = {achieved:.1f} TOPS (mean)")

    # The int8 result (outside the timed region); in the fused form the
    # step's fp32 output must equal dequantize(int8 result).
    gemm()
    torch.cuda.synchronize()
    fused_ok = None
    if args.step == "fused":
        deq_ref = torch.empty_like(y)
        check(lib.q8ta_dequantize_per_tensor(out.data_ptr(), deq_ref.data_ptr(), M * N,
                                             c.out_scale, c.out_zp, stream))
        torch.cuda.synchronize()
        fused_ok = bool(torch.equal(y.view(torch.int32), deq_ref.view(torch.int32)))
        del deq_ref
    gemm_out = out.cpu().numpy()

    roofline = {
        "bound": "mfma",
        "kernel": "k_gemm_w8 (v_mfma_i32_32x32x32_i8; 1 workgroup of 8 waves per CU, slabs "
                  "straight into LDS over 3 stages, mid-step barrier, transposed fp32 stores): "
                  "one launch of 256 tiles of 256x256 (waves of 128x64) for the first 8192 "
                  "columns, then 176 tiles of 256x128 (waves of 64x64) for the last 2816",
        "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_INT8_TOPS, 4),
        "traffic": traffic_from_profile("gemm_w8", os.path.join(CSRC, "gemm_w8.hip")),
        "per_launch_ops": ops, "avg_launch_us": dist["mean_us"],
        "launch_us": dist,
        "algorithmic_bytes_per_launch": int(M * K + N * K + 8 * N + 4 * M * N),
    }

    # ------------------------------------------------------------ the other workloads (GPU)
    extra, captured = {}, {}
    if not args.no_extra:
        extra, captured = run_extra(args, torch, np, q8, qi, lib, stream, timer, check, c, x, w,
                                    ws, b, y, step)
        extra["ceilings"] = run_ceilings(torch, stream, timer, operands=(x, w))
        log(f"  ceilings: {extra['ceilings']}")

    # ------------------------------------------------------------ CPU leg: oracle baseline + checks
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_leg(args, np, qi, c, gemm_out, extra, captured)

    line = {
        "metric": METRIC, "value": round(ops / step_s / 1e12, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "q8ta_linear GEMM M=2048 K=4096 N=11008 -> dequantize_per_tensor",
                   "M": M, "K": K, "N": N, "parallelism": "none (1 GPU)",
                   "settle_ms": args.settle_ms,
                   "step": ("one q8ta_linear_dq call (dequantize folded into the GEMM epilogue; "
                            "output equal to the two-call chain: %s)" % fused_ok)
                   if args.step == "fused" else "q8ta_linear, then q8ta_dequantize_per_tensor"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


def deconv_call(torch, lib, check, stream, d, xin, fused=False):
    """A q8ta_(quantize_)conv2d_transposed call on the workload d with input
    xin (int8, or fp32 for the fused form); returns (fn, out)."""
    N_, IC, H, W = xin.shape
    OC = d.w.shape[0]
    w_ = torch.from_numpy(d.w).cuda()
    s_ = torch.from_numpy(d.weight_scales).cuda()
    b_ = torch.from_numpy(d.bias).cuda()
    out = torch.empty((N_, OC, d.H_out, d.W_out), dtype=torch.int8, device="cuda")
    f = lib.q8ta_quantize_conv2d_transposed if fused else lib.q8ta_conv2d_transposed

    def fn(x_=xin):
        check(f(x_.data_ptr(), N_, IC, H, W, d.in_scale, d.in_zp, w_.data_ptr(), OC, d.Kh, d.Kw,
                d.w.shape[1], None, s_.data_ptr(), b_.data_ptr(), d.out_scale, d.out_zp,
                d.stride[0], d.stride[1], d.padding[0], d.padding[1], d.output_padding[0],
                d.output_padding[1], 1, 1, 1, b"none", out.data_ptr(), d.H_out, d.W_out, stream))
    fn.keep = (w_, s_, b_)
    return fn, out


def summary(ms, work, unit, peak):
    """Per-launch statistics of a timed workload, given (batch means in ms,
    launches per batch); the rate is the work per launch over the mean."""
    d = dist_us(*ms)
    rate = work / (d["mean_us"] / 1e6) / (1e9 if unit == "GB/s" else 1e12)
    d.update({"avg_launch_us": d["mean_us"], "rate": round(rate, 2), "unit": unit})
    if peak:
        d["frac"] = round(rate / peak, 4)
    return d


def run_extra(args, torch, np, q8, qi, lib, stream, timer, check, c, x, w, ws, b, y, step):
    res, cap = {}, {}
    M, K, N = c.M, c.K, c.N
    none = b"none"

    def timed(fns, n):
        timer.settle(fns, 30.0)
        return timer.batches(fns, n), n

    # ---- GEMM step forms: chain, presummed, prepacked, fused quantize chains
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    check(lib.q8ta_weight_sums(w.data_ptr(), N, K, sums.data_ptr(), stream))
    packed = torch.empty(lib.q8ta_weight_prepacked_bytes(N, K), dtype=torch.int8, device="cuda")
    check(lib.q8ta_weight_prepack(w.data_ptr(), N, K, packed.data_ptr(), stream))
    yp = torch.empty_like(y)
    q8out = torch.empty((M, N), dtype=torch.int8, device="cuda")

    def chain():
        check(lib.q8ta_linear(x.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(), N, None,
                              ws.data_ptr(), b.data_ptr(), c.out_scale, c.out_zp, none,
                              q8out.data_ptr(), stream))
        check(lib.q8ta_dequantize_per_tensor(q8out.data_ptr(), yp.data_ptr(), M * N, c.out_scale,
                                             c.out_zp, stream))

    def presummed():
        check(lib.q8ta_linear_dq_presummed(x.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(),
                                           N, sums.data_ptr(), ws.data_ptr(), b.data_ptr(),
                                           c.out_scale, c.out_zp, none, yp.data_ptr(), stream))

    def prepacked():
        check(lib.q8ta_linear_dq_prepacked(x.data_ptr(), M, K, c.in_scale, c.in_zp,
                                           packed.data_ptr(), N, sums.data_ptr(), ws.data_ptr(),
                                           b.data_ptr(), c.out_scale, c.out_zp, none,
                                           yp.data_ptr(), stream))
    step()
    torch.cuda.synchronize()
    for name, fn in (("gemm_step_chain", chain), ("gemm_step_fused", step),
                     ("gemm_step_fused_presummed", presummed),
                     ("gemm_step_fused_prepacked", prepacked)):
        r = summary(timed([fn], 60), 2.0 * M * N * K, "TOPS", PEAK_INT8_TOPS)
        if fn is not step:
            torch.cuda.synchronize()
            r["output_equal_to_fused_step"] = bool(torch.equal(yp.view(torch.int32),
                                                               y.view(torch.int32)))
        res[name] = r
    res["weight_prepack_us"] = dist_us(*timed(
        [lambda: check(lib.q8ta_weight_prepack(w.data_ptr(), N, K, packed.data_ptr(), stream))],
        20))["median_us"]
    res["weight_sums_us"] = dist_us(*timed(
        [lambda: check(lib.q8ta_weight_sums(w.data_ptr(), N, K, sums.data_ptr(), stream))],
        20))["median_us"]
    del packed, yp
    xf32 = torch.from_numpy(qi.x_fp32(qi.rng(2024), (M, K))).cuda()
    yq = torch.empty_like(y)

    def qchain_one_call():
        check(lib.q8ta_quantize_linear_dq(xf32.data_ptr(), M, K, c.in_scale, c.in_zp,
                                          w.data_ptr(), N, None, ws.data_ptr(), b.data_ptr(),
                                          c.out_scale, c.out_zp, none, yq.data_ptr(), stream))
    r = summary(timed([qchain_one_call], 40), 2.0 * M * N * K, "TOPS", PEAK_INT8_TOPS)
    r["note"] = "fp32 [2048,4096] -> quantize -> GEMM -> dequantize in one call"
    res["quantize_gemm_dq_one_call"] = r
    del xf32, yq, q8out
    log(f"  GEMM step forms: " + ", ".join(f"{k} {v['mean_us']} us" for k, v in res.items()
                                           if isinstance(v, dict)))

    # ---- GEMV M=1 K=4096 N=4096, HBM-bound: rotate 32 weight copies (537 MB)
    g = qi.make_gemv()
    log("extra: gemv 1x4096x4096")
    copies = 32
    ws_ = torch.from_numpy(g.weight_scales).cuda()
    b_ = torch.from_numpy(g.bias).cuda()
    x_ = torch.from_numpy(g.x).cuda()
    wl = [torch.from_numpy(g.w).cuda() for _ in range(copies)]
    outs = [torch.empty((1, g.N), dtype=torch.int8, device="cuda") for _ in range(copies)]
    fns = [(lambda i=i: check(lib.q8ta_linear_gemv(
        x_.data_ptr(), 1, g.K, g.in_scale, g.in_zp, wl[i].data_ptr(), g.N, None, ws_.data_ptr(),
        b_.data_ptr(), g.out_scale, g.out_zp, none, outs[i].data_ptr(), stream)))
        for i in range(copies)]
    gemv_bytes = g.N * g.K + g.K + 4 * g.N + 4 * g.N + g.N
    r = summary(timed(fns, 4 * copies), gemv_bytes, "GB/s", PEAK_HBM_GBS)
    r["algorithmic_bytes"] = gemv_bytes
    res["gemv_1x4096x4096_cold"] = r
    res["gemv_1x4096x4096_warm"] = summary(timed([fns[0]], 60), gemv_bytes, "GB/s", PEAK_HBM_GBS)
    torch.cuda.synchronize()
    cap["gemv"] = (g, outs[0].cpu().numpy())
    # fp32 activations: quantize folded into the weight stream
    xf_ = torch.from_numpy(qi.x_fp32(qi.rng(g.K), (1, g.K))).cuda()
    qfns = [(lambda i=i: check(lib.q8ta_quantize_linear(
        xf_.data_ptr(), 1, g.K, g.in_scale, g.in_zp, wl[i].data_ptr(), g.N, None, ws_.data_ptr(),
        b_.data_ptr(), g.out_scale, g.out_zp, none, outs[i].data_ptr(), stream)))
        for i in range(copies)]
    qbytes = g.N * g.K + 4 * g.K + 9 * g.N
    res["quantize_gemv_1x4096x4096_fused_cold"] = summary(timed(qfns, 4 * copies), qbytes, "GB/s",
                                                          PEAK_HBM_GBS)
    torch.cuda.synchronize()
    cap["quantize_gemv"] = (g, xf_.cpu().numpy(), outs[0].cpu().numpy())
    del wl, outs, fns, qfns

    # ---- quantize [8,256,64,64] (rotate 16 copies) and the large transposed conv
    d = qi.make_deconv_large()
    log("extra: quantize [8,256,64,64] + transposed conv -> [8,128,128,128]")
    copies = 16
    numel = d.x_fp32.size
    xs = [torch.from_numpy(d.x_fp32).cuda() for _ in range(copies)]
    qs = [torch.empty(d.x_fp32.shape, dtype=torch.int8, device="cuda") for _ in range(copies)]
    qfns = [(lambda i=i: check(lib.q8ta_quantize_per_tensor(
        xs[i].data_ptr(), qs[i].data_ptr(), numel, d.in_scale, d.in_zp, stream)))
        for i in range(copies)]
    r = summary(timed(qfns, 4 * copies), 5 * numel, "GB/s", PEAK_HBM_GBS)
    r["algorithmic_bytes"] = 5 * numel
    res["quantize_8x256x64x64_cold"] = r
    res["quantize_8x256x64x64_warm"] = summary(timed([qfns[0]], 60), 5 * numel, "GB/s",
                                               PEAK_HBM_GBS)
    torch.cuda.synchronize()
    cap["quantize_large"] = (d, qs[0].cpu().numpy())
    dops = deconv_ops(d)
    dfns = []
    for i in range(copies):
        fn, dout = deconv_call(torch, lib, check, stream, d, qs[i])
        dfns.append(fn)
    r = summary(timed(dfns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = dops
    r["algorithmic_bytes"] = int(numel + d.w.size + 8 * d.w.shape[0] + dout.numel())
    r["kernel"] = ("k_deconv_fixed<3x3 stride 2>: shift-major implicit GEMM on "
                   "v_mfma_i32_32x32x32_i8, two phase rows x 64 columns x 128 channels")
    r["traffic"] = traffic_from_profile("deconv_fixed", os.path.join(CSRC, "deconv_fixed.hip"))
    res["deconv_8x256x64x64_k3s2p1_to_8x128x128x128"] = r
    dfns[-1]()
    torch.cuda.synchronize()
    cap["deconv_large"] = (d, dout.cpu().numpy())
    # the same calls on a prepacked weight (packed once, outside the timed region)
    Nb, ICb, Hb, Wb = d.x_fp32.shape
    OCb = d.w.shape[0]
    wdev = torch.from_numpy(d.w).cuda()
    sdev = torch.from_numpy(d.weight_scales).cuda()
    bdev = torch.from_numpy(d.bias).cuda()
    pk = torch.empty(lib.q8ta_conv2d_transposed_weight_prepacked_bytes(OCb, ICb, d.Kh, d.Kw),
                     dtype=torch.int8, device="cuda")

    def prepack():
        check(lib.q8ta_conv2d_transposed_weight_prepack(wdev.data_ptr(), OCb, ICb, d.Kh, d.Kw,
                                                        d.w.shape[1], pk.data_ptr(), stream))
    prepack()
    pout = torch.empty_like(dout)
    pfns = [(lambda i=i: check(lib.q8ta_conv2d_transposed_prepacked(
        qs[i].data_ptr(), Nb, ICb, Hb, Wb, d.in_scale, d.in_zp, pk.data_ptr(), OCb, d.Kh, d.Kw,
        None, sdev.data_ptr(), bdev.data_ptr(), d.out_scale, d.out_zp, d.stride[0], d.stride[1],
        d.padding[0], d.padding[1], d.output_padding[0], d.output_padding[1], 1, 1, 1, b"none",
        pout.data_ptr(), d.H_out, d.W_out, stream))) for i in range(copies)]
    r = summary(timed(pfns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    r["weight_prepack_us"] = dist_us(*timed([prepack], 20))["median_us"]
    pfns[-1]()
    torch.cuda.synchronize()
    r["output_equal_to_plain_call"] = bool(torch.equal(pout, dout))
    r["note"] = "q8ta_conv2d_transposed_prepacked: weight rearranged once into 1 KiB fragments"
    res["deconv_prepacked_8x256x64x64_k3s2p1_to_8x128x128x128"] = r
    del dfns, qs, pfns
    # quantize -> transposed conv as one call
    ffns = []
    for i in range(copies):
        fn, fout = deconv_call(torch, lib, check, stream, d, xs[i], fused=True)
        ffns.append(fn)
    r = summary(timed(ffns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    r["note"] = "one call: quantize [8,256,64,64] fp32 (cold) + transposed conv"
    res["quantize_deconv_fused_8x256x64x64"] = r
    ffns[0]()
    torch.cuda.synchronize()
    cap["quantize_deconv_large"] = (d, fout.cpu().numpy())
    # the fused form on the prepacked weight
    qpfns = [(lambda i=i: check(lib.q8ta_quantize_conv2d_transposed_prepacked(
        xs[i].data_ptr(), Nb, ICb, Hb, Wb, d.in_scale, d.in_zp, pk.data_ptr(), OCb, d.Kh, d.Kw,
        None, sdev.data_ptr(), bdev.data_ptr(), d.out_scale, d.out_zp, d.stride[0], d.stride[1],
        d.padding[0], d.padding[1], d.output_padding[0], d.output_padding[1], 1, 1, 1, b"none",
        pout.data_ptr(), d.H_out, d.W_out, stream))) for i in range(copies)]
    r = summary(timed(qpfns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    qpfns[0]()
    torch.cuda.synchronize()
    r["output_equal_to_fused_call"] = bool(torch.equal(pout, fout))
    r["note"] = "one call on the prepacked weight: quantize [8,256,64,64] fp32 (cold) + conv"
    res["quantize_deconv_fused_prepacked_8x256x64x64"] = r
    del xs, ffns, qpfns, pk, pout

    # ---- dequantize [2048, 11008] (rotate 6 copies of 22.5 MB in / 90 MB out)
    log("extra: dequantize [2048,11008]")
    n = 2048 * 11008
    copies = 6
    qg = np.random.Generator(np.random.PCG64(77))
    qin_h = qg.integers(-128, 128, size=n, dtype=np.int8)
    qin = [torch.from_numpy(qin_h).cuda() for _ in range(copies)]
    fout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(copies)]
    dqf = [(lambda i=i: check(lib.q8ta_dequantize_per_tensor(
        qin[i].data_ptr(), fout[i].data_ptr(), n, 0.5, -5, stream))) for i in range(copies)]
    r = summary(timed(dqf, 4 * copies), 5 * n, "GB/s", PEAK_HBM_GBS)
    r["algorithmic_bytes"] = 5 * n
    res["dequantize_2048x11008_cold"] = r
    torch.cuda.synchronize()
    cap["dequantize"] = (qin_h, fout[0].cpu().numpy())
    del qin, fout, dqf

    # ---- small, latency-bound workloads
    log("extra: small chain and small transposed conv")
    c1 = qi.make_chain_small()
    xf = torch.from_numpy(c1.x_fp32).cuda()
    xq1 = torch.empty((c1.M, c1.K), dtype=torch.int8, device="cuda")
    w1 = torch.from_numpy(c1.w).cuda()
    s1 = torch.from_numpy(c1.weight_scales).cuda()
    b1 = torch.from_numpy(c1.bias).cuda()
    o1 = torch.empty((c1.M, c1.N), dtype=torch.int8, device="cuda")

    def chain_small():
        check(lib.q8ta_quantize_per_tensor(xf.data_ptr(), xq1.data_ptr(), c1.M * c1.K,
                                           c1.in_scale, c1.in_zp, stream))
        check(lib.q8ta_linear(xq1.data_ptr(), c1.M, c1.K, c1.in_scale, c1.in_zp, w1.data_ptr(),
                              c1.N, None, s1.data_ptr(), b1.data_ptr(), c1.out_scale, c1.out_zp,
                              none, o1.data_ptr(), stream))
    res["chain_quantize_4x64_linear_4x64x32"] = summary(timed([chain_small], 60),
                                                        2 * 4 * 64 * 32, "TOPS", None)
    torch.cuda.synchronize()
    cap["chain_small"] = (c1, o1.cpu().numpy())

    def chain_small_fused():
        check(lib.q8ta_quantize_linear(xf.data_ptr(), c1.M, c1.K, c1.in_scale, c1.in_zp,
                                       w1.data_ptr(), c1.N, None, s1.data_ptr(), b1.data_ptr(),
                                       c1.out_scale, c1.out_zp, none, o1.data_ptr(), stream))
    res["chain_quantize_4x64_linear_4x64x32_one_call"] = summary(
        timed([chain_small_fused], 60), 2 * 4 * 64 * 32, "TOPS", None)
    torch.cuda.synchronize()
    cap["chain_small_fused"] = (c1, o1.cpu().numpy())

    d4 = qi.make_deconv_small()
    fn4, o4 = deconv_call(torch, lib, check, stream, d4, torch.from_numpy(d4.x).cuda())
    r = summary(timed([fn4], 60), deconv_ops(d4), "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = deconv_ops(d4)
    res["deconv_1x64x32x32_k4s2p1_to_1x32x64x64"] = r
    torch.cuda.synchronize()
    cap["deconv_small"] = (d4, o4.cpu().numpy())

    # ---- forward conv [8,256,64,64] K3 s1 p1 -> [8,128,64,64]
    log("extra: conv2d [8,256,64,64] -> [8,128,64,64]")
    cc = qi.make_conv2d_large()
    cx, cw = torch.from_numpy(cc.x).cuda(), torch.from_numpy(cc.w).cuda()
    cs, cb = torch.from_numpy(cc.weight_scales).cuda(), torch.from_numpy(cc.bias).cuda()
    cN, cIC, cH, cW = cc.x.shape
    cOC = cc.w.shape[0]
    cout = torch.empty((cN, cOC, cc.H_out, cc.W_out), dtype=torch.int8, device="cuda")

    def conv():
        check(lib.q8ta_conv2d(
            cx.data_ptr(), cN, cIC, cH, cW, cc.in_scale, cc.in_zp, cw.data_ptr(), cOC, cc.Kh,
            cc.Kw, cc.w.shape[1], None, cs.data_ptr(), cb.data_ptr(), cc.out_scale, cc.out_zp,
            cc.stride[0], cc.stride[1], cc.padding[0], cc.padding[1], cc.dilation[0],
            cc.dilation[1], 1, b"none", cout.data_ptr(), cc.H_out, cc.W_out, stream))
    cops = conv_ops(cc)
    r = summary(timed([conv], 60), cops, "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = cops
    res["conv2d_8x256x64x64_k3s1p1_to_8x128x64x64"] = r
    torch.cuda.synchronize()
    cap["conv2d_large"] = (cc, cout.cpu().numpy())
    del cx, cout

    # ---- depthwise [8,256,64,64] K3 s1 p1, HBM-bound: rotate 40 input copies (335 MB)
    log("extra: depthwise conv [8,256,64,64]")
    dc = qi.make_depthwise_large()
    copies = 40
    dxs = [torch.from_numpy(dc.x).cuda() for _ in range(copies)]
    dw_, ds_, db_ = (torch.from_numpy(a_).cuda() for a_ in (dc.w, dc.weight_scales, dc.bias))
    dN, dC, dH, dW = dc.x.shape
    dout2 = torch.empty((dN, dC, dc.H_out, dc.W_out), dtype=torch.int8, device="cuda")

    def dw_call(i):
        check(lib.q8ta_conv2d(
            dxs[i].data_ptr(), dN, dC, dH, dW, dc.in_scale, dc.in_zp, dw_.data_ptr(), dC, dc.Kh,
            dc.Kw, dc.w.shape[1], None, ds_.data_ptr(), db_.data_ptr(), dc.out_scale, dc.out_zp,
            1, 1, 1, 1, 1, 1, dC, b"none", dout2.data_ptr(), dc.H_out, dc.W_out, stream))
    dwf = [(lambda i=i: dw_call(i)) for i in range(copies)]
    dbytes = int(dc.x.size + dout2.numel() + dc.w.size + 8 * dC)
    r = summary(timed(dwf, 4 * copies), dbytes, "GB/s", PEAK_HBM_GBS)
    r["algorithmic_bytes"] = dbytes
    res["depthwise_8x256x64x64_k3s1p1_cold"] = r
    torch.cuda.synchronize()
    cap["depthwise_large"] = (dc, dout2.cpu().numpy())
    del dxs, dout2
    for k_, v_ in res.items():
        log(f"  {k_}: {v_}")
    return res, cap


def cpu_leg(args, np, qi, c, gemm_out, extra, cap):
    """The CPU leg: the oracle timed on a sample of the GEMM workload (median
    of 3 runs on the host cores) for cpu_baseline, and every output captured
    by the GPU phase compared with the oracle over all of its elements."""
    import oracle
    M, K, N = c.M, c.K, c.N
    t = time.perf_counter()
    probe = oracle.linear(c.x[:8], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                          c.out_scale, c.out_zp)
    rate = 8 / (time.perf_counter() - t)           # rows per second
    rows = int(max(8, min(M, round(rate * args.cpu_seconds))))
    times = []
    for _ in range(3):
        t = time.perf_counter()
        ref = oracle.linear(c.x[:rows], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                            c.out_scale, c.out_zp)
        times.append(time.perf_counter() - t)
    dt = statistics.median(times)
    full = ref if rows == M else oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale,
                                               c.in_zp, c.out_scale, c.out_zp)
    cpu = {"value": round(2.0 * rows * N * K / dt / 1e12, 5), "unit": "TOPS",
           "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of the {M}x{K} activations against all {N} weight rows "
                     f"(contraction + epilogue), median of 3 runs: {dt:.2f} s",
           "sample_bitexact_vs_gpu": bool(np.array_equal(gemm_out[:rows], ref) and
                                         np.array_equal(gemm_out[:8], probe)),
           "full_output_bitexact_vs_gpu": bool(np.array_equal(gemm_out, full))}
    log(f"cpu oracle: {cpu}")
    if not cap:
        return cpu

    def mark(key, ok):
        if key in extra and isinstance(extra[key], dict):
            extra[key]["oracle_bitexact"] = bool(ok)

    g, got = cap["gemv"]
    mark("gemv_1x4096x4096_cold", np.array_equal(got, oracle.linear(
        g.x, g.w, g.weight_scales, g.bias, g.in_scale, g.in_zp, g.out_scale, g.out_zp)))
    g, xf, got = cap["quantize_gemv"]
    xq = oracle.quantize_per_tensor(xf, g.in_scale, g.in_zp)
    mark("quantize_gemv_1x4096x4096_fused_cold", np.array_equal(got, oracle.linear(
        xq, g.w, g.weight_scales, g.bias, g.in_scale, g.in_zp, g.out_scale, g.out_zp)))
    d, got = cap["quantize_large"]
    xq = oracle.quantize_per_tensor(d.x_fp32, d.in_scale, d.in_zp)
    mark("quantize_8x256x64x64_cold", np.array_equal(got, xq))
    dref = oracle.conv2d_transposed(xq, d.w, d.weight_scales, d.bias, d.in_scale, d.in_zp,
                                    d.out_scale, d.out_zp, d.Kh, d.Kw, d.stride, d.padding, (1, 1),
                                    d.H_out, d.W_out)
    mark("deconv_8x256x64x64_k3s2p1_to_8x128x128x128",
         np.array_equal(cap["deconv_large"][1], dref))
    mark("quantize_deconv_fused_8x256x64x64",
         np.array_equal(cap["quantize_deconv_large"][1], dref))
    qin, got = cap["dequantize"]
    mark("dequantize_2048x11008_cold", np.array_equal(
        got.view(np.uint32), oracle.dequantize_per_tensor(qin, 0.5, -5).view(np.uint32)))
    c1, got = cap["chain_small"]
    xq = oracle.quantize_per_tensor(c1.x_fp32, c1.in_scale, c1.in_zp)
    cref = oracle.linear(xq, c1.w, c1.weight_scales, c1.bias, c1.in_scale, c1.in_zp, c1.out_scale,
                         c1.out_zp)
    mark("chain_quantize_4x64_linear_4x64x32", np.array_equal(got, cref))
    mark("chain_quantize_4x64_linear_4x64x32_one_call",
         np.array_equal(cap["chain_small_fused"][1], cref))
    d4, got = cap["deconv_small"]
    mark("deconv_1x64x32x32_k4s2p1_to_1x32x64x64", np.array_equal(got, oracle.conv2d_transposed(
        d4.x, d4.w, d4.weight_scales, d4.bias, d4.in_scale, d4.in_zp, d4.out_scale, d4.out_zp,
        d4.Kh, d4.Kw, d4.stride, d4.padding, (1, 1), d4.H_out, d4.W_out)))
    cc, got = cap["conv2d_large"]
    mark("conv2d_8x256x64x64_k3s1p1_to_8x128x64x64", np.array_equal(got, oracle.conv2d(
        cc.x, cc.w, cc.weight_scales, cc.bias, cc.in_scale, cc.in_zp, cc.out_scale, cc.out_zp,
        cc.Kh, cc.Kw, cc.stride, cc.padding, cc.dilation, cc.H_out, cc.W_out)))
    dc, got = cap["depthwise_large"]
    mark("depthwise_8x256x64x64_k3s1p1_cold", np.array_equal(got, oracle.conv2d(
        dc.x, dc.w, dc.weight_scales, dc.bias, dc.in_scale, dc.in_zp, dc.out_scale, dc.out_zp,
        dc.Kh, dc.Kw, dc.stride, dc.padding, dc.dilation, dc.H_out, dc.W_out,
        groups=dc.x.shape[1])))
    # the GEMM step forms were compared with the fused step on the GPU; the
    # fused step's int8 result is the one compared in full above
    checked = [k_ for k_, v_ in extra.items() if isinstance(v_, dict) and "oracle_bitexact" in v_]
    cpu["extra_outputs_checked"] = len(checked)
    cpu["extra_outputs_bitexact"] = all(extra[k_]["oracle_bitexact"] for k_ in checked)
    log(f"oracle checks: {[(k_, extra[k_]['oracle_bitexact']) for k_ in checked]}")
    return cpu


def profile_copy(torch, stream):
    """Three launches of the 16-byte calibration copy over 256 MiB (reads and
    writes 268,435,456 bytes each): the reference for scaling HBM counters."""
    cl = ctypes.CDLL(os.path.join(ROOT, "int8_quantized_amd", "libq8ta_calib.so"))
    cl.q8ta_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        cl.q8ta_calib_copy(src.data_ptr(), dst.data_ptr(), n // 16, 256 * 8, stream)
    torch.cuda.synchronize()


def run_ceilings(torch, stream, timer, operands=None):
    """Achieved ceilings on this GPU (libq8ta_calib.so), next to the published
    peaks: a plain 16-byte copy, a read-only stream of the GEMV's weight size
    from HBM, an empty launch of the GEMV's grid, and register-only loops of
    independent int8 MFMAs -- on near-constant operands, and (`operands`: the
    GEMM's activations and weights) on operands taken from the GEMM's own
    data, which the matrix cores run markedly slower."""
    path = os.path.join(ROOT, "int8_quantized_amd", "libq8ta_calib.so")
    if not os.path.exists(path):
        return None
    cl = ctypes.CDLL(path)
    cl.q8ta_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    cl.q8ta_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p]
    cl.q8ta_calib_empty.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    cl.q8ta_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    cl.q8ta_calib_mfma_data.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    out = torch.empty(512 * 256, dtype=torch.int32, device="cuda")

    def run(fns, n):
        timer.settle(fns, 20.0)
        return dist_us(timer.batches(fns, n), n)

    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    cp = run([lambda: cl.q8ta_calib_copy(src.data_ptr(), dst.data_ptr(), n // 16, 256 * 8,
                                         stream)], 10)
    del src, dst
    # 32 rotating buffers (537 MB) so that every launch reads from HBM
    nr = 4096 * 4096
    bufs = [torch.empty(nr, dtype=torch.uint8, device="cuda") for _ in range(32)]
    rd = run([lambda b=b: cl.q8ta_calib_read(b.data_ptr(), nr // 16, out.data_ptr(), stream)
              for b in bufs], 128)
    del bufs
    em = run([lambda: cl.q8ta_calib_empty(out.data_ptr(), 512, stream)], 200)
    mfma = {}
    for kind, name, per in ((0, "mfma_16x16x64_i8_loop_tops", 16 * 32768),
                            (1, "mfma_32x32x32_i8_loop_tops", 8 * 65536)):
        mb, mi = 512, 2000
        d = run([lambda k=kind: cl.q8ta_calib_mfma(out.data_ptr(), mb, mi, k, stream)], 5)
        mfma[name] = round(mb * 4 * mi * per / (d["median_us"] / 1e6) / 1e12, 1)
    if operands is not None:
        xa, wb = operands
        mb, mi = 512, 2000
        d = run([lambda: cl.q8ta_calib_mfma_data(xa.data_ptr(), xa.numel() // 16, wb.data_ptr(),
                                                 wb.numel() // 16, out.data_ptr(), mb, mi,
                                                 stream)], 5)
        mfma["mfma_32x32x32_i8_loop_tops_on_gemm_operands"] = round(
            mb * 4 * mi * 8 * 65536 / (d["median_us"] / 1e6) / 1e12, 1)
    return {**mfma, "int8_mfma_peak_tops": PEAK_INT8_TOPS,
            "copy_256MiB_gbs": round(2 * n / (cp["median_us"] / 1e6) / 1e9, 1),
            "hbm_peak_gbs": PEAK_HBM_GBS,
            "read_16MiB_cold_us": rd["median_us"],
            "read_16MiB_cold_gbs": round(nr / (rd["median_us"] / 1e6) / 1e9, 1),
            "empty_launch_us": em["median_us"]}


if __name__ == "__main__":
    main()
