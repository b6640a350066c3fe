#!/usr/bin/env python3
"""Benchmark of the q8ta int8 path on one MI355X.

A step is one pass of the measured workload over resident synthetic inputs.
The default workload is the large linear:
    q8ta_linear GEMM  M=2048 K=4096 N=11008  (int8 x int8 -> int32 -> int8)
    -> dequantize_per_tensor of the int8 output to fp32
`value` is 2*M*N*K int8 operations per step divided by the step time (TOPS).

The JSON line also carries
  roofline      the GEMM call's own rate (HIP events around each call in the
                timed region, on the stream it runs on) against the v_dot4
                vector-ALU peak it is bound by (and, beside it, the fraction
                of the dense int8 MFMA peak);
  cpu_baseline  the CPU oracle timed on a sample of the same workload
                (a block of rows; the GPU's rows are compared with it);
  extra         the other workloads of the op family, each timed with events:
                GEMV, quantize, dequantize and the two transposed convolutions;
                HBM-bound kernels rotate through enough buffer copies to
                exceed the 256 MB last-level cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                       [--profile-only gemm-and-copy|deconv]
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
# Vector-ALU int8 peak: 256 CUs x 2.4 GHz x 64 lanes/clk x 4 MACs (v_dot4) x 2 ops.
PEAK_DOT4_TOPS = 256 * 2.4e9 * 64 * 4 * 2 / 1e12


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
    WRITE_SIZE, scaled by a copy kernel of known size) and stored beside the
    profiles; only used while the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != file_hash(src):
        return None
    return d.get("bytes_per_launch")


class Timer:
    """HIP events on torch's current stream (the stream libq8ta launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def time_calls(self, fns, reps, budget_s=4.0, batches=5):
        """Average duration (ms) of back-to-back launches, cycling through
        `fns`: each of `batches` batches of `reps` launches is bracketed by two
        events; fewer launches when one call is slow, to stay within about
        `budget_s` seconds.  Returns the per-launch average of every batch."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fns[0]()
        e1.record()
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1) / 1e3, 1e-6)
        reps = int(max(1, min(reps, budget_s / batches / one)))
        out = []
        for _ in range(batches):
            e0.record()
            for i in range(reps):
                fns[i % len(fns)]()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / reps)
        return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first: the GPU clock settles over the first ~50 ms of "
                         "back-to-back GEMMs (50 steps measured ~12%% slower than 500)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--step", choices=["fused", "chain"], default="fused",
                    help="fused: one q8ta_linear_dq call (the dequantize folded into the GEMM "
                         "epilogue); chain: q8ta_linear then q8ta_dequantize_per_tensor")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--profile-only", choices=["gemm-and-copy", "deconv"], default=None,
                    help="for hardware-counter runs: run `--steps` steps of the GEMM workload "
                         "and the 256 MiB calibration copy 3 times (gemm-and-copy), or the "
                         "large transposed conv `--steps` times (deconv); print nothing else")
    args = ap.parse_args()

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

    # A step is the whole workload, q8ta_linear -> dequantize_per_tensor; `call`
    # is the GEMM call the roofline times (the fused call is the whole step).
    if args.step == "fused":
        call, rest = gemm_dq, (lambda: None)
    else:
        call, rest = gemm, deq

    if args.profile_only == "deconv":
        d = qi.make_deconv_large()
        xq = torch.empty(d.x_fp32.shape, dtype=torch.int8, device="cuda")
        check(lib.q8ta_quantize_per_tensor(torch.from_numpy(d.x_fp32).cuda().data_ptr(),
                                           xq.data_ptr(), d.x_fp32.size, d.in_scale, d.in_zp,
                                           stream))
        w_ = torch.from_numpy(d.w).cuda()
        dws = torch.from_numpy(d.weight_scales).cuda()
        db = torch.from_numpy(d.bias).cuda()
        N_, IC, H, W = d.x_fp32.shape
        dout = torch.empty((N_, d.w.shape[0], d.H_out, d.W_out), dtype=torch.int8, device="cuda")
        for _ in range(args.steps):
            check(lib.q8ta_conv2d_transposed(
                xq.data_ptr(), N_, IC, H, W, d.in_scale, d.in_zp, w_.data_ptr(), d.w.shape[0],
                d.Kh, d.Kw, d.w.shape[1], None, dws.data_ptr(), db.data_ptr(), d.out_scale,
                d.out_zp, d.stride[0], d.stride[1], d.padding[0], d.padding[1],
                d.output_padding[0], d.output_padding[1], 1, 1, 1, b"none", dout.data_ptr(),
                d.H_out, d.W_out, stream))
        torch.cuda.synchronize()
        log(f"profiled {args.steps} launches of the large transposed conv")
        return

    if args.profile_only == "gemm-and-copy":
        for _ in range(args.steps):
            call()
            rest()
        torch.cuda.synchronize()
        profile_copy(torch, stream)
        log(f"profiled {args.steps} steps ({args.step}) and 3 copies of 256 MiB")
        return

    for _ in range(args.warmup):
        call()
        rest()
    torch.cuda.synchronize()
    # The fused step is the one GEMM launch: an event at every step boundary
    # times each launch (kernel plus the gap to the next) without a second
    # marker per step.  The chain step brackets the GEMM with its own pair.
    if args.step == "fused":
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.step == "fused":
        bounds[0].record()
        for i in range(args.steps):
            call()
            bounds[i + 1].record()
    else:
        for i in range(args.steps):
            ev[i][0].record()
            call()
            ev[i][1].record()
            rest()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    ops = 2.0 * M * N * K
    if args.step == "fused":
        gemm_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]
    else:
        gemm_ms = [a.elapsed_time(bb) for a, bb in ev]
    gemm_avg_s = statistics.mean(gemm_ms) / 1e3
    achieved = ops / gemm_avg_s / 1e12
    log(f"step {step_s * 1e6:.1f} us; GEMM avg {gemm_avg_s * 1e6:.1f} us "
        f"(min {min(gemm_ms) * 1e3:.1f}) = {achieved:.1f} TOPS")

    # The int8 result for the checks below (outside the timed region); in the
    # fused form the step's fp32 output must equal dequantize(int8 result).
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

    roofline = {
        "bound": "mfma",
        "kernel": "k_gemm_mx<256x128x64 tile, 2x2 waves of 128x64, 2 workgroups/CU, "
                  "store-first K loop, transposed fp32 stores> (v_mfma_i32_32x32x32_i8)",
        "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_INT8_TOPS, 4),
        "traffic": traffic_from_profile("gemm_mx", os.path.join(
            ROOT, "int8_quantized_amd", "csrc", "gemm_mx.hip")),
    }
    roofline.update({"per_launch_ops": ops, "avg_launch_us": round(gemm_avg_s * 1e6, 2)})

    # ------------------------------------------------------------ CPU baseline (oracle sample)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        got = out.cpu().numpy()
        t = time.perf_counter()
        probe = oracle.linear(c.x[:8], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                              c.out_scale, c.out_zp)
        rate = 8 / (time.perf_counter() - t)           # rows per second
        rows = int(max(8, min(M, round(rate * args.cpu_seconds))))
        t = time.perf_counter()
        ref = oracle.linear(c.x[:rows], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                            c.out_scale, c.out_zp)
        dt = time.perf_counter() - t
        cpu = {"value": round(2.0 * rows * N * K / dt / 1e12, 5), "unit": "TOPS",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"rows 0..{rows - 1} of the {M}x{K} activations against all {N} weight "
                         f"rows (contraction + epilogue), {dt:.1f} s",
               "sample_bitexact_vs_gpu": bool(np.array_equal(got[:rows], ref) and
                                             np.array_equal(got[:8], probe))}
        log(f"cpu oracle: {cpu}")

    # ------------------------------------------------------------ the other workloads
    extra = {}
    if not args.no_extra:
        def chain():
            gemm()
            deq()
        sums = torch.empty(N, dtype=torch.int32, device="cuda")
        check(lib.q8ta_weight_sums(w.data_ptr(), N, K, sums.data_ptr(), stream))

        def gemm_dq_presummed():
            check(lib.q8ta_linear_dq_presummed(x.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(),
                                               N, sums.data_ptr(), ws.data_ptr(), b.data_ptr(),
                                               c.out_scale, c.out_zp, none, y.data_ptr(), stream))
        packed = torch.empty(lib.q8ta_weight_prepacked_bytes(N, K), dtype=torch.int8, device="cuda")
        check(lib.q8ta_weight_prepack(w.data_ptr(), N, K, packed.data_ptr(), stream))
        yp = torch.empty_like(y)

        def gemm_dq_prepacked():
            check(lib.q8ta_linear_dq_prepacked(x.data_ptr(), M, K, c.in_scale, c.in_zp,
                                               packed.data_ptr(), N, sums.data_ptr(), ws.data_ptr(),
                                               b.data_ptr(), c.out_scale, c.out_zp, none,
                                               yp.data_ptr(), stream))
        gemm_dq_prepacked()
        gemm_dq()
        torch.cuda.synchronize()
        extra["prepacked_output_equal"] = bool(torch.equal(yp.view(torch.int32),
                                                           y.view(torch.int32)))
        # the CPU leg leaves the GPU idle and its clock low: warm it again
        timer.time_calls([gemm_dq], args.warmup, budget_s=0.2, batches=1)
        for name, fn in (("gemm_step_chain_us", chain), ("gemm_step_fused_us", gemm_dq),
                         ("gemm_step_fused_presummed_us", gemm_dq_presummed),
                         ("gemm_step_fused_prepacked_us", gemm_dq_prepacked)):
            extra[name] = round(min(timer.time_calls([fn], 50, batches=3)) * 1e3, 1)
        extra["gemm_prepacked_tops"] = round(2.0 * M * N * K / extra["gemm_step_fused_prepacked_us"]
                                             / 1e6, 1)
        extra["weight_prepack_us"] = round(min(timer.time_calls(
            [lambda: check(lib.q8ta_weight_prepack(w.data_ptr(), N, K, packed.data_ptr(), stream))],
            20, batches=3)) * 1e3, 1)
        del yp
        # fp32 activations in, fp32 out: the whole quantize -> linear -> dequantize
        # chain in one call (its quantize goes through the library's workspace at
        # this M) against the three separate calls
        xf32 = torch.from_numpy(qi.x_fp32(qi.rng(2024), (M, K))).cuda()
        xq32 = torch.empty((M, K), dtype=torch.int8, device="cuda")
        yq = torch.empty_like(y)

        def qchain_one_call():
            check(lib.q8ta_quantize_linear_dq(xf32.data_ptr(), M, K, c.in_scale, c.in_zp,
                                              w.data_ptr(), N, None, ws.data_ptr(), b.data_ptr(),
                                              c.out_scale, c.out_zp, none, yq.data_ptr(), stream))

        def qchain_three_calls():
            check(lib.q8ta_quantize_per_tensor(xf32.data_ptr(), xq32.data_ptr(), M * K,
                                               c.in_scale, c.in_zp, stream))
            check(lib.q8ta_linear(xq32.data_ptr(), M, K, c.in_scale, c.in_zp, w.data_ptr(), N,
                                  None, ws.data_ptr(), b.data_ptr(), c.out_scale, c.out_zp, none,
                                  q8out.data_ptr(), stream))
            check(lib.q8ta_dequantize_per_tensor(q8out.data_ptr(), y.data_ptr(), M * N,
                                                 c.out_scale, c.out_zp, stream))
        q8out = torch.empty((M, N), dtype=torch.int8, device="cuda")
        qchain_one_call()
        qchain_three_calls()
        torch.cuda.synchronize()
        extra["quantize_gemm_dq_output_equal"] = bool(torch.equal(yq.view(torch.int32),
                                                                  y.view(torch.int32)))
        for name, fn in (("quantize_gemm_dq_one_call_us", qchain_one_call),
                         ("quantize_gemm_dq_three_calls_us", qchain_three_calls)):
            extra[name] = round(min(timer.time_calls([fn], 50, batches=3)) * 1e3, 1)
        del xf32, xq32, yq, q8out
        extra["weight_sums_us"] = round(min(timer.time_calls(
            [lambda: check(lib.q8ta_weight_sums(w.data_ptr(), N, K, sums.data_ptr(), stream))], 20,
            batches=3)) * 1e3, 1)
        log(f"  step forms: chain {extra['gemm_step_chain_us']} us, "
            f"fused {extra['gemm_step_fused_us']} us, fused with precomputed weight sums "
            f"{extra['gemm_step_fused_presummed_us']} us (+ {extra['weight_sums_us']} us once per weight), "
            f"prepacked weight {extra['gemm_step_fused_prepacked_us']} us (+ {extra['weight_prepack_us']} us "
            f"once per weight; output equal: {extra['prepacked_output_equal']})")
        extra.update(run_extra(torch, np, q8, qi, lib, stream, timer, check))
        extra["ceilings"] = run_ceilings(torch, stream, timer)
        log(f"  ceilings: {extra['ceilings']}")

    line = {
        "metric": METRIC, "value": round(ops / step_s / 1e12, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "q8ta_linear GEMM M=2048 K=4096 N=11008 -> dequantize_per_tensor",
                   "M": M, "K": K, "N": N, "parallelism": "none (1 GPU)",
                   "step": ("one q8ta_linear_dq call (dequantize folded into the GEMM epilogue; "
                            "output equal to the two-call chain: %s)" % fused_ok)
                   if args.step == "fused" else "q8ta_linear, then q8ta_dequantize_per_tensor"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


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


def run_ceilings(torch, stream, timer):
    """Achieved ceilings on this GPU: a register-only v_dot4 loop and a plain
    16-byte copy (libq8ta_calib.so), next to the published peaks."""
    path = os.path.join(ROOT, "int8_quantized_amd", "libq8ta_calib.so")
    if not os.path.exists(path):
        return None
    cl = ctypes.CDLL(path)
    cl.q8ta_calib_dot4.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cl.q8ta_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    blocks, iters = 256 * 16, 1024
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    ms = timer.time_calls([lambda: cl.q8ta_calib_dot4(out.data_ptr(), blocks, iters, stream)], 3,
                          batches=3)
    dot4_tops = blocks * 256 * iters * 16 * 8 / (min(ms) / 1e3) / 1e12
    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    ms = timer.time_calls([lambda: cl.q8ta_calib_copy(src.data_ptr(), dst.data_ptr(), n // 16,
                                                      256 * 8, stream)], 10, batches=3)
    copy_gbs = 2 * n / (min(ms) / 1e3) / 1e9
    del src, dst
    # read-only stream of the GEMV's weight size, 32 rotating copies (537 MB) so
    # that every launch reads from HBM; and an empty launch of the GEMV's grid
    cl.q8ta_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    cl.q8ta_calib_empty.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    nr = 4096 * 4096
    bufs = [torch.empty(nr, dtype=torch.uint8, device="cuda") for _ in range(32)]
    ms = timer.time_calls([lambda b=b: cl.q8ta_calib_read(b.data_ptr(), nr // 16, out.data_ptr(),
                                                          stream) for b in bufs], 128, batches=3)
    read_us = min(ms) * 1e3
    del bufs
    ms = timer.time_calls([lambda: cl.q8ta_calib_empty(out.data_ptr(), 512, stream)], 200,
                          batches=3)
    empty_us = min(ms) * 1e3
    # register-only loops of independent int8 MFMAs, one wave per SIMD (512
    # workgroups of 4 waves): the matrix cores' issue ceiling per instruction
    cl.q8ta_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    mfma = {}
    for kind, name, per in ((0, "mfma_16x16x64_i8_loop_tops", 16 * 32768),
                            (1, "mfma_32x32x32_i8_loop_tops", 8 * 65536)):
        mb, mi = 512, 2000
        ms = timer.time_calls([lambda k=kind: cl.q8ta_calib_mfma(out.data_ptr(), mb, mi, k, stream)],
                              3, batches=3)
        mfma[name] = round(mb * 4 * mi * per / (min(ms) / 1e3) / 1e12, 1)
    return {"dot4_loop_tops": round(dot4_tops, 1), "dot4_peak_tops_derived": round(PEAK_DOT4_TOPS, 1),
            **mfma, "int8_mfma_peak_tops": PEAK_INT8_TOPS,
            "copy_256MiB_gbs": round(copy_gbs, 1), "hbm_peak_gbs": PEAK_HBM_GBS,
            "read_16MiB_cold_us": round(read_us, 2),
            "read_16MiB_cold_gbs": round(nr / (read_us / 1e6) / 1e9, 1),
            "empty_launch_us": round(empty_us, 2)}


def run_extra(torch, np, q8, qi, lib, stream, timer, check):
    res = {}
    reps = 60

    def summary(ms, work, unit, peak):
        med = statistics.median(ms) / 1e3
        rate = work / med / (1e9 if unit == "GB/s" else 1e12)
        d = {"avg_launch_us": round(med * 1e6, 2), "best_batch_us": round(min(ms) * 1e3, 2),
             "rate": round(rate, 2), "unit": unit}
        if peak:
            d["frac"] = round(rate / peak, 4)
        return d

    # ---- GEMV M=1 K=4096 N=4096, HBM-bound: rotate 32 weight copies (537 MB)
    c = qi.make_gemv()
    log("extra: gemv 1x4096x4096")
    copies = 32
    ws_ = torch.from_numpy(c.weight_scales).cuda()
    b_ = torch.from_numpy(c.bias).cuda()
    x_ = torch.from_numpy(c.x).cuda()
    wl = [torch.from_numpy(c.w).cuda() for _ in range(copies)]
    outs = [torch.empty((1, c.N), dtype=torch.int8, device="cuda") for _ in range(copies)]
    fns = [(lambda i=i: check(lib.q8ta_linear_gemv(
        x_.data_ptr(), 1, c.K, c.in_scale, c.in_zp, wl[i].data_ptr(), c.N, None, ws_.data_ptr(),
        b_.data_ptr(), c.out_scale, c.out_zp, b"none", outs[i].data_ptr(), stream)))
        for i in range(copies)]
    gemv_bytes = c.N * c.K + c.K + 4 * c.N + 4 * c.N + c.N
    timer.time_calls(fns, copies)
    res["gemv_1x4096x4096_cold"] = summary(timer.time_calls(fns, 4 * copies), gemv_bytes, "GB/s",
                                           PEAK_HBM_GBS)
    res["gemv_1x4096x4096_warm"] = summary(timer.time_calls([fns[0]], reps), gemv_bytes, "GB/s",
                                           PEAK_HBM_GBS)
    res["gemv_1x4096x4096_cold"]["algorithmic_bytes"] = gemv_bytes
    # fp32 activations: quantize folded into the weight-streaming kernel
    # against the two calls (quantize_per_tensor, then the int8 GEMV)
    xf_ = torch.from_numpy(qi.x_fp32(qi.rng(c.K), (1, c.K))).cuda()
    xq_ = torch.empty((1, c.K), dtype=torch.int8, device="cuda")
    qfns = [(lambda i=i: check(lib.q8ta_quantize_linear(
        xf_.data_ptr(), 1, c.K, c.in_scale, c.in_zp, wl[i].data_ptr(), c.N, None,
        ws_.data_ptr(), b_.data_ptr(), c.out_scale, c.out_zp, b"none", outs[i].data_ptr(),
        stream))) for i in range(copies)]

    def _chain(i):
        check(lib.q8ta_quantize_per_tensor(xf_.data_ptr(), xq_.data_ptr(), c.K, c.in_scale,
                                           c.in_zp, stream))
        check(lib.q8ta_linear_gemv(xq_.data_ptr(), 1, c.K, c.in_scale, c.in_zp, wl[i].data_ptr(),
                                   c.N, None, ws_.data_ptr(), b_.data_ptr(), c.out_scale, c.out_zp,
                                   b"none", outs[i].data_ptr(), stream))
    cfns = [(lambda i=i: _chain(i)) for i in range(copies)]
    qgemv_bytes = c.N * c.K + 4 * c.K + 4 * c.N + 4 * c.N + c.N
    timer.time_calls(qfns, copies)
    res["quantize_gemv_1x4096x4096_fused_cold"] = summary(
        timer.time_calls(qfns, 4 * copies), qgemv_bytes, "GB/s", PEAK_HBM_GBS)
    timer.time_calls(cfns, copies)
    res["quantize_gemv_1x4096x4096_two_calls_cold"] = summary(
        timer.time_calls(cfns, 4 * copies), qgemv_bytes, "GB/s", PEAK_HBM_GBS)
    qfns[0]()
    fused_q = outs[0].clone()
    cfns[0]()
    torch.cuda.synchronize()
    res["quantize_gemv_1x4096x4096_fused_cold"]["output_equal_to_two_calls"] = bool(
        torch.equal(fused_q, outs[0]))
    del wl, outs, fns, qfns, cfns

    # ---- quantize [8,256,64,64] (rotate 16 copies) and the large transposed conv
    d = qi.make_deconv_large()
    log("extra: quantize [8,256,64,64] + deconv -> [8,128,128,128]")
    copies = 16
    numel = d.x_fp32.size
    xs = [torch.from_numpy(d.x_fp32).cuda() for _ in range(copies)]
    qs = [torch.empty(d.x_fp32.shape, dtype=torch.int8, device="cuda") for _ in range(copies)]
    qfns = [(lambda i=i: check(lib.q8ta_quantize_per_tensor(
        xs[i].data_ptr(), qs[i].data_ptr(), numel, d.in_scale, d.in_zp, stream)))
        for i in range(copies)]
    timer.time_calls(qfns, copies)
    res["quantize_8x256x64x64_cold"] = summary(timer.time_calls(qfns, 4 * copies), 5 * numel,
                                               "GB/s", PEAK_HBM_GBS)
    res["quantize_8x256x64x64_warm"] = summary(timer.time_calls([qfns[0]], reps), 5 * numel,
                                               "GB/s", PEAK_HBM_GBS)
    xq = qs[0]
    del xs, qfns
    w_ = torch.from_numpy(d.w).cuda()
    dws = torch.from_numpy(d.weight_scales).cuda()
    db = torch.from_numpy(d.bias).cuda()
    N_, IC, H, W = d.x_fp32.shape
    OC = d.w.shape[0]
    dout = torch.empty((N_, OC, d.H_out, d.W_out), dtype=torch.int8, device="cuda")

    def dc_large(xq=xq):
        check(lib.q8ta_conv2d_transposed(
            xq.data_ptr(), N_, IC, H, W, d.in_scale, d.in_zp, w_.data_ptr(), OC, d.Kh, d.Kw,
            d.w.shape[1], None, dws.data_ptr(), db.data_ptr(), d.out_scale, d.out_zp,
            d.stride[0], d.stride[1], d.padding[0], d.padding[1], d.output_padding[0],
            d.output_padding[1], 1, 1, 1, b"none", dout.data_ptr(), d.H_out, d.W_out, stream))
    dops = deconv_ops(d)
    dfns = [(lambda i=i: dc_large(qs[i])) for i in range(copies)]
    timer.time_calls(dfns, copies)
    r = summary(timer.time_calls(dfns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = dops
    r["algorithmic_bytes"] = int(numel + d.w.size + 8 * OC + dout.numel())
    res["deconv_8x256x64x64_k3s2p1_to_8x128x128x128"] = r
    del qs, dfns

    # quantize -> transposed conv as one call (quantize folded into the input copy)
    xs = [torch.from_numpy(d.x_fp32).cuda() for _ in range(copies)]

    def qdc(xf):
        check(lib.q8ta_quantize_conv2d_transposed(
            xf.data_ptr(), N_, IC, H, W, d.in_scale, d.in_zp, w_.data_ptr(), OC, d.Kh, d.Kw,
            d.w.shape[1], None, dws.data_ptr(), db.data_ptr(), d.out_scale, d.out_zp,
            d.stride[0], d.stride[1], d.padding[0], d.padding[1], d.output_padding[0],
            d.output_padding[1], 1, 1, 1, b"none", dout.data_ptr(), d.H_out, d.W_out, stream))
    qfns = [(lambda i=i: qdc(xs[i])) for i in range(copies)]
    timer.time_calls(qfns, copies)
    r = summary(timer.time_calls(qfns, 4 * copies), dops, "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = dops
    r["note"] = "one call: quantize [8,256,64,64] fp32 (cold) + transposed conv"
    res["quantize_deconv_fused_8x256x64x64"] = r
    del xs, qfns

    # ---- dequantize [2048, 11008] (rotate 8 copies of 22.5 MB in / 90 MB out)
    log("extra: dequantize [2048,11008]")
    n = 2048 * 11008
    copies = 6
    qin = [torch.randint(-128, 128, (n,), dtype=torch.int8, device="cuda") for _ in range(copies)]
    fout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(copies)]
    dqf = [(lambda i=i: check(lib.q8ta_dequantize_per_tensor(
        qin[i].data_ptr(), fout[i].data_ptr(), n, 0.5, -5, stream))) for i in range(copies)]
    timer.time_calls(dqf, copies)
    res["dequantize_2048x11008_cold"] = summary(timer.time_calls(dqf, 4 * copies), 5 * n, "GB/s",
                                                PEAK_HBM_GBS)
    del qin, fout, dqf

    # ---- small, latency-bound workloads
    log("extra: small chain and small deconv")
    c1 = qi.make_chain_small()
    xf = torch.from_numpy(c1.x_fp32).cuda()
    xq1 = torch.empty((c1.M, c1.K), dtype=torch.int8, device="cuda")
    w1 = torch.from_numpy(c1.w).cuda()
    s1 = torch.from_numpy(c1.weight_scales).cuda()
    b1 = torch.from_numpy(c1.bias).cuda()
    o1 = torch.empty((c1.M, c1.N), dtype=torch.int8, device="cuda")

    def chain():
        check(lib.q8ta_quantize_per_tensor(xf.data_ptr(), xq1.data_ptr(), c1.M * c1.K,
                                           c1.in_scale, c1.in_zp, stream))
        check(lib.q8ta_linear(xq1.data_ptr(), c1.M, c1.K, c1.in_scale, c1.in_zp, w1.data_ptr(),
                              c1.N, None, s1.data_ptr(), b1.data_ptr(), c1.out_scale, c1.out_zp,
                              b"none", o1.data_ptr(), stream))
    timer.time_calls([chain], 10)
    res["chain_quantize_4x64_linear_4x64x32"] = summary(timer.time_calls([chain], reps),
                                                        2 * 4 * 64 * 32, "TOPS", None)

    def chain_fused():
        check(lib.q8ta_quantize_linear(xf.data_ptr(), c1.M, c1.K, c1.in_scale, c1.in_zp,
                                       w1.data_ptr(), c1.N, None, s1.data_ptr(), b1.data_ptr(),
                                       c1.out_scale, c1.out_zp, b"none", o1.data_ptr(), stream))
    timer.time_calls([chain_fused], 10)
    res["chain_quantize_4x64_linear_4x64x32_one_call"] = summary(
        timer.time_calls([chain_fused], reps), 2 * 4 * 64 * 32, "TOPS", None)

    d4 = qi.make_deconv_small()
    x4 = torch.from_numpy(d4.x).cuda()
    w4 = torch.from_numpy(d4.w).cuda()
    s4 = torch.from_numpy(d4.weight_scales).cuda()
    b4 = torch.from_numpy(d4.bias).cuda()
    o4 = torch.empty((1, 32, 64, 64), dtype=torch.int8, device="cuda")

    def dc_small():
        check(lib.q8ta_conv2d_transposed(
            x4.data_ptr(), 1, 64, 32, 32, d4.in_scale, d4.in_zp, w4.data_ptr(), 32, 4, 4, 1024,
            None, s4.data_ptr(), b4.data_ptr(), d4.out_scale, d4.out_zp, 2, 2, 1, 1, 0, 0, 1, 1,
            1, b"none", o4.data_ptr(), 64, 64, stream))
    timer.time_calls([dc_small], 10)
    r = summary(timer.time_calls([dc_small], reps), deconv_ops(d4), "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = deconv_ops(d4)
    res["deconv_1x64x32x32_k4s2p1_to_1x32x64x64"] = r

    # ---- forward conv [8,256,64,64] K3 s1 p1 -> [8,128,64,64] (implicit GEMM)
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
    timer.time_calls([conv], 5)
    cops = conv_ops(cc)
    r = summary(timer.time_calls([conv], reps), cops, "TOPS", PEAK_INT8_TOPS)
    r["exact_valid_tap_ops"] = cops
    res["conv2d_8x256x64x64_k3s1p1_to_8x128x64x64"] = r
    del cx, cout

    # ---- depthwise [8,256,64,64] K3 s1 p1, HBM-bound: rotate 40 input copies (335 MB)
    log("extra: depthwise conv [8,256,64,64]")
    dc = qi.make_depthwise_large()
    copies = 40
    dxs = [torch.from_numpy(dc.x).cuda() for _ in range(copies)]
    dw_, ds_, db_ = (torch.from_numpy(a).cuda() for a in (dc.w, dc.weight_scales, dc.bias))
    dN, dC, dH, dW = dc.x.shape
    dout2 = torch.empty((dN, dC, dc.H_out, dc.W_out), dtype=torch.int8, device="cuda")

    def dw_call(i):
        check(lib.q8ta_conv2d(
            dxs[i].data_ptr(), dN, dC, dH, dW, dc.in_scale, dc.in_zp, dw_.data_ptr(), dC, dc.Kh,
            dc.Kw, dc.w.shape[1], None, ds_.data_ptr(), db_.data_ptr(), dc.out_scale, dc.out_zp,
            1, 1, 1, 1, 1, 1, dC, b"none", dout2.data_ptr(), dc.H_out, dc.W_out, stream))
    dwf = [(lambda i=i: dw_call(i)) for i in range(copies)]
    dbytes = int(dc.x.size + dout2.numel() + dc.w.size + 8 * dC)
    timer.time_calls(dwf, copies)
    r = summary(timer.time_calls(dwf, 4 * copies), dbytes, "GB/s", PEAK_HBM_GBS)
    r["algorithmic_bytes"] = dbytes
    res["depthwise_8x256x64x64_k3s1p1_cold"] = r
    del dxs, dout2
    for k, v in res.items():
        log(f"  {k}: {v}")
    return res


if __name__ == "__main__":
    main()
