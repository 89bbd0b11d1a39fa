"""Throughput of the fp16 TN GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--all] [--no-cpu-baseline]

A step is one GEMM D = alpha * A @ B^T + beta * C over the workload's seeded
synthetic inputs, already resident in HBM.  The default workload is the
compute-bound 4096 x 4096 x 4096 product with fp16 D.  The timed region is
K back-to-back calls on one stream, bracketed by device synchronisations,
and timed with HIP events recorded on that same stream.  One JSON line goes
to stdout; `--all` adds a table of every workload on stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

PEAK_F16_MFMA_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0           # HBM3E


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3_4096")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload (stderr table)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def _device_inputs(w, torch):
    A = torch.from_numpy(np.ascontiguousarray(w.A)).cuda()
    B = torch.from_numpy(np.ascontiguousarray(w.B)).cuda()
    C = None
    if w.C is not None:
        C = torch.from_numpy(np.ascontiguousarray(w.C)).cuda()
    dt = torch.float16 if w.out_dtype == "f16" else torch.float32
    D = torch.empty((w.batch, w.M, w.N), dtype=dt, device="cuda")
    return A, B, C, D


def time_workload(w, steps, warmup):
    """Average time of one call (seconds), HIP events on the launch stream."""
    import torch
    import dense_gemm_fp16_amd as g
    A, B, C, D = _device_inputs(w, torch)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.gemm_tn(A, B, w.alpha, w.beta, C, out=D, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.gemm_tn(A, B, w.alpha, w.beta, C, out=D, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def cpu_baseline(w, target_s):
    """The oracle on the host cores over the first R rows of D, R chosen so
    the run takes about target_s seconds; rate scaled to TFLOP/s."""
    import oracle
    threads = oracle.default_threads()
    rows_total = w.batch * w.M
    # grow the sample until one run takes a quarter of the target, then
    # size the measured run from that rate
    rows = min(rows_total, max(threads, 16))
    while True:
        t = time.perf_counter()
        oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C, rows=(0, rows),
                       threads=threads)
        dt = time.perf_counter() - t
        if dt >= target_s / 4 or rows >= rows_total:
            break
        rows = min(rows_total, rows * 4)
    if rows < rows_total and dt < target_s:
        rows = int(min(rows_total, rows * target_s / max(dt, 1e-6)))
        t = time.perf_counter()
        oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C, rows=(0, rows),
                       threads=threads)
        dt = time.perf_counter() - t
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {rows} of {rows_total} rows of D "
                      f"({rows}x{w.N}x{w.K}, fp64 sequential k-sum), "
                      f"{dt:.1f} s on {threads} threads of "
                      f"{platform.processor() or platform.machine()}"}


def describe(w):
    import dense_gemm_fp16_amd as g
    return g.describe(w.batch, w.M, w.N, w.K, w.beta, w.out_dtype, True)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not "
              "supported (the GEMM runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import seeded_inputs as si

    w = si.workload(a.workload)
    sec = time_workload(w, a.steps, a.warmup)
    tflops = w.flops / sec / 1e12
    gbs = w.algorithmic_bytes / sec / 1e9
    compute_bound = w.flops / w.algorithmic_bytes > (
        PEAK_F16_MFMA_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
    if compute_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2),
                "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_F16_MFMA_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof["traffic"] = None
    line = {
        "metric": "GEMM TFLOP/s (fp16 in, fp32 acc) at 4096^3; "
                  "% of MI355X fp16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "pct_of_peak": round(100 * tflops / PEAK_F16_MFMA_TFLOPS, 2),
        "config": {"workload": f"tn_gemm_{w.M}x{w.N}x{w.K}"
                               + (f"_batch{w.batch}" if w.batch > 1 else ""),
                   "M": w.M, "N": w.N, "K": w.K, "batch": w.batch,
                   "alpha": w.alpha, "beta": w.beta,
                   "in": "f16", "acc": "f32", "out": w.out_dtype,
                   "kernel": describe(w)},
        "roofline": roof,
    }
    if a.all:
        print(f"{'workload':<14}{'kernel':<60}{'us':>10}{'TFLOP/s':>10}"
              f"{'%peak':>8}{'GB/s':>9}{'%HBM':>7}", file=sys.stderr)
        for name in si.WORKLOADS:
            wx = si.workload(name)
            s = time_workload(wx, a.steps, a.warmup)
            tf = wx.flops / s / 1e12
            gb = wx.algorithmic_bytes / s / 1e9
            print(f"{name:<14}{describe(wx):<60}{s * 1e6:>10.2f}{tf:>10.1f}"
                  f"{100 * tf / PEAK_F16_MFMA_TFLOPS:>8.2f}{gb:>9.0f}"
                  f"{100 * gb / PEAK_HBM_GBS:>7.1f}", file=sys.stderr)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
