"""Throughput of the fp16 TN GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--all] [--no-cpu-baseline]

A step is one GEMM D = alpha * A @ B^T + beta * C over the workload's seeded
synthetic inputs, already resident in HBM.  The default workload is the
compute-bound 4096 x 4096 x 4096 product with fp16 D.  The timed region is
K back-to-back calls on one stream, bracketed by device synchronisations,
and timed with HIP events recorded on that same stream.  One JSON line goes
to stdout; `--all` adds a table of every workload on stderr.

The fp32 transpose of the pages is measured the same way with
`--workload transpose_1024` (their 1024 x 1024 case) or `transpose_8192`
(8192 x 8192, 512 MiB moved: past the 256 MB last-level cache, so HBM).
The attention forward pass O = softmax(scale Q K^T) V runs with
`--workload attn_64x1024` (64 heads of 1024 queries and keys, d = 64: the
score product completed into the forward pass) or `attn_small`, and the
fp16-accumulating GEMM with `--workload f16acc_4096`.
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

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "dense_gemm_fp16_amd", "csrc")
# device code of the GEMM kernels (host-side planning is not part of it)
KERNEL_SOURCES = ("gemm_tn_kernels.hpp", "gemm_tn_config.hpp",
                  "gemm_tn_launch.hpp", "gemm_tn_tile256.hip",
                  "gemm_tn_tile128.hip", "gemm_tn_tile64.hip",
                  "lds_layout.hpp")
TRANSPOSE_SOURCES = ("transpose.hip", "lds_layout.hpp")
ATTENTION_SOURCES = ("attention_fwd.hip", "gemm_tn_kernels.hpp",
                     "gemm_tn_config.hpp", "lds_layout.hpp")
ATTENTIONS = ("attn_64x1024", "attn_small")
F16ACC_SOURCES = ("gemm_f16acc.hip", "gemm_tn_kernels.hpp", "gemm_tn_config.hpp",
                  "lds_layout.hpp")
# fp16-accumulating GEMMs: name -> (batch, M, N, K)
F16ACCS = {"f16acc_4096": (1, 4096, 4096, 4096)}
# fp32 transposes: name -> (batch, M, N)
TRANSPOSES = {"transpose_1024": (1, 1024, 1024),
              "transpose_8192": (1, 8192, 8192)}


def _sources(workload: str):
    if workload in TRANSPOSES:
        return TRANSPOSE_SOURCES
    if workload in ATTENTIONS:
        return ATTENTION_SOURCES
    if workload in F16ACCS:
        return F16ACC_SOURCES
    return KERNEL_SOURCES


def _kernel_names(workload: str):
    """Names (substrings) of the kernels one call of the workload runs."""
    if workload in TRANSPOSES:
        return ("transpose_f32_kernel",)
    if workload in ATTENTIONS:
        return ("attn_fwd_kernel",)
    if workload in F16ACCS:
        return ("gemm_f16acc_kernel",)
    return ("gemm_tn_kernel", "splitk_reduce")


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (an edit of a comment
    does not change the kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_fingerprint(workload: str = "c3_4096") -> str:
    """Hash of the kernel sources' code; a traffic figure measured on other
    code does not describe the kernel being timed."""
    import hashlib
    h = hashlib.sha256()
    for f in _sources(workload):
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(CSRC, f)).read()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    prefix = "" if (workload in TRANSPOSES or workload in ATTENTIONS
                    or workload in F16ACCS) else "gemm_tn_"
    return os.path.join(PROFILES, f"{prefix}{workload}_traffic.json")


def load_traffic(workload: str):
    """HBM bytes per launch measured by the counters, if they were taken on
    the current kernel sources; otherwise None."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("fingerprint") != kernel_fingerprint(workload):
        return None
    return t


def summarize_pmc(fetch_csv, write_csv, workload, cal_mib):
    """Per-launch HBM bytes of the GEMM kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reports for the
    calibration copy of cal_mib MiB (which reads and writes cal_mib MiB)."""
    import csv
    import statistics

    wanted = _kernel_names(workload)

    def per_kernel(path, counter):
        gemm, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if any(k in name for k in wanted):
                gemm.append((int(r["Dispatch_Id"]), name, v))
            elif "copy" in name.lower():
                copy.append(v)
        return gemm, copy

    out = {"workload": workload, "fingerprint": kernel_fingerprint(workload),
           "calibration_mib": cal_mib}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                               ("write", write_csv, "WRITE_SIZE")):
        gemm, copy = per_kernel(path, counter)
        if not gemm or not copy:
            raise SystemExit(f"{path}: no {counter} rows for the GEMM or "
                             "the calibration copy")
        cal_kib = max(copy)
        factor = cal_mib * 1024.0 / cal_kib
        # all kernels of one GEMM call (split-K adds a reduction) summed
        names = sorted({n for _, n, _ in gemm})
        per_name = {n: statistics.median(v for _, m, v in gemm if m == n)
                    for n in names}
        kib = sum(per_name.values())
        out[f"{key}_kib_raw"] = kib
        out[f"{key}_calibration_kib_raw"] = cal_kib
        out[f"{key}_scale"] = factor
        out[f"{key}_bytes"] = kib * 1024.0 * factor
    out["bytes_per_launch"] = out["fetch_bytes"] + out["write_bytes"]
    return out


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
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (the "
                         "known-size reference for HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV",
                                                          "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv "
                         "files (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--copy-calibration-mib into a traffic summary")
    ap.add_argument("--calibration-mib", type=int, default=256,
                    help="size of the calibration copy in --summarize-pmc")
    ap.add_argument("--cold", action="store_true",
                    help="also time the GEMM with cold caches: a 512 MiB "
                         "write before every launch evicts the operands "
                         "from the L2s and the Infinity Cache")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="median / min / max kernel time per call of "
                         "--workload from a rocprofv3 kernel_trace.csv")
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


def time_workload_cold(w, steps):
    """Median time of one call (seconds) with cold caches: before each
    launch a 512 MiB fill (more than the 256 MB Infinity Cache and the
    L2s) evicts A, B and C; HIP events bracket the GEMM alone."""
    import statistics
    import torch
    import dense_gemm_fp16_amd as g
    A, B, C, D = _device_inputs(w, torch)
    flush = torch.empty(512 * 1024 * 1024 // 4, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for i in range(steps + 1):
        flush.fill_(float(i))
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        g.gemm_tn(A, B, w.alpha, w.beta, C, out=D, stream=stream)
        stop.record(stream)
        torch.cuda.synchronize()
        if i:
            times.append(start.elapsed_time(stop) / 1e3)
    return statistics.median(times)


def summarize_trace(csv_path, workload):
    """Per-call kernel time of `workload` from a rocprofv3 kernel trace:
    the kernels of one call (a split-K or tail-split call runs two or three)
    are summed in dispatch order."""
    import csv
    import statistics
    wanted = _kernel_names(workload)
    rows = [r for r in csv.DictReader(open(csv_path))
            if any(k in r["Kernel_Name"] for k in wanted)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    names = [r["Kernel_Name"] for r in rows]
    # a call starts with the first kernel name seen (the GEMM kernel of the
    # first part; a reduction or a second part follows it)
    per_call = []
    first = names[0] if names else None
    for n, d in zip(names, durs):
        if n == first or not per_call:
            per_call.append(d)
        else:
            per_call[-1] += d
    ns = sorted(per_call)
    return {"workload": workload, "calls": len(ns),
            "kernels_per_call": len(durs) / max(len(ns), 1),
            "median_ns": statistics.median(ns) if ns else None,
            "min_ns": ns[0] if ns else None, "max_ns": ns[-1] if ns else None}


def _cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the architecture."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


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
                      f"{dt:.1f} s on {threads} threads of {_cpu_model()}; "
                      f"{flops / dt / 1e9:.1f} GFLOP/s"}


def _transpose_input(batch, M, N, torch):
    """Seeded uniform [-1, 1) fp32 values, drawn on the GPU (the values do
    not change the copy's speed; the parity tests use the seeded host
    generator)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED0100 + M)
    return torch.rand((batch, M, N), generator=gen, device="cuda") * 2 - 1


def time_transpose(batch, M, N, steps, warmup):
    import torch
    import dense_gemm_fp16_amd as g
    x = _transpose_input(batch, M, N, torch)
    y = torch.empty((batch, N, M), device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.transpose_f32(x, out=y, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.transpose_f32(x, out=y, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def cpu_baseline_transpose(batch, M, N, target_s):
    """The transpose oracle (one thread: it is numpy row copies) on the first
    R rows of a host copy of the input, rate scaled to GB/s moved."""
    from oracle import transpose as T
    x = np.random.default_rng(0).random((1, M, N), dtype=np.float32)
    rows, reps = min(M, 256), 1
    while True:
        t = time.perf_counter()
        for _ in range(reps):
            T.transpose(x[:, :rows])
        dt = time.perf_counter() - t
        if dt >= target_s / 4:
            break
        if rows < M:
            rows = min(M, rows * 4)
        else:
            reps *= 4
    return {"value": 8.0 * rows * N * reps / dt / 1e9, "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{reps} x the first {rows} of {M} rows of the "
                      f"{M}x{N} input ({dt:.2f} s on {_cpu_model()})"}


def _attention_inputs(w, torch):
    return [torch.from_numpy(x).cuda() for x in (w.Q, w.K, w.V)]


def time_attention(w, steps, warmup):
    """Average time of one attention_fwd call (seconds), HIP events on the
    launch stream; the seeded inputs are resident in HBM."""
    import torch
    import dense_gemm_fp16_amd as g
    q, k, v = _attention_inputs(w, torch)
    dt = torch.float16 if w.out_dtype == "f16" else torch.float32
    o = torch.empty(q.shape, dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.attention_fwd(q, k, v, w.scale, out=o, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.attention_fwd(q, k, v, w.scale, out=o, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def cpu_baseline_attention(w, target_s):
    """The attention oracle (float64 numpy; its products run on the BLAS
    threads) over the first H heads, repeated until the run takes about a
    quarter of target_s; rate scaled to TFLOP/s of the workload's count."""
    from oracle import attention as AT
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()]
                    or [1])
    except Exception:                       # noqa: BLE001
        cores = 1
    heads, reps = 1, 1
    while True:
        t = time.perf_counter()
        for _ in range(reps):
            AT.attention(w.Q[:heads], w.K[:heads], w.V[:heads], w.scale)
        dt = time.perf_counter() - t
        if dt >= target_s / 4:
            break
        if heads < w.batch:
            heads = min(w.batch, heads * 4)
        else:
            reps *= 2
    flops = 4.0 * heads * reps * w.Lq * w.Lk * w.d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x the first {heads} of {w.batch} heads "
                      f"({w.Lq}x{w.Lk}x{w.d}, float64 numpy), {dt:.2f} s "
                      f"on {_cpu_model()}"}


def attention_main(a):
    import seeded_inputs as si
    w = si.attention_workload(a.workload)
    sec = time_attention(w, a.steps, a.warmup)
    tflops = w.flops / sec / 1e12
    t = load_traffic(a.workload)
    line = {
        "metric": (f"attention forward TFLOP/s ({w.batch} heads, "
                   f"{w.Lq} queries x {w.Lk} keys, d {w.d}; fp16 in, fp32 "
                   f"acc); % of MI355X fp16 MFMA peak"),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"attention_fwd_{w.batch}x{w.Lq}x{w.Lk}x{w.d}",
                   "batch": w.batch, "Lq": w.Lq, "Lk": w.Lk, "d": w.d,
                   "scale": w.scale, "out": w.out_dtype},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_F16_MFMA_TFLOPS, 4),
                     "traffic": round(t["bytes_per_launch"]) if t else None},
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_attention(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)


def time_f16acc(batch, M, N, K, steps, warmup):
    """Average time of one gemm_tn_f16acc call (seconds); inputs uniform in
    [-1, 1), drawn on the GPU (the values do not change the speed)."""
    import torch
    import dense_gemm_fp16_amd as g
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED0300 + K)
    A = (torch.rand((batch, M, K), generator=gen, device="cuda") * 2 - 1).half()
    B = (torch.rand((batch, N, K), generator=gen, device="cuda") * 2 - 1).half()
    D = torch.empty((batch, M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.gemm_tn_f16acc(A, B, out=D, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.gemm_tn_f16acc(A, B, out=D, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def cpu_baseline_f16acc(batch, M, N, K, target_s):
    """The fp16-accumulating oracle (float64 numpy, one product per 16-deep
    step) over the first R rows of D; rate scaled to TFLOP/s."""
    from oracle import gemm_f16acc as F
    r = np.random.default_rng(0)
    A = r.uniform(-1, 1, (1, M, K)).astype(np.float16)
    B = r.uniform(-1, 1, (1, N, K)).astype(np.float16)
    rows = 16
    while True:
        t = time.perf_counter()
        F.gemm_tn_f16acc(A[:, :rows], B)
        dt = time.perf_counter() - t
        if dt >= target_s / 4 or rows >= M:
            break
        rows = min(M, rows * 4)
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s",
            "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {M} rows of D ({M}x{N}x{K}), "
                      f"{dt:.2f} s on {_cpu_model()}"}


def f16acc_main(a):
    batch, M, N, K = F16ACCS[a.workload]
    sec = time_f16acc(batch, M, N, K, a.steps, a.warmup)
    tflops = 2.0 * batch * M * N * K / sec / 1e12
    t = load_traffic(a.workload)
    line = {
        "metric": (f"fp16-accumulating GEMM TFLOP/s at {M}x{N}x{K} (fp16 in, "
                   f"fp16 sum every 16 k); % of MI355X fp16 MFMA peak"),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"tn_gemm_f16acc_{M}x{N}x{K}", "M": M, "N": N,
                   "K": K, "batch": batch},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_F16_MFMA_TFLOPS, 4),
                     "traffic": round(t["bytes_per_launch"]) if t else None},
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_f16acc(batch, M, N, K,
                                                   a.cpu_seconds)
    print(json.dumps(line), flush=True)


def transpose_main(a):
    batch, M, N = TRANSPOSES[a.workload]
    sec = time_transpose(batch, M, N, a.steps, a.warmup)
    nbytes = 8.0 * batch * M * N
    gbs = nbytes / sec / 1e9
    t = load_traffic(a.workload)
    line = {
        "metric": f"fp32 transpose GB/s ({M}x{N}); % of MI355X HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"transpose_f32_{M}x{N}"
                               + (f"_batch{batch}" if batch > 1 else ""),
                   "M": M, "N": N, "batch": batch},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": round(t["bytes_per_launch"]) if t else None},
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_transpose(batch, M, N,
                                                      a.cpu_seconds)
    print(json.dumps(line), flush=True)


def describe(w):
    import dense_gemm_fp16_amd as g
    return g.describe(w.batch, w.M, w.N, w.K, w.beta, w.out_dtype, True)


def main():
    a = _args()
    if a.summarize_trace:
        print(json.dumps(summarize_trace(a.summarize_trace, a.workload)))
        return
    if a.summarize_pmc:
        t = summarize_pmc(a.summarize_pmc[0], a.summarize_pmc[1], a.workload,
                          a.calibration_mib)
        os.makedirs(PROFILES, exist_ok=True)
        with open(traffic_path(a.workload), "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not "
              "supported (the GEMM runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import seeded_inputs as si

    if a.copy_calibration_mib:
        n = a.copy_calibration_mib * 1024 * 1024 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if a.workload in TRANSPOSES:
        transpose_main(a)
        return
    if a.workload in ATTENTIONS:
        attention_main(a)
        return
    if a.workload in F16ACCS:
        f16acc_main(a)
        return
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
    t = load_traffic(a.workload)
    roof["traffic"] = round(t["bytes_per_launch"]) if t else None
    line = {
        "metric": (f"GEMM TFLOP/s (fp16 in, fp32 acc) at "
                   + ("4096^3" if a.workload == "c3_4096"
                      else f"{w.M}x{w.N}x{w.K}" + (
                          f" batch {w.batch}" if w.batch > 1 else ""))
                   + "; % of MI355X fp16 MFMA peak"),
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
        for name in ATTENTIONS:
            wa = si.attention_workload(name)
            s = time_attention(wa, a.steps, a.warmup)
            tf = wa.flops / s / 1e12
            gb = wa.algorithmic_bytes / s / 1e9
            print(f"{name:<14}{'attention forward, 128 queries x 64 keys':<60}"
                  f"{s * 1e6:>10.2f}{tf:>10.1f}"
                  f"{100 * tf / PEAK_F16_MFMA_TFLOPS:>8.2f}{gb:>9.0f}"
                  f"{100 * gb / PEAK_HBM_GBS:>7.1f}", file=sys.stderr)
        for name, (batch, M, N, K) in F16ACCS.items():
            s = time_f16acc(batch, M, N, K, a.steps, a.warmup)
            tf = 2.0 * batch * M * N * K / s / 1e12
            gb = 2.0 * batch * (M * K + N * K + M * N) / s / 1e9
            print(f"{name:<14}{'fp16 accumulation, 128x128x32, k16 MFMA':<60}"
                  f"{s * 1e6:>10.2f}{tf:>10.1f}"
                  f"{100 * tf / PEAK_F16_MFMA_TFLOPS:>8.2f}{gb:>9.0f}"
                  f"{100 * gb / PEAK_HBM_GBS:>7.1f}", file=sys.stderr)
        for name, (batch, M, N) in TRANSPOSES.items():
            s = time_transpose(batch, M, N, a.steps, a.warmup)
            gb = 8.0 * batch * M * N / s / 1e9
            print(f"{name:<14}{'fp32 transpose, 64x64 tiles':<60}"
                  f"{s * 1e6:>10.2f}{'-':>10}{'-':>8}{gb:>9.0f}"
                  f"{100 * gb / PEAK_HBM_GBS:>7.1f}", file=sys.stderr)
    if a.cold:
        cs = time_workload_cold(w, a.steps)
        line["cold"] = {"ms_per_call": round(cs * 1e3, 5),
                        "tflops": round(w.flops / cs / 1e12, 2),
                        "flush_mib": 512}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
