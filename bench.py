"""Throughput of the fp16 TN GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--all] [--no-cpu-baseline]

A step is one GEMM D = alpha * A @ B^T + beta * C over the workload's seeded
synthetic inputs, already resident in HBM.  The default workload is the
compute-bound 4096 x 4096 x 4096 product with fp16 D.  The timed region is
K back-to-back calls on one stream, bracketed by device synchronisations,
and timed with HIP events recorded on that same stream.  One JSON line goes
to stdout.  `--all` first prints one JSON record per configuration of the
study (256^3, 1024^3 with C, 4096^3, 1000x1030x1000, 128x4096x8192, the
64-batch score product), each with TFLOP/s, GB/s, both roofline fractions,
and the CPU oracle run over every output on the host's cores (its time is
the record's CPU baseline; its results check the GPU output, and the
integer variant's bit for bit); `--extras` adds a stderr table of the other
workloads.  Under `rocprofv3 --kernel-trace`, `--summarize-trace-all`
turns the trace of such a run into per-configuration kernel times.

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
import re
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
                  "gemm_tn_onek.hip", "lds_layout.hpp")
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
    return ("gemm_tn_kernel", "gemm_onek_kernel", "splitk_reduce")


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
                    help="first print one JSON record per configuration of "
                         "the study (c1 ... c5), each with its full-output "
                         "oracle run as CPU baseline and parity check")
    ap.add_argument("--extras", action="store_true",
                    help="also time the workloads beyond the study's "
                         "configurations (stderr table)")
    ap.add_argument("--summarize-trace-all", nargs="+",
                    metavar=("KERNEL_TRACE_CSV", "BENCH_JSONL"),
                    help="per-configuration kernel times from a rocprofv3 "
                         "kernel_trace.csv of a --all run (markdown table; "
                         "with the run's stdout, its HIP-event times and "
                         "oracle times beside them)")
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
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.matmul (the vendor BLAS) on the "
                         "same inputs, interleaved with this library "
                         "(context only; plain products)")
    ap.add_argument("--ab", metavar="LIB[@FORCE],...",
                    help="time builds of the library against each other in "
                         "one process: gemm_tn_ex of each shared library "
                         "(optionally with a GEMM_TN_FORCE value, ';' for "
                         "','), interleaved bursts over --ab-shapes")
    ap.add_argument("--ab-shapes", default="1x4096x4096x4096",
                    help="BxMxNxK[xOUT[xC]] list: OUT 1 = fp32 D, C 1 = "
                         "alpha 1.5, beta 0.5 with a C read")
    ap.add_argument("--ab-rounds", type=int, default=16)
    ap.add_argument("--plan-grid", nargs="?", const=PLAN_GRID_SHAPES,
                    metavar="BxMxNxK,...",
                    help="time every tile x split-K choice and the "
                         "planner's own on each shape (JSON lines)")
    ap.add_argument("--summarize-plan-grid", metavar="PLAN_GRID_JSONL",
                    help="markdown table of a --plan-grid run")
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


def time_workload(w, steps, warmup, return_output=False):
    """Average time of one call (seconds), HIP events on the launch stream
    (and the output of the last call, on the host, with return_output)."""
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
    sec = start.elapsed_time(stop) / 1e3 / steps
    if return_output:
        return sec, D.cpu().numpy()
    return sec


def time_workload_graph(w, steps, warmup):
    """Average time of one call (seconds) when `steps` back-to-back calls
    are captured into one HIP graph and the graph is replayed: the GPU-side
    time per call without the host's per-call cost (argument checks,
    planning, the launch through the binding), which bounds small
    problems when they are called one by one."""
    import torch
    import dense_gemm_fp16_amd as g
    A, B, C, D = _device_inputs(w, torch)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(warmup, 1)):   # plans and workspaces made here
            g.gemm_tn(A, B, w.alpha, w.beta, C, out=D)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            g.gemm_tn(A, B, w.alpha, w.beta, C, out=D)
    graph.replay()                        # first replay uploads the graph
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def time_vendor_interleaved(w, rounds=6, burst=10):
    """Context, not a target: median time per call (seconds) of this library
    and of torch.matmul (the vendor BLAS) on the same device inputs, in
    interleaved bursts of `burst` back-to-back calls, HIP events around each
    burst.  Only for plain products (alpha 1, beta 0)."""
    import statistics
    import torch
    import dense_gemm_fp16_amd as g
    A, B, C, D = _device_inputs(w, torch)
    ours = lambda: g.gemm_tn(A, B, out=D)
    if w.batch == 1:        # one 2-D product, B passed as a transposed view
        A2, Bt, V = A[0], B[0].t(), torch.empty_like(D[0])
    else:                   # batched: a contiguous transposed copy of B
        A2, Bt, V = A, B.transpose(-1, -2).contiguous(), torch.empty_like(D)
    if D.dtype == torch.float16:
        vendor = lambda: torch.matmul(A2, Bt, out=V)
    elif w.batch == 1:      # fp16 operands, fp32 output from the BLAS
        vendor = lambda: torch.mm(A2, Bt, out_dtype=torch.float32)
    else:
        vendor = lambda: torch.bmm(A2, Bt, out_dtype=torch.float32)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    times = {"library": [], "torch_matmul": []}
    for _ in range(rounds):
        for name, f in (("library", ours), ("torch_matmul", vendor)):
            f()
            f()
            start.record()
            for _ in range(burst):
                f()
            stop.record()
            torch.cuda.synchronize()
            times[name].append(start.elapsed_time(stop) / 1e3 / burst)
    return {k: statistics.median(v) for k, v in times.items()}


PLAN_GRID_SPLITS = (1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 24, 32, 48, 64, 96, 128,
                    192, 256)
PLAN_GRID_SHAPES = (
    "1x512x512x2048,1x512x512x8192,1x768x768x4096,1x1024x1024x2048,"
    "1x1024x1024x4096,1x1024x1024x8192,1x1024x1024x16384,1x1536x1536x2048,"
    "1x1536x1536x4096,1x1536x1536x8192,1x2048x2048x2048,1x2048x2048x4096,"
    "1x2048x2048x8192,1x2560x2560x4096,1x3072x3072x2048,1x3072x3072x4096,"
    "1x256x256x16384,1x256x2048x8192,1x512x4096x4096,1x2816x2816x6144,"
    "2x1024x1024x4096")


def plan_grid(shapes, rounds=4, burst=10):
    """For each BxMxNxK shape (fp16 D, alpha 1, beta 0): the median time per
    call of every tile x split-K choice (forced, slices of at least 256
    along K, partials within the no-allocation scratch) and of the
    planner's own choice, in interleaved bursts of `burst` calls, HIP
    events around each burst.  One JSON line per shape.  A suffix "@la.lb"
    stores A (la = 1) or B (lb = 1) along M or N instead of along K."""
    import statistics
    import torch
    import dense_gemm_fp16_amd as g

    def cdiv(x, y):
        return -(-x // y)

    def plan_of(b, M, N, K, tail=False):
        d = dict(kv.split("=") for kv in
                 g.describe(b, M, N, K, layouts=lay).split())
        p = (int(d["tile"].split("x")[0]), int(d["split"]))
        return p + (int(d["tail_rows"]), int(d["tail_split"])) if tail else p

    gen = torch.Generator(device="cuda")
    for tok in shapes.split(","):
        dims, _, lays = tok.partition("@")
        b, M, N, K = (int(x) for x in dims.split("x"))
        lay = tuple(int(x) for x in lays.split(".")) if lays else (0, 0)
        specs = {}
        for tile in (256, 128, 64):
            if tile == 256 and (M < 256 or N < 256):
                continue
            for s in PLAN_GRID_SPLITS:
                if s > 1 and K // s < 256:
                    break
                se = cdiv(K, cdiv(cdiv(K, s), 64) * 64)
                if se > 1 and se * b * M * cdiv(N, 4) * 16 > \
                        g.NOALLOC_SCRATCH_BYTES:
                    break
                specs.setdefault((tile, se), f"tile={tile},split={se},tail=0")
        gen.manual_seed(b * 7919 + M * 31 + N * 17 + K)
        def operand(rows, along_rows):
            if along_rows:     # stored K x rows, passed as a transposed view
                x = torch.rand(b, K, rows, device="cuda", generator=gen)
                return (x * 2 - 1).half().transpose(1, 2)
            x = torch.rand(b, rows, K, device="cuda", generator=gen)
            return (x * 2 - 1).half()
        A = operand(M, lay[0] == 1)
        B = operand(N, lay[1] == 1)
        D = torch.empty(b, M, N, device="cuda", dtype=torch.float16)
        runs = [("planner", "")] + [(k, v) for k, v in specs.items()]
        times = {k: [] for k, _ in runs}
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        old = os.environ.get("GEMM_TN_FORCE")
        try:
            for _ in range(rounds):
                for key, spec in runs:
                    os.environ["GEMM_TN_FORCE"] = spec
                    g.gemm_tn(A, B, out=D)
                    g.gemm_tn(A, B, out=D)
                    start.record()
                    for _ in range(burst):
                        g.gemm_tn(A, B, out=D)
                    stop.record()
                    stop.synchronize()
                    times[key].append(start.elapsed_time(stop) * 1e3 / burst)
            for key, spec in runs[1:]:
                os.environ["GEMM_TN_FORCE"] = spec
                assert plan_of(b, M, N, K) == key, (tok, key)
            os.environ["GEMM_TN_FORCE"] = ""
            chosen = plan_of(b, M, N, K, tail=True)
        finally:
            if old is None:
                os.environ.pop("GEMM_TN_FORCE", None)
            else:
                os.environ["GEMM_TN_FORCE"] = old
        med = {k: statistics.median(v) for k, v in times.items()}
        print(json.dumps({
            "shape": [b, M, N, K], "layouts": list(lay), "rounds": rounds,
            "burst": burst,
            "planner": {"tile": chosen[0], "split": chosen[1],
                        "tail_rows": chosen[2], "tail_split": chosen[3],
                        "us": round(med["planner"], 2)},
            "choices": [[k[0], k[1], round(med[k], 2)] for k in specs]}),
            flush=True)
        del A, B, D


def ab_compare(variants, shapes, rounds=16, burst=20):
    """Builds of the library timed against each other in one process, so
    that the machine's clock state is shared: each variant is a shared
    library (built with `python -m dense_gemm_fp16_amd.build --defines ...
    --out LIB`) whose gemm_tn_ex is called through ctypes, optionally with
    a GEMM_TN_FORCE value after '@'.  Per shape, `rounds` rounds of a burst
    of `burst` calls per variant (order reversed every other round), HIP
    events around each burst; one JSON line with the median and minimum
    time per call and whether every variant wrote the same bits."""
    import ctypes
    import statistics
    import torch
    i64, f32, vp, ci = (ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                        ctypes.c_int)
    libs, vs = {}, []
    for v in variants.split(","):
        path, _, force = v.partition("@")
        if path not in libs:
            lib = ctypes.CDLL(os.path.abspath(path))
            lib.gemm_tn_ex.argtypes = [i64, i64, i64, i64, f32, vp, ci, i64,
                                       i64, vp, ci, i64, i64, f32, vp, i64,
                                       i64, vp, i64, i64, ci, vp]
            lib.gemm_tn_ex.restype = ci
            libs[path] = lib
        vs.append((v, libs[path], force.replace(";", ",")))
    old = os.environ.get("GEMM_TN_FORCE")
    try:
        for tok in shapes.split(","):
            dims = [int(x) for x in tok.split("x")]
            b, M, N, K = dims[:4]
            f32_out = len(dims) > 4 and dims[4] == 1
            with_c = len(dims) > 5 and dims[5] == 1
            gen = torch.Generator(device="cuda")
            gen.manual_seed(b * 7919 + M * 31 + N * 17 + K)
            A = (torch.rand(b, M, K, device="cuda", generator=gen) * 2 - 1)
            B = (torch.rand(b, N, K, device="cuda", generator=gen) * 2 - 1)
            A, B = A.half(), B.half()
            dt = torch.float32 if f32_out else torch.float16
            C = ((torch.rand(b, M, N, device="cuda", generator=gen) * 2 - 1)
                 .to(dt) if with_c else None)
            Ds = [torch.empty(b, M, N, device="cuda", dtype=dt) for _ in vs]
            stream = torch.cuda.current_stream().cuda_stream
            alpha, beta = (1.5, 0.5) if with_c else (1.0, 0.0)

            def call(i):
                _, lib, force = vs[i]
                os.environ["GEMM_TN_FORCE"] = force
                st = lib.gemm_tn_ex(
                    b, M, N, K, alpha, A.data_ptr(), 0, K, M * K,
                    B.data_ptr(), 0, K, N * K, beta,
                    C.data_ptr() if with_c else None, N, M * N,
                    Ds[i].data_ptr(), N, M * N, 1 if f32_out else 0, stream)
                if st != 0:
                    raise SystemExit(f"{vs[i][0]} {tok}: status {st}")

            times = [[] for _ in vs]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            for i in range(len(vs)):
                for _ in range(3):
                    call(i)
            torch.cuda.synchronize()
            for r in range(rounds):
                order = range(len(vs)) if r % 2 == 0 else \
                    reversed(range(len(vs)))
                for i in order:
                    call(i)
                    call(i)
                    e0.record()
                    for _ in range(burst):
                        call(i)
                    e1.record()
                    e1.synchronize()
                    times[i].append(e0.elapsed_time(e1) * 1e3 / burst)
            print(json.dumps({
                "shape": tok, "rounds": rounds, "burst": burst,
                "bitwise_same": all(torch.equal(Ds[0], d) for d in Ds[1:]),
                "median_us": {v[0]: round(statistics.median(t), 2)
                              for v, t in zip(vs, times)},
                "min_us": {v[0]: round(min(t), 2)
                           for v, t in zip(vs, times)}}), flush=True)
    finally:
        if old is None:
            os.environ.pop("GEMM_TN_FORCE", None)
        else:
            os.environ["GEMM_TN_FORCE"] = old


def summarize_plan_grid(path):
    """Markdown table of a --plan-grid run: per shape the planner's choice
    and the fastest choice, each with its time, and their ratio.  The
    planner's time is the grid's for the same choice, or its own run's
    where the grid has no such choice (the grid runs whole tiles without a
    tail split)."""
    rows, ratios = [], []
    for line in open(path):
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        best = min(r["choices"], key=lambda c: c[2])
        p = r["planner"]
        tail = p.get("tail_rows", 0)
        own = [c for c in r["choices"] if c[0] == p["tile"] and
               c[1] == p["split"]] if not tail else []
        t = own[0][2] if own else p["us"]
        ratios.append(t / best[2])
        b, M, N, K = r["shape"]
        lay = r.get("layouts", [0, 0])
        shape = f"{b}x{M}x{N}x{K}" + ("" if lay == [0, 0] else
                                      f" @{lay[0]}.{lay[1]}")
        name = f"{p['tile']} / {p['split']}" + (
            f" + tail {tail} x {p['tail_split']}" if tail else "")
        rows.append(f"| {shape} | {name} | "
                    f"{t:.2f} | {best[0]} / {best[1]} | {best[2]:.2f} | "
                    f"{t / best[2]:.3f} |")
    out = ["| batch x M x N x K | planner: tile / split | us | fastest: "
           "tile / split | us | ratio |", "|---|---|---|---|---|---|"]
    out += rows
    if ratios:
        out.append(f"\nplanner / fastest: mean "
                   f"{sum(ratios) / len(ratios):.3f}, max {max(ratios):.3f} "
                   f"over {len(ratios)} shapes")
    return "\n".join(out)


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


def trace_signatures(w):
    """(kernel name part, Grid_Size_X, Workgroup_Size_X) of every kernel one
    call of workload w launches, from the plan describe() reports: the tile
    kernel (64 threads per wave of the plan's waves), the split-K
    reduction, and for a tail split the tail rows' kernel and reduction.
    A problem within one k-tile runs the persistent one-k kernel alone."""
    kv = dict(x.split("=", 1) for x in describe(w).split())
    if kv.get("sched") == "persistent-onek":
        return [("gemm_onek_kernel", int(kv["grid"]) * 256, 256)]
    bm = int(kv["tile"].split("x")[0])
    wm, wn = (int(x) for x in kv["waves"].split("x"))
    wg = 64 * wm * wn

    def reduce_sig(rows):
        work = w.batch * rows * ((w.N + 3) // 4)
        return ("splitk_reduce", (work + 255) // 256 * 256, 256)

    # the tile's edge is in the (mangled) kernel name: launches of two tiles
    # may agree in grid and workgroup size (256 workgroups of 256 threads)
    part = f"gemm_tn_kernelILi{bm}ELi{bm}E"
    sigs = [(part, int(kv["grid"]) * wg, wg)]
    if int(kv["split"]) > 1:
        sigs.append(reduce_sig(w.M))
    tail_rows = int(kv["tail_rows"])
    if tail_rows > 0:
        sigs.append((part, int(kv["tail_grid"]) * wg, wg))
        sigs.append(reduce_sig(w.M - (-(-w.M // bm) - tail_rows) * bm))
    return sigs


def _name_has(part, name):
    """Whether a kernel name from a trace holds `part`, which names a tile
    kernel in its mangled form (gemm_tn_kernelILi256ELi256E): rocprofv3
    reports some names demangled (gemm_tn_kernel<256, 256, ...>)."""
    if part in name:
        return True
    m = re.fullmatch(r"(\w+?)ILi(\d+)ELi(\d+)E", part)
    return bool(m) and f"{m.group(1)}<{m.group(2)}, {m.group(3)}, " in name


def summarize_trace_all(csv_path, bench_jsonl=None):
    """Markdown table of the kernel times of every configuration in one
    rocprofv3 kernel trace (a --all run): each kernel of a call is found by
    its signature (trace_signatures), and a call's time is the sum of its
    kernels' medians.  With the run's stdout, the HIP-event time per call
    and the oracle's time are set beside them."""
    import csv
    import statistics
    import seeded_inputs as si
    rows = list(csv.DictReader(open(csv_path)))
    recs = {}
    if bench_jsonl:
        for line in open(bench_jsonl):
            line = line.strip()
            if line.startswith("{"):
                r = json.loads(line)
                if r.get("record") == "config":
                    recs[r["workload"]] = r
    out = ["| config | kernels (grid threads) | launches | kernel median "
           "us | min us | TFLOP/s | % MFMA peak | GB/s | % HBM | HIP events "
           "us per call | oracle s (threads) | parity float / int |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in CONFIGS:
        w = si.workload_shape(name)
        med = mins = 0.0
        launches = []
        for part, grid, wg in trace_signatures(w):
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                 for r in rows
                 if _name_has(part, r["Kernel_Name"])
                 and int(r["Grid_Size_X"]) == grid
                 and int(r["Workgroup_Size_X"]) == wg]
            if not d:
                raise SystemExit(f"{name}: no {part} dispatch of grid {grid}")
            med += statistics.median(d)
            mins += min(d)
            launches.append(f"{part} ({grid})")
            n = len(d)
        us = med / 1e3
        rec = recs.get(name, {})
        cb = rec.get("cpu_baseline", {})
        par = rec.get("parity", {})
        out.append(
            f"| {name} | {', '.join(launches)} | {n} | {us:.2f} | "
            f"{mins / 1e3:.2f} | {w.flops / us / 1e6:.1f} | "
            f"{100 * w.flops / us / 1e6 / PEAK_F16_MFMA_TFLOPS:.2f} | "
            f"{w.algorithmic_bytes / us / 1e3:.0f} | "
            f"{100 * w.algorithmic_bytes / us / 1e3 / PEAK_HBM_GBS:.1f} | "
            f"{rec.get('us_per_call', '-')} | "
            f"{cb.get('seconds', '-')} ({cb.get('cores', '-')}) | "
            f"{par.get('float_within_tolerance', '-')} / "
            f"{par.get('integer_bit_exact', '-')} |")
    return "\n".join(out)


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


def _host_cpus():
    """(threads the oracle uses, CPUs this process may run on, CPUs the
    host has).  The oracle's threads are capped at 16, the CPU share the
    measurement host grants one GPU."""
    import oracle
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return oracle.default_threads(), affinity, os.cpu_count() or 1


def oracle_full_check(w, d, exact):
    """The oracle over every output of w, in blocks of 1024 flattened rows,
    checked against the GPU result d (tolerance, or bit for bit with
    exact).  Returns (seconds spent in the oracle, threads, passed, the
    worst block's result text)."""
    import oracle
    threads = oracle.default_threads()
    flat = np.asarray(d).reshape(w.batch * w.M, w.N)
    spent, ok, worst = 0.0, True, ""
    for r0 in range(0, w.batch * w.M, 1024):
        r1 = min(r0 + 1024, w.batch * w.M)
        t = time.perf_counter()
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C, rows=(r0, r1),
                             threads=threads)
        spent += time.perf_counter() - t
        res = (oracle.check_exact(flat[r0:r1], ref, w.out_dtype) if exact
               else oracle.check(flat[r0:r1], ref, w.K, w.out_dtype))
        if not res.ok or not worst:
            worst = str(res)
        ok = ok and res.ok
    return spent, threads, ok, worst


def roofline_of(w, sec, traffic=None):
    """The workload's bound by arithmetic intensity, and both fractions."""
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
    roof["traffic"] = round(traffic["bytes_per_launch"]) if traffic else None
    return tflops, gbs, roof


# The configurations of the study: the small square product, 1024^3 with
# C, the 4096^3 headline, the two ragged shapes and the batched score product.
CONFIGS = ("c1_256", "c2_1024", "c3_4096", "c4a_ragged", "c4b_skinny",
           "c5_qk")


def config_record(name, steps, warmup, cpu=True):
    """One JSON record for one configuration: GPU time per call (HIP events
    over `steps` back-to-back calls), TFLOP/s and GB/s with both roofline
    fractions, and, with cpu, the oracle over every output on the host's
    cores (its time is the CPU baseline; its results check the GPU's, in
    float within tolerance and, for the integer variant, bit for bit)."""
    import dense_gemm_fp16_amd as g
    import seeded_inputs as si
    w = si.workload(name)
    sec, d = time_workload(w, steps, warmup, return_output=True)
    gsec = time_workload_graph(w, steps, warmup)
    tflops, gbs, roof = roofline_of(w, sec, load_traffic(name))
    rec = {"record": "config", "workload": name,
           "shape": {"batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
                     "alpha": w.alpha, "beta": w.beta, "out": w.out_dtype},
           "kernel": describe(w), "steps": steps, "warmup": warmup,
           "us_per_call": round(sec * 1e6, 3),
           "us_per_call_graph": round(gsec * 1e6, 3),
           "tflops_graph": round(w.flops / gsec / 1e12, 2),
           "gbs_graph": round(w.algorithmic_bytes / gsec / 1e9, 1),
           "tflops": round(tflops, 2),
           "pct_mfma_peak": round(100 * tflops / PEAK_F16_MFMA_TFLOPS, 2),
           "gbs": round(gbs, 1),
           "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
           "roofline": roof}
    if cpu:
        spent, threads, ok, worst = oracle_full_check(w, d, exact=False)
        wi = si.workload(name, int_values=True)
        di = run_once(wi)
        _, _, ok_i, worst_i = oracle_full_check(wi, di, exact=True)
        used, affinity, host = _host_cpus()
        rec["parity"] = {"float_within_tolerance": ok, "float": worst,
                         "integer_bit_exact": ok_i, "integer": worst_i,
                         "elements": w.batch * w.M * w.N}
        rec["cpu_baseline"] = {
            "value": w.flops / spent / 1e12, "unit": "TFLOP/s",
            "cores": threads, "affinity_cpus": affinity, "host_cpus": host,
            "kind": "oracle", "seconds": round(spent, 3),
            "sample": f"every output ({w.batch}x{w.M}x{w.N}x{w.K}, fp64 "
                      f"sequential k-sum) on {threads} threads of "
                      f"{_cpu_model()}; {w.flops / spent / 1e9:.1f} GFLOP/s",
            "gpu_speedup": round(spent / sec, 1)}
    return rec


def run_once(w):
    """One call of workload w; its output on the host."""
    import torch
    import dense_gemm_fp16_amd as g
    A, B, C, D = _device_inputs(w, torch)
    g.gemm_tn(A, B, w.alpha, w.beta, C, out=D)
    torch.cuda.synchronize()
    return D.cpu().numpy()


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
    _, affinity, host = _host_cpus()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "affinity_cpus": affinity, "host_cpus": host, "kind": "oracle",
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


def extras_table(a):
    """stderr table of the workloads beyond the study's configurations: the
    tail-split shape, the attention forward pass, the fp16-accumulating
    GEMM and the transposes (HIP events, a steps x back-to-back calls)."""
    import seeded_inputs as si
    print(f"{'workload':<14}{'kernel':<60}{'us':>10}{'TFLOP/s':>10}"
          f"{'%peak':>8}{'GB/s':>9}{'%HBM':>7}", file=sys.stderr)
    for name in si.WORKLOADS:
        if name in CONFIGS:
            continue
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


def gemm_workload(name):
    """A workload of the study by name, or `tn_MxNxK`: an M x N x K product
    of seeded uniform [-1, 1] fp16 operands with fp16 D, alpha 1, beta 0
    (the 4096^3 recipe at other sizes, for sweeps)."""
    import re
    import seeded_inputs as si
    m = re.fullmatch(r"tn_(\d+)x(\d+)x(\d+)", name)
    if m is None:
        return si.workload(name)
    M, N, K = (int(x) for x in m.groups())
    return si.build(name, 1, M, N, K, 1.0, 0.0, "f16", "uniform",
                    si.SEED_BASE + 0x300)


def describe(w):
    import dense_gemm_fp16_amd as g
    return g.describe(w.batch, w.M, w.N, w.K, w.beta, w.out_dtype, True)


def main():
    a = _args()
    if a.summarize_trace:
        print(json.dumps(summarize_trace(a.summarize_trace, a.workload)))
        return
    if a.summarize_trace_all:
        print(summarize_trace_all(*a.summarize_trace_all[:2]))
        return
    if a.summarize_plan_grid:
        print(summarize_plan_grid(a.summarize_plan_grid))
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
    if a.ab:
        ab_compare(a.ab, a.ab_shapes, a.ab_rounds)
        return
    if a.plan_grid:
        plan_grid(a.plan_grid)
        return
    if a.workload in TRANSPOSES:
        transpose_main(a)
        return
    if a.workload in ATTENTIONS:
        attention_main(a)
        return
    if a.workload in F16ACCS:
        f16acc_main(a)
        return
    if a.all:
        # one record per configuration of the study, each with its oracle
        for name in CONFIGS:
            print(json.dumps(config_record(name, a.steps, a.warmup,
                                           cpu=not a.no_cpu_baseline)),
                  flush=True)
    if a.extras:
        extras_table(a)
    w = gemm_workload(a.workload)
    sec = time_workload(w, a.steps, a.warmup)
    tflops, gbs, roof = roofline_of(w, sec, load_traffic(a.workload))
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
    if a.cold:
        cs = time_workload_cold(w, a.steps)
        line["cold"] = {"ms_per_call": round(cs * 1e3, 5),
                        "tflops": round(w.flops / cs / 1e12, 2),
                        "flush_mib": 512}
    if a.vendor and w.alpha == 1.0 and w.beta == 0.0:
        v = time_vendor_interleaved(w)
        line["vendor_context"] = {
            "us_per_call": {k: round(t * 1e6, 2) for k, t in v.items()},
            "tflops": {k: round(w.flops / t / 1e12, 1) for k, t in v.items()},
            "method": "6 interleaved bursts of 10 calls, medians"}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
