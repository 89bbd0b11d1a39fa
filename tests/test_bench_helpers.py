"""bench.py's host-side helpers, on the CPU: the kernel fingerprint that
guards the stored traffic figures, the per-call kernel-trace summary, the
HBM-traffic summary from two counter runs, and the refusal of more than one
GPU."""
import csv
import re
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_lines():
    src = ("int a; // note\n\n/* block\n comment */ int b;\n"
           "  // whole line\nint c = 1; /* x */ int d;\n")
    assert bench._code_only(src) == "int a;\n int b;\nint c = 1;  int d;"
    # a comment edit leaves the code, and so the fingerprint, alone
    assert bench._code_only(src.replace("note", "other words")) == \
        bench._code_only(src)
    assert bench._code_only(src.replace("int c = 1", "int c = 2")) != \
        bench._code_only(src)


def test_fingerprints_differ_between_kernels():
    fps = {w: bench.kernel_fingerprint(w)
           for w in ("c3_4096", "attn_64x1024", "transpose_8192",
                     "f16acc_4096")}
    assert len(set(fps.values())) == 4
    assert all(len(f) == 16 for f in fps.values())


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for name, t0, t1 in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t0,
                        "End_Timestamp": t1})


def test_summarize_trace_sums_the_kernels_of_a_call(tmp_path):
    gemm = "void gtn::gemm_tn_kernel<64, 64, 64, 2, 2, 4, 0, float, true>"
    red = "void gtn::splitk_reduce_kernel<float, true>"
    rows = [(gemm, 0, 100), (red, 100, 130), ("other_kernel", 130, 500),
            (gemm, 1000, 1110), (red, 1110, 1140),
            (gemm, 2000, 2090), (red, 2090, 2130)]
    p = tmp_path / "t_kernel_trace.csv"
    _write_trace(p, rows)
    t = bench.summarize_trace(str(p), "c4b_skinny")
    assert t["calls"] == 3 and t["kernels_per_call"] == 2.0
    assert (t["min_ns"], t["median_ns"], t["max_ns"]) == (130, 130, 140)


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": v})


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    k = "_ZN3gtn14gemm_tn_kernelILi256E"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the 256 MiB copy reads half as much as it moves in FETCH_SIZE units
    _write_pmc(fetch, "FETCH_SIZE", [(copy, 131072.0), (k, 1000.0),
                                     (k, 1002.0), (k, 998.0)])
    _write_pmc(write, "WRITE_SIZE", [(copy, 262144.0), (k, 500.0),
                                     (k, 500.0), (k, 500.0)])
    t = bench.summarize_pmc(str(fetch), str(write), "c3_4096", 256)
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["fetch_bytes"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert t["write_bytes"] == pytest.approx(500.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx((2000.0 + 500.0) * 1024)
    assert t["fingerprint"] == bench.kernel_fingerprint("c3_4096")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_summarize_trace_all_finds_each_configuration(tmp_path):
    """Each configuration's kernels are picked out of one mixed trace by
    name, grid and workgroup size; a split-K call adds its reduction; the
    run's stdout records are set beside the kernel times."""
    import seeded_inputs as si
    rows, t = [], 0
    for i, name in enumerate(bench.CONFIGS):
        for part, grid, wg in bench.trace_signatures(si.workload_shape(name)):
            for rep in range(3):
                dur = 1000 * (i + 1) + 10 * rep + (7 if "reduce" in part
                                                    else 0)
                # the 256 tile's name mangled, the others demangled, as
                # rocprofv3 reports them within one trace
                name = (part if "ILi256E" in part
                        else re.sub(r"ILi(\d+)ELi(\d+)E$", r"<\1, \2, ...>",
                                    part))
                rows.append({"Kernel_Name": f"void gtn::{name}<...>",
                             "Start_Timestamp": t, "End_Timestamp": t + dur,
                             "Grid_Size_X": grid, "Workgroup_Size_X": wg})
                t += dur + 5
    p = tmp_path / "k_kernel_trace.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    j = tmp_path / "b.jsonl"
    j.write_text('{"record": "config", "workload": "c4b_skinny", '
                 '"us_per_call": 12.5, "cpu_baseline": {"seconds": 0.7, '
                 '"cores": 16}, "parity": {"float_within_tolerance": true, '
                 '"integer_bit_exact": true}}\n{"metric": "x"}\n')
    table = bench.summarize_trace_all(str(p), str(j)).splitlines()
    assert len(table) == 2 + len(bench.CONFIGS)
    by = {r.split("|")[1].strip(): r.split("|") for r in table[2:]}
    # c3, the third configuration: median of 3000, 3010, 3020 ns
    assert by["c3_4096"][4].strip() == "3.01"
    # c4b: gemm median 5010 + reduction median 5017
    assert by["c4b_skinny"][4].strip() == "10.03"
    assert "12.5" in by["c4b_skinny"][10] and "0.7 (16)" in by["c4b_skinny"][11]
    assert by["c1_256"][10].strip() == "-"


def test_summarize_plan_grid_compares_the_planner_with_the_fastest(tmp_path):
    import json
    p = tmp_path / "grid.jsonl"
    p.write_text("\n".join([
        "not a record",
        json.dumps({"shape": [1, 1024, 1024, 8192], "rounds": 4, "burst": 10,
                    "planner": {"tile": 128, "split": 4, "us": 29.3},
                    "choices": [[64, 1, 37.9], [128, 4, 29.0],
                                [256, 8, 31.0]]}),
        json.dumps({"shape": [2, 512, 512, 4096], "rounds": 4, "burst": 10,
                    "planner": {"tile": 64, "split": 1, "us": 20.0},
                    "choices": [[64, 1, 20.0], [64, 2, 16.0]]})]) + "\n")
    md = bench.summarize_plan_grid(str(p))
    lines = md.splitlines()
    # the planner's time is the grid's time of the same choice
    assert "| 1x1024x1024x8192 | 128 / 4 | 29.00 | 128 / 4 | 29.00 | 1.000 |" \
        in lines
    assert "| 2x512x512x4096 | 64 / 1 | 20.00 | 64 / 2 | 16.00 | 1.250 |" \
        in lines
    assert lines[-1] == ("planner / fastest: mean 1.125, max 1.250 over 2 "
                         "shapes")
    # a plan with a tail split is not among the grid's whole-tile choices:
    # the planner's own run counts
    p.write_text(json.dumps({
        "shape": [1, 4352, 4352, 4096], "rounds": 4, "burst": 10,
        "planner": {"tile": 256, "split": 1, "tail_rows": 2, "tail_split": 4,
                    "us": 134.0},
        "choices": [[256, 1, 170.0], [128, 1, 155.0]]}) + "\n")
    lines = bench.summarize_plan_grid(str(p)).splitlines()
    assert "| 1x4352x4352x4096 | 256 / 1 + tail 2 x 4 | 134.00 | 128 / 1 | " \
        "155.00 | 0.865 |" in lines


def test_summarize_plan_grid_names_the_layouts(tmp_path):
    import json
    p = tmp_path / "grid.jsonl"
    p.write_text(json.dumps({
        "shape": [1, 512, 512, 1024], "layouts": [1, 0], "rounds": 4,
        "burst": 10, "planner": {"tile": 64, "split": 1, "tail_rows": 0,
                                 "tail_split": 1, "us": 6.0},
        "choices": [[64, 1, 6.0], [128, 1, 7.5]]}) + "\n")
    lines = bench.summarize_plan_grid(str(p)).splitlines()
    assert "| 1x512x512x1024 @1.0 | 64 / 1 | 6.00 | 64 / 1 | 6.00 | 1.000 |" \
        in lines


def test_ab_mode_is_offered():
    """`--ab` (builds of the library timed against each other in one
    process) is part of the command line, with its shape syntax."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    assert "--ab LIB[@FORCE]" in r.stdout and "--ab-shapes" in r.stdout
    assert callable(bench.ab_compare)
