"""The C-ABI library on the CPU: it loads, exports what include/gemm_tn.h
declares, rejects bad arguments before touching the GPU, and plans the
expected kernel configurations.  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

g = pytest.importorskip("dense_gemm_fp16_amd")

OK, INVALID, UNSUPPORTED = g.OK, g.ERR_INVALID_ARG, g.ERR_UNSUPPORTED
F16, F32 = g.GEMM_TN_F16, g.GEMM_TN_F32
# Dummy non-NULL addresses: argument checks never dereference them.
P = ctypes.c_void_p(0x1000)
NULL = None
S = ctypes.c_void_p(0)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^(?:int|const char \*)\s*(\w+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(g.EXPORTS)
    lib = g.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert g.version() == (1, 2)
    assert g.status_string(OK) == "ok"
    assert g.status_string(INVALID) == "invalid argument"
    assert g.status_string(99) == "unknown status"


def call(M, N, K, A=P, B=P, beta=0.0, C=NULL, D=P, dt=F16, alpha=1.0):
    return g.gemm_tn_raw(M, N, K, alpha, A, B, beta, C, D, dt, S)


def batched(batch, M, N, K, sA, sB, sC, sD, beta=0.0, C=NULL, dt=F32):
    return g.gemm_tn_strided_batched(batch, M, N, K, 1.0, P, sA, P, sB, beta,
                                     C, sC, P, sD, dt, S)


@pytest.mark.parametrize("args,status", [
    (dict(M=-1, N=4, K=4), INVALID),
    (dict(M=4, N=-1, K=4), INVALID),
    (dict(M=4, N=4, K=-1), INVALID),
    (dict(M=4, N=4, K=4, dt=2), INVALID),
    (dict(M=4, N=4, K=4, dt=-1), INVALID),
    (dict(M=4, N=4, K=4, D=NULL), INVALID),
    (dict(M=4, N=4, K=4, A=NULL), INVALID),
    (dict(M=4, N=4, K=4, B=NULL), INVALID),
    (dict(M=4, N=4, K=4, beta=0.5, C=NULL), INVALID),
    (dict(M=2 ** 40, N=2 ** 40, K=4), INVALID),         # M*N overflows bytes
    (dict(M=4, N=4, K=2 ** 21 + 8), UNSUPPORTED),
    (dict(M=4, N=2 ** 20 + 4, K=8), UNSUPPORTED),
    (dict(M=2 ** 31, N=4, K=8), UNSUPPORTED),
    # nothing to compute: OK without touching the GPU, NULLs allowed
    (dict(M=0, N=4, K=4, A=NULL, B=NULL, D=NULL), OK),
    (dict(M=4, N=0, K=4, A=NULL, B=NULL, D=NULL), OK),
])
def test_argument_checks(args, status):
    assert call(**args) == status


def test_batched_argument_checks():
    # overlapping D batches
    assert batched(2, 4, 4, 4, 16, 16, 16, 15) == INVALID
    # negative strides
    assert batched(2, 4, 4, 4, -16, 16, 16, 16) == INVALID
    assert batched(-1, 4, 4, 4, 16, 16, 16, 16) == INVALID
    # batch 0: no-op
    assert batched(0, 4, 4, 4, 16, 16, 16, 16) == OK
    # stride * batch overflow
    assert batched(2 ** 40, 4, 4, 4, 2 ** 40, 16, 16, 16) == INVALID


def ex(batch, M, N, K, lda, ldb, ldc, ldd, sA=0, sB=0, sC=0, sD=0,
       beta=0.0, C=NULL, dt=F32):
    return g.gemm_tn_ex(batch, M, N, K, 1.0, P, lda, sA, P, ldb, sB, beta, C,
                        ldc, sC, P, ldd, sD, dt, S)


@pytest.mark.parametrize("args,status", [
    ((1, 4, 4, 8, 7, 8, 4, 4), INVALID),                  # lda < K
    ((1, 4, 4, 8, 8, 7, 4, 4), INVALID),                  # ldb < K
    ((1, 4, 4, 8, 8, 8, 4, 3), INVALID),                  # ldd < N
    ((1, 4, 4, 8, 8, 8, 3, 4, 0, 0, 0, 0, 0.5, P), INVALID),  # ldc < N
    ((1, 4, 4, 8, 2 ** 21 + 8, 8, 4, 4), UNSUPPORTED),    # lda too large
    ((1, 4, 4, 8, 8, 8, 4, 2 ** 20 + 4), UNSUPPORTED),    # ldd too large
    # batches of D: extent (M - 1) * ldd + N = 3 * 10 + 4 = 34
    ((2, 4, 4, 8, 8, 8, 4, 10, 0, 0, 0, 33), INVALID),
    ((1, 2 ** 62, 4, 8, 2 ** 21, 8, 4, 4), INVALID),      # A extent overflows
])
def test_leading_dimension_checks(args, status):
    assert ex(*args) == status


@pytest.mark.parametrize("args", [
    (1, 4, 4, 8, (8, 8, 4, 4), (0, 0, 0, 0)),             # packed
    (1, 4, 4, 8, (16, 9, 4, 7), (0, 0, 0, 0)),            # padded rows
    (2, 4, 4, 8, (8, 8, 4, 10), (32, 32, 16, 34)),        # D batches touch
    (3, 4, 4, 8, (8, 8, 4, 4), (0, 0, 16, 16)),           # A, B broadcast
])
def test_leading_dimensions_accepted(args):
    batch, M, N, K, lds, strides = args
    assert "error" not in g.describe(batch, M, N, K, lds=lds,
                                     strides=strides)


def ex_layout(layout_a, layout_b, M, N, K, lda, ldb):
    return g.gemm_tn_ex(1, M, N, K, 1.0, P, lda, 0, P, ldb, 0, 0.0, NULL, N,
                        0, P, N, 0, F32, S, layout_a, layout_b)


ROW_K, ROW_MN = g.GEMM_TN_ROW_K, g.GEMM_TN_ROW_MN


@pytest.mark.parametrize("args,status", [
    ((2, ROW_K, 4, 6, 8, 8, 8), INVALID),        # unknown layout value
    ((ROW_K, -1, 4, 6, 8, 8, 8), INVALID),
    ((ROW_MN, ROW_K, 4, 6, 8, 3, 8), INVALID),   # A stored K x M: lda >= M
    ((ROW_K, ROW_MN, 4, 6, 8, 8, 5), INVALID),   # B stored K x N: ldb >= N
    ((ROW_MN, ROW_K, 2 ** 21 + 8, 6, 8, 2 ** 21 + 8, 8), UNSUPPORTED),
])
def test_layout_checks(args, status):
    assert ex_layout(*args) == status


@pytest.mark.parametrize("la,lb", [(ROW_K, ROW_MN), (ROW_MN, ROW_K),
                                   (ROW_MN, ROW_MN)])
def test_operands_stored_along_m_or_n_are_planned(la, lb):
    # lda >= M for A stored K x M (here M = 300 > K = 64 is fine)
    # rows of 8-element multiples: direct loader with transposing LDS
    # reads, on the 256-wide tile for either or both operands
    p = describe(1, 4096, 4096, 4096, layouts=(la, lb))
    assert p["loader"] == "direct"
    assert p["tile"].startswith("256x256")
    assert (p["a_along"], p["b_along"]) == ("m" if la else "k",
                                            "n" if lb else "k")
    # M = 300 is not a multiple of 8: an A stored along M needs the element
    # loader (its last 16-byte chunk would read past row end)
    p = describe(1, 300, 200, 64, layouts=(la, lb))
    assert p["loader"] == ("elem" if la else "direct")
    # the element loader has no kernels for these layouts on 256 x 256
    p = describe(1, 4000, 4000, 4096, layouts=(la, lb), lds=(
        4003 if la else 4096, 4003 if lb else 4096, 4000, 4000))
    assert p["loader"] == "elem" and p["tile"].startswith("128x128")
    # a row stride that only covers K is too short for a row of M / N
    short = (64, 64, 200, 200)
    assert g.describe(1, 300, 200, 64, layouts=(la, lb), lds=short) \
        == "error:1"


def test_leading_dimensions_choose_the_loaders():
    # rows of A padded to a multiple of 8 elements: vector loader kept
    p = describe(1, 512, 512, 512, lds=(520, 512, 512, 512))
    assert p["loader"] == "direct"
    # an odd row stride rules out 16-byte loads
    assert describe(1, 512, 512, 512, lds=(513, 512, 512, 512))["loader"] \
        == "elem"
    # D rows of 516 fp16 (1032 bytes) are not 16-byte aligned: element stores
    assert describe(1, 512, 512, 512, lds=(512, 512, 512, 516))["vec_out"] \
        == "0"
    assert describe(1, 512, 512, 512, lds=(512, 512, 512, 520))["vec_out"] \
        == "1"


def describe(batch, M, N, K, beta=0.0, out="f16", aligned=True, lds=None,
             layouts=(0, 0)):
    d = g.describe(batch, M, N, K, beta, out, aligned, lds=lds,
                   layouts=layouts)
    return dict(kv.split("=") for kv in d.split()) if "=" in d else d


def test_plans_for_the_workloads():
    # 4096^3: one 256x256 tile per CU, vector loader, no split, on four
    # waves (one per SIMD)
    p = describe(1, 4096, 4096, 4096)
    assert p["tile"].startswith("256x256x") and p["split"] == "1"
    assert p["grid"] == "256" and p["loader"] != "elem"
    assert (p["waves"], p["sched"]) == ("2x2", "four-wave")
    # 1024^3 and the ragged 1000x1030x1000: 64x64 tiles, enough of them
    # (whole-K problems on the 64 tile take its two-stage ring of 128-deep
    # k-tiles)
    p = describe(1, 1024, 1024, 1024, 0.5, "f32")
    assert p["tile"] == "64x64x128" and p["stages"] == "2"
    p = describe(1, 1000, 1030, 1000, 0.0, "f32")
    assert p["tile"] == "64x64x128" and p["vec_out"] == "0"   # N % 4 != 0
    assert p["stages"] == "2"
    # skinny 128x4096x8192: split-K, slices on the four-stage ring
    p = describe(1, 128, 4096, 8192, 0.0, "f32")
    assert int(p["split"]) > 1 and int(p["k_split"]) % 64 == 0
    assert p["tile"] == "64x64x64" and p["stages"] == "4"
    assert int(p["split"]) * int(p["k_split"]) >= 8192
    # batched QK^T: 64 x (1024 x 1024 x 64): K within one k-tile, 4096
    # tiles of 128 walked by one persistent workgroup per CU
    p = describe(64, 1024, 1024, 64, 0.0, "f32")
    assert p["tile"].startswith("128x128x") and int(p["grid"]) == 256
    assert p["sched"] == "persistent-onek"
    # too few tiles, C rows off 16 bytes, or K past one k-tile: not it
    assert describe(1, 1024, 1024, 64)["sched"] != "persistent-onek"
    assert describe(64, 1024, 1030, 64, 0.0, "f32")["sched"] != \
        "persistent-onek"
    assert describe(64, 1024, 1024, 72, 0.0, "f32")["sched"] != \
        "persistent-onek"
    # K not a multiple of 8, or misaligned: element loader
    assert describe(1, 100, 100, 33)["loader"] == "elem"
    assert describe(1, 128, 128, 64, aligned=False)["loader"] == "elem"
    assert describe(1, 0, 5, 5) == "noop"


def test_tail_split_plans(monkeypatch):
    # 17 x 17 tiles of 256 on 256 CUs: one wave plus 33 tiles; the last two
    # tile rows (34 tiles) split round(sqrt(9 * 64 / 34)) = 4 ways (a wave
    # would hold 7), the rest one wave of whole tiles
    p = describe(1, 4352, 4352, 4096)
    assert p["tile"].startswith("256x256x")
    assert (p["tail_rows"], p["tail_split"], p["grid"], p["tail_grid"]) == \
        ("2", "4", "255", "136")
    assert int(p["tail_k_split"]) * 4 >= 4096
    # 72 tail tiles: round(sqrt(9 * 64 / 72)) = 3, as many as a wave holds
    p = describe(1, 6144, 6144, 4096)
    assert (p["tail_rows"], p["tail_split"]) == ("3", "3")
    # a longer K takes more slices: round(sqrt(9 * 128 / 34)) = 6
    assert describe(1, 4352, 4352, 8192)["tail_split"] == "6"
    # whole waves, or a tail of more than half a wave: no tail split
    for shape in [(1, 4096, 4096, 4096), (1, 8192, 8192, 8192),
                  (1, 5000, 5000, 5000), (1, 1000, 1030, 1000),
                  (64, 1024, 1024, 64), (1, 128, 4096, 8192)]:
        assert describe(*shape)["tail_rows"] == "0", shape
    # tiles with two workgroups per CU take no tail split by themselves
    p = describe(1, 3072, 3072, 448)
    assert p["tile"].startswith("128x128x") and p["tail_rows"] == "0"
    # too short a K for two slices of four k-tiles: no tail split
    assert describe(1, 4352, 4352, 448)["tail_rows"] == "0"
    monkeypatch.setenv("GEMM_TN_FORCE", "tail=0")
    assert describe(1, 4352, 4352, 4096)["tail_rows"] == "0"
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=64,tail=2,tail_split=3")
    p = describe(2, 600, 260, 1088)
    assert (p["tail_rows"], p["tail_split"]) == ("2", "3")
    assert p["grid"] == str((10 - 2) * 5 * 2)
    assert p["tail_grid"] == str(2 * 5 * 2 * 3)


def _plan(shape, out="f16"):
    p = describe(*shape, 0.0, out)
    return int(p["tile"].split("x")[0]), int(p["split"])


def test_cost_model_plans(monkeypatch):
    """K of 512 or more with 16-byte loads: the tile and split-K factor (and,
    on the 256 tile, the tail split) of least estimated time.  Each pin is
    the fastest of the choices timed on that shape."""
    # 144 or 225 tiles of 256: one partial wave of whole tiles, not the
    # 128 tile (3072^2 x 4096: 76 against 93 us) nor a split of the 256
    # tile into more workgroups than CUs (3840^2 x 4096: 90 against 150 us)
    assert _plan((1, 3072, 3072, 4096)) == (256, 1)
    assert _plan((1, 3840, 3840, 4096)) == (256, 1)
    # 64 tiles of 256 over K = 8192: four slices fill one wave
    assert _plan((1, 2048, 2048, 8192)) == (256, 4)
    # 2048^2 x 4096: 256 tiles of 128, one per CU, no split
    assert _plan((1, 2048, 2048, 4096)) == (128, 1)
    # 144 tiles of 128 in three slices (51.5 against 81 us on 64 tiles)
    assert _plan((1, 1536, 1536, 8192)) == (128, 3)
    # 144 tiles of 64 in three slices
    assert _plan((1, 768, 768, 4096)) == (64, 3)
    # K of 1024: 144 whole tiles of 256 (25.2 against 28.0 us on the 128
    # tile); 512^2 x 1024 unsplit (6.0 against 9.5 us in four slices)
    assert _plan((1, 3072, 3072, 1024)) == (256, 1)
    assert _plan((1, 512, 512, 1024)) == (64, 1)
    # M below 256: no 256 tile; the skinny workload keeps its 4 slices
    assert _plan((1, 192, 6144, 8192)) == (128, 5)
    assert _plan((1, 128, 4096, 8192), "f32") == (64, 4)
    # a tiny output over the longest K: 256 slices of 8192
    assert _plan((1, 16, 24, 2 ** 21), "f32") == (64, 256)
    # one wave of 256 tiles of 256 (4096^3); 289 tiles: the bottom two tile
    # rows split 4 ways (134 us against 156 on the 128 tile and 170 for
    # whole tiles), unless K is short (4352^2 x 1024: the 128 tile, 45.4
    # against 52.6 us); the six workloads keep their plans
    # (test_plans_for_the_workloads)
    assert _plan((1, 4096, 4096, 4096)) == (256, 1)
    p = describe(1, 4352, 4352, 4096)
    assert (p["tile"][:3], p["tail_rows"], p["tail_split"]) == \
        ("256", "2", "4")
    assert _plan((1, 4352, 4352, 1024)) == (128, 1)
    # K of 512 to 1023 (the fastest timed choice on each)
    assert _plan((1, 1536, 1536, 768)) == (128, 1)
    assert _plan((1, 3000, 3000, 960)) == (256, 1)
    assert _plan((1, 1000, 1030, 1000), "f32") == (64, 1)
    # operands stored along M or N: the same ranking (the 256 tile on eight
    # waves at 3072^2 x 4096: 90.8 us against 108.1 on the 128 tile; 128
    # tile in 3 slices at 1536^2 x 8192: 54.1 against 101.6 on the 64 tile)
    p = describe(1, 3072, 3072, 4096, layouts=(1, 0))
    assert (p["tile"][:3], p["split"], p["sched"]) == \
        ("256", "1", "pingpong-split")
    p = describe(1, 1536, 1536, 8192, layouts=(1, 1))
    assert (p["tile"][:3], p["split"]) == ("128", "3")
    # outside the model: K below 512, an element loader (K % 8 != 0); and
    # any forced tile or split
    assert _plan((1, 3072, 3072, 448)) == (128, 1)
    assert describe(1, 1500, 1700, 4100)["loader"] == "elem"
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=128")
    assert _plan((1, 3072, 3072, 4096)) == (128, 1)
    monkeypatch.setenv("GEMM_TN_FORCE", "split=2")
    assert _plan((1, 3072, 3072, 4096))[1] == 2


def test_split_rule_fills_one_wave():
    """Outside the cost model a split fills one wave of the tile: as many
    slices as the CUs hold workgroups of it (one per CU for the 256 tile,
    two for the others), never more."""
    # 196 tiles of 256 (K % 8 != 0: element loads, no cost model): one wave
    # holds them whole, no split (on TN operands three slices, as the rule
    # once chose, took 142 us against 80)
    p = describe(1, 3584, 3584, 4100)
    assert p["tile"].startswith("256x256x") and p["split"] == "1"
    assert p["loader"] == "elem"
    # 165 tiles of 64 (element loader): 3 slices = 495 workgroups <= 512
    p = describe(1, 700, 900, 4100)
    assert p["tile"].startswith("64x64x") and p["split"] == "3"
    # the skinny workload: 128 tiles of 64, 4 slices = 512
    assert describe(1, 128, 4096, 8192, 0.0, "f32")["split"] == "4"


def test_planned_partials_fit_the_noalloc_scratch():
    """No plan of the planner's own writes more split-K partials than the
    no-allocation entry point's fixed scratch holds, so both entry points
    run the same plan: a split fills at most one wave of 256 x 256 fp32
    tiles, and the cost model skips splits beyond the scratch."""
    limit = g.NOALLOC_SCRATCH_BYTES
    for M in (256, 700, 1024, 1536, 2000, 2304, 3000, 3840, 4352, 6144):
        for N in (256, 1030, 2048, 3333, 4096, 8192):
            for K in (2048, 8192, 65536):
                p = describe(1, M, N, K, 0.0, "f32")
                ws_ld = (N + 3) // 4 * 4
                split, tail = int(p["split"]), int(p["tail_rows"])
                if split > 1:
                    assert split * M * ws_ld * 4 <= limit, (M, N, K, p)
                if tail:
                    bm = int(p["tile"].split("x")[0])
                    tail_m = M - (-(-M // bm) - tail) * bm
                    assert int(p["tail_split"]) * tail_m * ws_ld * 4 <= \
                        limit, (M, N, K, p)


def test_four_wave_plans(monkeypatch):
    # four waves need TN operands, direct loads and 16-byte output rows;
    # otherwise (and with w4=0) the 256 tile runs on eight
    assert describe(1, 4096, 4096, 4096, 0.5, "f32")["sched"] == "four-wave"
    p = describe(1, 4096, 4100, 4096)        # 8200-byte rows: no 16-byte
    assert p["tile"].startswith("256x256x") and p["vec_out"] == "0"
    assert (p["waves"], p["sched"]) == ("2x4", "pingpong-split")
    p = describe(1, 4096, 4096, 4096, layouts=(1, 0))
    assert (p["waves"], p["sched"]) == ("2x4", "pingpong-split")
    monkeypatch.setenv("GEMM_TN_FORCE", "w4=0")
    p = describe(1, 4096, 4096, 4096)
    assert (p["waves"], p["sched"]) == ("2x4", "pingpong-split")
    # split-K slices and the tail split keep four waves
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=256,split=3")
    assert describe(1, 512, 512, 4096)["sched"] == "four-wave"
    monkeypatch.delenv("GEMM_TN_FORCE")
    p = describe(1, 4352, 4352, 4096)
    assert p["tail_rows"] != "0" and p["sched"] == "four-wave"


def test_override_spec(monkeypatch):
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=128,split=2,loader=0,group=2")
    p = describe(1, 512, 512, 1024)
    assert p["tile"].startswith("128x128x") and p["split"] == "2"
    assert p["loader"] == "direct" and p["group_m"] == "2"
    # a vector loader is refused when alignment does not allow it
    p = describe(1, 512, 512, 1000 + 3)
    assert p["loader"] == "elem"


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4), INVALID), ((1, -4, 4), INVALID), ((1, 4, -4), INVALID),
    ((2 ** 40, 2 ** 20, 2 ** 20), INVALID),            # size overflow
    ((1, 2 ** 23 + 4, 8), UNSUPPORTED), ((1, 8, 2 ** 23 + 4), UNSUPPORTED),
    ((0, 4, 4), OK), ((3, 0, 4), OK), ((3, 4, 0), OK),  # nothing to do
])
def test_transpose_argument_checks(args, status):
    batch, M, N = args
    # distinct dummy buffers far apart: the checks never touch them
    assert g.transpose_f32_raw(batch, M, N, ctypes.c_void_p(0x1000),
                               ctypes.c_void_p(0x1000 + 2 ** 62), S) == status


def test_transpose_rejects_overlap_and_null():
    x = ctypes.c_void_p(0x100000)
    assert g.transpose_f32_raw(1, 4, 4, x, ctypes.c_void_p(0x100000 + 60),
                               S) == INVALID          # 64-byte ranges overlap
    assert g.transpose_f32_raw(1, 4, 4, None, x, S) == INVALID
    assert g.transpose_f32_raw(1, 4, 4, x, None, S) == INVALID


def _attn(batch=2, Lq=8, Lk=8, d=64, scale=0.125, o_dtype=F16, lse=None,
          q=0x10000, k=0x20000, v=0x30000, o=0x40000):
    ptr = lambda a: ctypes.c_void_p(a) if a is not None else None
    return g.attention_fwd_raw(batch, Lq, Lk, d, scale, ptr(q), ptr(k),
                               ptr(v), ptr(o), o_dtype, ptr(lse), S)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), INVALID), (dict(Lq=-1), INVALID), (dict(Lk=-1), INVALID),
    (dict(d=-1), INVALID), (dict(o_dtype=7), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(Lk=0), INVALID),                       # softmax over no keys
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID),
    (dict(o=0x10000 + 16), INVALID),             # O overlaps Q
    (dict(o=0x30000 + 2048 - 16), INVALID),      # O overlaps V's tail
    (dict(lse=0x40000 + 8), INVALID),            # lse overlaps O
    (dict(batch=2 ** 40, Lq=2 ** 20), INVALID),  # size overflow
    (dict(d=128), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(Lk=2 ** 23 + 1, k=0x10 ** 12, v=0x20 ** 12, o=0x30 ** 12),
     UNSUPPORTED),
    (dict(q=0x10008), UNSUPPORTED),              # not 16-byte aligned
    (dict(o=0x40004), UNSUPPORTED),
    (dict(lse=0x50002), UNSUPPORTED),
    (dict(batch=0), OK), (dict(Lq=0), OK),       # nothing to do
    (dict(batch=0, Lk=0), OK), (dict(Lq=0, q=None, o=None), OK),
])
def test_attention_argument_checks(kw, status):
    assert _attn(**kw) == status


def _acc(batch=2, M=8, N=8, K=32, sA=None, sB=None, sD=None, a=0x100000,
         b=0x200000, d=0x300000):
    ptr = lambda x: ctypes.c_void_p(x) if x is not None else None
    return g.gemm_tn_f16acc_raw(batch, M, N, K, ptr(a),
                                M * K if sA is None else sA, ptr(b),
                                N * K if sB is None else sB, ptr(d),
                                M * N if sD is None else sD, S)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), INVALID), (dict(M=-1), INVALID), (dict(N=-1), INVALID),
    (dict(K=-1), INVALID), (dict(sA=-1), INVALID), (dict(sD=-8), INVALID),
    (dict(sD=8), INVALID),                      # batches of D overlap
    (dict(sA=8), INVALID),                      # batches of A overlap
    (dict(d=None), INVALID), (dict(a=None), INVALID), (dict(b=None), INVALID),
    (dict(d=0x100000 + 64), INVALID),           # D overlaps A
    (dict(d=0x200000 + 500), INVALID),          # D overlaps B's tail
    (dict(M=2 ** 40, N=2 ** 40), INVALID),      # size overflow
    (dict(K=2 ** 21 + 8, a=0x10 ** 12, b=0x20 ** 12, d=0x30 ** 12),
     UNSUPPORTED),
    (dict(N=2 ** 20 + 4, a=0x10 ** 12, b=0x20 ** 12, d=0x30 ** 12),
     UNSUPPORTED),
    (dict(batch=0), OK), (dict(M=0), OK), (dict(N=0), OK),
    (dict(batch=0, a=None, b=None, d=None), OK),
])
def test_f16acc_argument_checks(kw, status):
    assert _acc(**kw) == status


def test_f16acc_broadcast_strides_are_accepted_by_the_checks():
    # stride 0 broadcasts A or B; only the checks run (batch 0 is a no-op,
    # so use the overlap check to see that a 0 stride is not rejected)
    assert _acc(sA=0, d=0x100000 + 64) == INVALID     # still overlaps A
    assert _acc(batch=0, sA=0, sB=0) == OK


def test_noalloc_rejects_plans_beyond_its_scratch(monkeypatch):
    """gemm_tn_ex_noalloc refuses, before any launch, a problem whose
    split-K partials exceed its fixed scratch.  The planner's own plans
    stay within it (one wave of 256 x 256 fp32 tiles at most: 64 MiB); a
    forced 8-way split of 4096^2 x 4096 needs 8 x 64 MiB."""
    M = N = K = 4096
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=256,split=8")
    st = g.gemm_tn_ex_noalloc(1, M, N, K, 1.0, P, K, M * K, P, K, N * K, 0.0,
                              NULL, N, M * N, P, N, M * N, F32, S)
    assert st == g.ERR_SCRATCH
    assert "static maximum" in g.status_string(st)
    # argument errors are still reported first
    assert g.gemm_tn_ex_noalloc(1, -1, N, K, 1.0, P, K, 0, P, K, 0, 0.0, NULL,
                                N, 0, P, N, 0, F32, S) == INVALID


def test_fast_binding_is_loaded_and_hands_back_what_it_does_not_take():
    """The binding's C++ fast path is built next to the library and loaded;
    it returns -1 (leaving the call to the checked Python path) for every
    call outside the plain cases, before touching a device."""
    torch = pytest.importorskip("torch")
    assert g._fast is not None, "fast binding not built (build())"
    h = torch.float16
    A = torch.zeros(4, 8, dtype=h)
    B = torch.zeros(5, 8, dtype=h)
    D = torch.zeros(4, 5, dtype=h)
    f = g._fast.gemm_tn_fast
    assert f(A, B, D, 1.0, 0.0, None, 0) == -1          # host tensors
    assert f(A.float(), B, D, 1.0, 0.0, None, 0) == -1  # A not fp16
    assert f(A, B[:, :4], D, 1.0, 0.0, None, 0) == -1   # K mismatch
    assert f(A, B, D, 1.0, 0.5, None, 0) == -1          # beta without C
    with pytest.raises(ValueError, match="on the GPU"):
        g.gemm_tn(A, B, out=D)                          # checked path
