"""Checks of the GEMM kernels' generated gfx950 assembly (CPU only: hipcc
cross-compiles).

- No mixed-precision FMA with a zero addend: hipcc can select
  (_Float16)(x * y) as v_fma_mixlo_f16 d, x, y, 0, which turns a -0
  product into +0 (alpha < 0 times an exactly cancelling sum).  Every fp16
  conversion of a bare product goes through to_half.
- No scratch (register spills to private memory) in any GEMM kernel.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "dense_gemm_fp16_amd"))
import build as B  # noqa: E402  (the library's own build flags)

SOURCES = ["gemm_tn_tile256.hip", "gemm_tn_tile128.hip", "gemm_tn_tile64.hip",
           "gemm_tn_onek.hip", "gemm_tn_api.hip"]

ZERO_ADDEND = re.compile(
    r"v_fma_mix(lo|hi)?_f(16|32)\s+[^,]+,\s*[^,]+,\s*[^,]+,\s*-?0(\s|$)")


def _assembly(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = ([B.HIPCC] + B.FLAGS + B.FILE_FLAGS.get(src, [])
           + ["--cuda-device-only", "-S", os.path.join(B.CSRC, src),
              "-o", out])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    assert r.returncode == 0, r.stdout
    return open(out).read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _assembly(s, d), SOURCES))
    return dict(zip(SOURCES, texts))


def _kernels(text):
    """(name, body, metadata tail) of every gtn function in an assembly
    file (data symbols, such as the no-allocation scratch array, are
    skipped)."""
    for name in re.findall(r"\.type\s+(_ZN3gtn[^,\s]+),@function", text):
        start = text.index(name + ":")
        end = text.index(".Lfunc_end", start)
        yield name, text[start:end], text[end:end + 4000]


@pytest.mark.parametrize("src", SOURCES)
def test_no_mixed_fma_with_a_zero_addend(assembly, src):
    bad = [(name[:80], ln.strip())
           for name, body, _ in _kernels(assembly[src])
           for ln in body.splitlines() if ZERO_ADDEND.search(ln)]
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(assembly, src):
    kernels = list(_kernels(assembly[src]))
    assert kernels, "no kernels found"
    bad = []
    for name, _, tail in kernels:
        m = re.search(r"; ScratchSize: (\d+)", tail)
        if m and int(m.group(1)) > 0:
            bad.append((name[:80], m.group(1)))
    assert not bad, bad[:5]


# Four-wave 256-tile kernels (MIN_WAVES 1, SCHED 3, 16x16 MFMA): their
# MFMAs are inline asm, so the compiler pads none of their hazards.
FOUR_WAVE = re.compile(r"Li1ELi3ELi16ELi0EE")
MFMA_LINE = re.compile(r"^\s*v_mfma\S*\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")


def _vregs(op):
    """VGPR numbers named by an operand such as v7 or v[94:97]."""
    m = re.fullmatch(r"v(\d+)", op) or re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def _instructions(body):
    """Instruction lines of a function body (no labels, comments, asm
    markers or directives)."""
    out = []
    for ln in body.splitlines():
        t = ln.strip()
        if not t or t.startswith((";", ".", "_")) or t.endswith(":"):
            continue
        out.append(t.split(";")[0].strip())
    return out


def _slots(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _four_wave_kernels(assembly):
    ks = [(n, b) for n, b, _ in _kernels(assembly["gemm_tn_tile256.hip"])
          if FOUR_WAVE.search(n)]
    assert len(ks) == 3, [n for n, _ in ks]   # f16 / f32 output, split-K
    return ks


def _fresh_operands(ins):
    """(VALU instruction, MFMA) pairs where the MFMA reads, as source A or
    B, a VGPR the vector-ALU instruction wrote less than two wait states
    before."""
    bad = []
    for k, t in enumerate(ins):
        m = MFMA_LINE.match(t)
        if not m:
            continue
        srcs = _vregs(m.group(2)) | _vregs(m.group(3))
        slots, q = 0, k - 1
        while q >= 0 and slots < 2:
            prev = ins[q]
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                dst = prev.split()[1].rstrip(",")
                if _vregs(dst) & srcs:
                    bad.append((prev, t))
            slots += _slots(prev)
            q -= 1
    return bad


def _padding_after_last_mfma(ins):
    """Wait states from the last MFMA to the first instruction after it
    that names an accumulation register."""
    last = max(k for k, t in enumerate(ins) if MFMA_LINE.match(t))
    slots = 0
    for t in ins[last + 1:]:
        if re.search(r"\ba(\d+|\[\d+:\d+\])", t):
            break
        slots += _slots(t)
    return slots


def test_four_wave_mfma_operands_are_not_fresh_valu_results(assembly):
    """An MFMA reading a VGPR that a vector-ALU instruction wrote needs two
    wait states between them; the asm MFMAs get none from the compiler, so
    their fragment registers must come from loads only."""
    for name, body in _four_wave_kernels(assembly):
        bad = _fresh_operands(_instructions(body))
        assert not bad, (name[:60], bad[:3])


def test_four_wave_results_are_read_after_the_padding(assembly):
    """Every instruction that reads the accumulation registers after the
    last MFMA (the epilogue's reads, or stores straight from them) comes at
    least 18 wait states after it (an 8-pass MFMA's result needs fewer)."""
    for name, body in _four_wave_kernels(assembly):
        slots = _padding_after_last_mfma(_instructions(body))
        assert slots >= 18, (name[:60], slots)


def test_the_hazard_checks_catch_what_they_look_for():
    mfma = "v_mfma_f32_16x16x32_f16 a[0:3], v[94:97], v[42:45], a[0:3]"
    assert _fresh_operands(["v_add_u32_e32 v95, s1, v2", mfma])
    assert _fresh_operands(["v_mov_b32_e32 v44, 0", "s_nop 0", mfma])
    assert not _fresh_operands(["v_mov_b32_e32 v44, 0", "s_nop 1", mfma])
    assert not _fresh_operands(["v_add_u32_e32 v98, s1, v2", mfma])
    assert not _fresh_operands(["ds_read_b128 v[94:97], v1", mfma])
    assert _padding_after_last_mfma(
        [mfma, "s_nop 7", "v_accvgpr_read_b32 v1, a0"]) == 8
    assert _padding_after_last_mfma(
        [mfma, "s_nop 7", "s_nop 7", "s_nop 7", "ds_write_b128 v1, a[0:3]"]) \
        == 24


def test_the_zero_addend_pattern_matches_the_miscompiled_form():
    """The pattern catches the instruction the old epilogue produced and
    leaves the legitimate forms alone."""
    assert ZERO_ADDEND.search("\tv_fma_mixlo_f16 v136, s36, v4, 0")
    assert ZERO_ADDEND.search("\tv_fma_mix_f32 v1, s2, v3, -0 op_sel_hi:[0,1,0]")
    assert not ZERO_ADDEND.search(
        "\tv_fma_mixlo_f16 v128, s37, v148, v126 op_sel_hi:[0,1,0]")
    assert not ZERO_ADDEND.search("\tv_fma_f32 v1, v2, v3, 0")
