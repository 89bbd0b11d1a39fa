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


def test_the_zero_addend_pattern_matches_the_miscompiled_form():
    """The pattern catches the instruction the old epilogue produced and
    leaves the legitimate forms alone."""
    assert ZERO_ADDEND.search("\tv_fma_mixlo_f16 v136, s36, v4, 0")
    assert ZERO_ADDEND.search("\tv_fma_mix_f32 v1, s2, v3, -0 op_sel_hi:[0,1,0]")
    assert not ZERO_ADDEND.search(
        "\tv_fma_mixlo_f16 v128, s37, v148, v126 op_sel_hi:[0,1,0]")
    assert not ZERO_ADDEND.search("\tv_fma_f32 v1, v2, v3, 0")
