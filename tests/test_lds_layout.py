"""The kernels' LDS layouts, checked on the CPU (no GPU needed).

tests/lds/lds_layout_check.cpp compiles the kernels' own layout header
(dense_gemm_fp16_amd/csrc/lds_layout.hpp) as plain C++ and checks, for every
tile the kernels instantiate: each swizzle is a bijection of a row's
chunks; every lane group of every LDS access (fragment reads, staged tile
stores, transposing reads, epilogue staging, the attention K / V / O tiles,
the transpose tile) reaches distinct banks of gfx950's 64-bank LDS; the
transposing reads' per-lane base XOR 32 f lands on the element the layout
defines; and every 64- and 128-bit access is aligned.  Page "cute(8)
smem_gemm" (yuyanqi.com), section 3, makes conflict-freedom the checkable
property of a swizzle (3.7 checks it)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "lds", "lds_layout_check.cpp")
CSRC = os.path.join(ROOT, "dense_gemm_fp16_amd", "csrc")


def _build(tmp_path, extra=()):
    exe = str(tmp_path / "lds_layout_check")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                           "-D__host__=", "-D__device__=", "-I" + CSRC,
                           *extra, SRC, "-o", exe])
    return exe


def test_every_lds_layout_is_a_conflict_free_bijection(tmp_path):
    r = subprocess.run([_build(tmp_path)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 failures" in r.stdout, r.stdout


def test_the_check_catches_a_row_mod_8_swizzle(tmp_path):
    """The map a 32-bank LDS would want (chunk XOR row mod 8) puts two rows
    of one 16-lane group on the same banks of gfx950's LDS: the check must
    reject it (and the padded attention O rows it found before)."""
    hdr = tmp_path / "lds_layout.hpp"
    text = open(os.path.join(CSRC, "lds_layout.hpp")).read()
    good = "return chunk ^ ((row / (128 / BK)) % (BK / 8));"
    assert good in text
    hdr.write_text(text.replace(good, "return chunk ^ (row % (BK / 8));"))
    exe = str(tmp_path / "mutant")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-D__host__=",
                           "-D__device__=", "-I" + str(tmp_path), SRC, "-o",
                           exe])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode != 0 and "fragment read" in r.stderr, r.stderr
