"""CPU oracle for the fp16 TN GEMM  D = alpha * A @ B^T + beta * C.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this package.  The product path
(the HIP library and its Python binding) never imports, loads or calls it,
and the two share no code: only the seeded input bits cross over.

The arithmetic lives in `gemm_oracle.c` (plain C, fp64, sequential k sum;
see its header for the passages it follows).  This module loads it through
ctypes and adds the acceptance test for the GPU result:

  |d - ref| <= 1e-3*|ref| + 1e-4*sqrt(K)  (+ half an fp16 ulp of rn16(ref)
                                             when D is fp16)

and a bit-exact comparison against rn_out(ref) for integer-valued inputs.

Pins (tests/test_oracle.py): the binary16 codec against all 65536 patterns
and numpy's IEEE conversions; the GEMM against identity and permutation
operands, K = 1 outer products, alpha/beta special cases, hand-expanded 4x4
sums, exact int64 products for integer inputs, and a worked example stored
under tests/golden/.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgemm_oracle.so")
_lib = None

C_F16, C_F32 = 0, 1


# Planted mistakes (a CPU-only device for testing the pins): number ->
# (what it models, [(text of gemm_oracle.c, replacement)]).  A mutant copy
# of the source is written next to the build and compiled under its own
# name; the oracle's own source holds no trace of them.
MUTANTS = {
    1: ("last k term dropped",
        [("for (int64_t k = 0; k < K; ++k)",
          "for (int64_t k = 0; k < K - (K > 0); ++k)")]),
    2: ("B read as K x N",
        [("const double *brow = job->b + (bi * job->N + j) * job->K;",
          "const double *brow = job->b + bi * job->N * job->K + j;"),
         ("int64_t bstep = 1;", "int64_t bstep = job->N;")]),
    3: ("sign of the beta term",
        [("r = r + beta * load_c(C, c_dtype, cidx);",
          "r = r - beta * load_c(C, c_dtype, cidx);")]),
    4: ("fp16 subnormals flushed",
        [("v = ldexp((double)m, -24);", "v = 0.0;")]),
    5: ("encode truncates",
        [("if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))",
          "if (0)")]),
    6: ("batch index of B ignored",
        [("int64_t bi = r / job->M;", "int64_t bi = 0;")]),
}


def _mutant_source(n: int) -> str:
    text = open(_SRC).read()
    for old, new in MUTANTS[n][1]:
        if text.count(old) != 1:
            raise RuntimeError(f"mutant {n}: {old!r} not found once")
        text = text.replace(old, new)
    path = os.path.join(_HERE, "_mutant%d.c" % n)
    with open(path, "w") as f:
        f.write(text)
    return path


def build(force: bool = True, mutant: int = 0) -> str:
    """Compile the oracle with gcc (no fused multiply-add, no fast-math).

    `mutant` > 0 builds a copy with planted mistake number `mutant` (see
    MUTANTS) under a separate name; the tests use those copies to show that
    the pins reject each mistake."""
    path = _LIB_PATH if mutant == 0 else os.path.join(
        _HERE, "libgemm_oracle_mutant%d.so" % mutant)
    if force or not os.path.exists(path):
        src = _SRC if mutant == 0 else _mutant_source(mutant)
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
             "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-o", tmp, src,
             "-lm"])
        os.replace(tmp, path)
        if src != _SRC:
            os.remove(src)
    return path


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.gemm_oracle_half_to_double.restype = dbl
    lib.gemm_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.gemm_oracle_double_to_half.restype = ctypes.c_uint16
    lib.gemm_oracle_double_to_half.argtypes = [dbl]
    for name in ("gemm_oracle_decode_f16", "gemm_oracle_encode_f16",
                 "gemm_oracle_encode_f32"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [vp, vp, i64]
    lib.gemm_oracle_tn_rows.restype = ctypes.c_int
    lib.gemm_oracle_tn_rows.argtypes = [i64, i64, i64, i64, dbl, vp, vp, dbl,
                                        vp, ctypes.c_int, vp, i64, i64,
                                        ctypes.c_int]
    lib.gemm_oracle_tn_points.restype = ctypes.c_int
    lib.gemm_oracle_tn_points.argtypes = [i64, i64, i64, i64, dbl, vp, vp,
                                          dbl, vp, ctypes.c_int, vp, i64, vp]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def mutant(n: int):
    """Within the block, every oracle function runs a copy built with
    planted mistake number n (a CPU-only device for testing the pins)."""
    global _lib
    saved = _load()
    _lib = _bind(build(force=False, mutant=n))
    try:
        yield
    finally:
        _lib = saved


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on,
    capped at 16 (the CPU share of one GPU on the measurement host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- binary16 codec ------------------------------------------------------

def decode_f16(bits) -> np.ndarray:
    """uint16 bit patterns (or a float16 array) -> exact float64 values."""
    b = np.ascontiguousarray(np.asarray(bits).view(np.uint16)
                             if np.asarray(bits).dtype == np.float16
                             else np.asarray(bits, dtype=np.uint16))
    out = np.empty(b.shape, dtype=np.float64)
    _load().gemm_oracle_decode_f16(_p(b), _p(out), b.size)
    return out


def rn16_bits(x) -> np.ndarray:
    """float64 -> binary16 bits, round to nearest even, overflow to inf."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().gemm_oracle_encode_f16(_p(x), _p(out), x.size)
    return out


def rn32(x) -> np.ndarray:
    """float64 -> binary32, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    _load().gemm_oracle_encode_f32(_p(x), _p(out), x.size)
    return out


# ---- the GEMM --------------------------------------------------------------

def _operands(A, B, C, batch, M, N, K, beta):
    A = np.ascontiguousarray(A, dtype=np.float16).reshape(batch, M, K)
    B = np.ascontiguousarray(B, dtype=np.float16).reshape(batch, N, K)
    c_code, Cc = C_F32, None
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        Cc = np.ascontiguousarray(C).reshape(batch, M, N)
        if Cc.dtype == np.float16:
            c_code = C_F16
        elif Cc.dtype == np.float32:
            c_code = C_F32
        else:
            raise TypeError("C must be float16 or float32")
    return A.view(np.uint16), B.view(np.uint16), Cc, c_code


def gemm_tn(A, B, alpha=1.0, beta=0.0, C=None, *, threads=None,
            rows=None) -> np.ndarray:
    """ref = alpha * A @ B^T + beta * C in float64, batched.

    A: (batch, M, K) or (M, K) float16; B: (batch, N, K) or (N, K) float16;
    C: same leading shape as the result, float16 or float32, read only when
    beta != 0.  `rows=(r0, r1)` restricts the result to flattened rows
    [r0, r1) of the (batch*M) x N output.  Returns float64 of shape
    (batch, M, N) (or (M, N) for 2-D inputs, or (r1-r0, N) with rows)."""
    A = np.asarray(A)
    B = np.asarray(B)
    two_d = A.ndim == 2
    if two_d:
        A, B = A[None], B[None]
        if C is not None:
            C = np.asarray(C)[None]
    batch, M, K = A.shape
    N = B.shape[1]
    if B.shape != (batch, N, K):
        raise ValueError("B must be (batch, N, K) with A's batch and K")
    Ab, Bb, Cc, c_code = _operands(A, B, C, batch, M, N, K, beta)
    r0, r1 = (0, batch * M) if rows is None else rows
    out = np.empty((r1 - r0, N), dtype=np.float64)
    rc = _load().gemm_oracle_tn_rows(
        batch, M, N, K, float(alpha), _p(Ab), _p(Bb), float(beta),
        _p(Cc) if Cc is not None else None, c_code, _p(out), r0, r1,
        threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    if rows is not None:
        return out
    out = out.reshape(batch, M, N)
    return out[0] if two_d else out


def gemm_tn_points(A, B, points, alpha=1.0, beta=0.0, C=None) -> np.ndarray:
    """ref at selected (b, i, j) triples (an (n, 3) integer array)."""
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim == 2:
        A, B = A[None], B[None]
        if C is not None:
            C = np.asarray(C)[None]
    batch, M, K = A.shape
    N = B.shape[1]
    Ab, Bb, Cc, c_code = _operands(A, B, C, batch, M, N, K, beta)
    pts = np.ascontiguousarray(points, dtype=np.int64).reshape(-1, 3)
    out = np.empty(len(pts), dtype=np.float64)
    rc = _load().gemm_oracle_tn_points(
        batch, M, N, K, float(alpha), _p(Ab), _p(Bb), float(beta),
        _p(Cc) if Cc is not None else None, c_code, _p(pts), len(pts),
        _p(out))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return out


# ---- acceptance -------------------------------------------------------------

def ulp16(x16: np.ndarray) -> np.ndarray:
    """Spacing of binary16 values at x (x already a binary16 value):
    2^(max(floor(log2|x|), -14) - 10)."""
    a = np.abs(np.asarray(x16, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2^e, f in [0.5, 1)
    e = np.where(a > 0, e - 1, -14)
    return np.ldexp(1.0, np.maximum(e, -14) - 10)


def tolerance(ref: np.ndarray, K: int, out_dtype: str) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    tol = 1e-3 * np.abs(ref) + 1e-4 * math.sqrt(K)
    if out_dtype == "f16":
        tol = tol + 0.5 * ulp16(decode_f16(rn16_bits(ref)))
    return tol


@dataclass
class Check:
    ok: bool
    n_bad: int
    n: int
    worst_index: tuple | None
    worst_ratio: float      # max |d - ref| / tol (<= 1 passes)

    def __str__(self):
        return (f"ok={self.ok} bad={self.n_bad}/{self.n} "
                f"worst={self.worst_index} ratio={self.worst_ratio:.3g}")


def check(d: np.ndarray, ref: np.ndarray, K: int, out_dtype: str) -> Check:
    """Element-wise tolerance test of a GPU result d against ref."""
    d = np.asarray(d)
    ref = np.asarray(ref, dtype=np.float64)
    if d.shape != ref.shape:
        raise ValueError(f"shape mismatch {d.shape} vs {ref.shape}")
    dv = d.astype(np.float64)
    tol = tolerance(ref, K, out_dtype)
    out_inf = (np.isinf(decode_f16(rn16_bits(ref))) if out_dtype == "f16"
               else np.isinf(rn32(ref).astype(np.float64)))
    with np.errstate(invalid="ignore"):
        err = np.abs(dv - ref)
        ratio = np.where(out_inf, np.where(dv == np.sign(ref) * np.inf, 0.0,
                                           np.inf), err / tol)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    bad = ratio > 1.0
    n_bad = int(bad.sum())
    worst = None
    wr = 0.0
    if ratio.size:
        w = int(np.argmax(ratio))
        worst = np.unravel_index(w, ratio.shape)
        wr = float(ratio.reshape(-1)[w])
    return Check(n_bad == 0, n_bad, int(ratio.size), worst, wr)


def expected_bits(ref: np.ndarray, out_dtype: str) -> np.ndarray:
    """rn_out(ref) as raw bits (uint16 for f16, uint32 for f32)."""
    if out_dtype == "f16":
        return rn16_bits(ref)
    return rn32(ref).view(np.uint32)


def check_exact(d: np.ndarray, ref: np.ndarray, out_dtype: str) -> Check:
    """Bit-exact test: d must equal the correctly rounded ref, bit for bit,
    the sign of a zero included.  For integer-valued inputs that sign is
    unique: under IEEE 754 round-to-nearest, x + (-x) is +0 and +0 + (-0) is
    +0, so a sum that starts at +0 and whose exact value is 0 ends at +0 in
    any order of the additions; alpha * (+0) and the beta term then follow
    the same sign rules on both sides."""
    d = np.ascontiguousarray(d)
    want = expected_bits(ref, out_dtype)
    got = d.view(np.uint16 if out_dtype == "f16" else np.uint32)
    bad = got != want
    n_bad = int(bad.sum())
    worst = None
    if n_bad:
        worst = np.unravel_index(int(np.argmax(bad)), bad.shape)
    return Check(n_bad == 0, n_bad, int(bad.size), worst,
                 0.0 if n_bad == 0 else math.inf)
