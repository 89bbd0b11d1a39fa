"""Pins for the CPU oracle, on values fixed by the definition and by
mathematics rather than by the oracle itself.

Each `pin_*` function raises AssertionError on a mismatch.  The pins run
once against the oracle proper and once against each planted-mistake build
(`oracle.mutant(n)`): every planted mistake must fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# ---- binary16 codec ----------------------------------------------------------

def pin_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_f16(bits)
    want = bits.view(np.float16).astype(np.float64)   # numpy's IEEE decode
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_decode_golden():
    g = json.load(open(os.path.join(GOLDEN, "fp16_values.json")))
    for h, v in g["decode"]:
        got = oracle.decode_f16(np.array([int(h, 16)], np.uint16))[0]
        assert got == float(v), (h, got, v)


def pin_encode_golden():
    g = json.load(open(os.path.join(GOLDEN, "fp16_values.json")))
    for name, v, h in g["encode_rne"]:
        got = int(oracle.rn16_bits(np.array([v]))[0])
        assert got == int(h, 16), (name, hex(got), h)


def pin_encode_matches_numpy():
    r = _rng(5)
    xs = np.concatenate([
        r.uniform(-1, 1, 20000),
        r.standard_normal(20000) * 1e-5,               # subnormal range
        r.uniform(-70000, 70000, 20000),               # overflow range
        np.ldexp(r.uniform(1, 2, 20000), r.integers(-30, 17, 20000)),
        # exact ties between adjacent binary16 values
        (np.arange(1, 5000) + 0.5) * 2.0 ** -10,
        (np.arange(1, 5000) + 0.5) * 2.0 ** -24,
    ])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)  # numpy's RNE cast
    got = oracle.rn16_bits(xs)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def pin_rn32_matches_numpy():
    xs = _rng(6).standard_normal(10000) * 10.0 ** _rng(7).integers(-30, 30,
                                                                    10000)
    assert np.array_equal(oracle.rn32(xs).view(np.uint32),
                          xs.astype(np.float32).view(np.uint32))


# ---- the GEMM -------------------------------------------------------------------

def pin_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "gemm_worked_examples.json")))
    for c in g["cases"]:
        C = None if c["C"] is None else np.array(c["C"], np.float32)
        got = oracle.gemm_tn(_f16(c["A"]), _f16(c["B"]), c["alpha"],
                             c["beta"], C)
        assert np.array_equal(got, np.array(c["D"], float)), (c["name"], got)


def pin_identity():
    r = _rng(1)
    M, K = 37, 24
    A = _f16(r.uniform(-1, 1, (M, K)))
    C = r.uniform(-1, 1, (M, K)).astype(np.float32)
    got = oracle.gemm_tn(A, _f16(np.eye(K)), 2.0, -0.5, C)
    want = 2.0 * A.astype(np.float64) - 0.5 * C.astype(np.float64)
    assert np.array_equal(got, want)


def pin_permutation():
    # B row j = e_{pi(j)}  =>  d(i, j) = a(i, pi(j)).  pi is not an
    # involution, so reading B as K x N (A @ B instead of A @ B^T) fails.
    r = _rng(2)
    M, K = 19, 16
    pi = np.roll(np.arange(K), 3)
    A = _f16(r.uniform(-4, 4, (M, K)))
    B = np.zeros((K, K))
    B[np.arange(K), pi] = 1.0
    got = oracle.gemm_tn(A, _f16(B))
    assert np.array_equal(got, A.astype(np.float64)[:, pi])


def pin_k1_outer_product():
    r = _rng(3)
    a = _f16(r.uniform(-1, 1, (9, 1)))
    b = _f16(r.uniform(-1, 1, (13, 1)))
    got = oracle.gemm_tn(a, b, 1.5)
    want = 1.5 * np.outer(a.astype(np.float64)[:, 0], b.astype(np.float64)[:, 0])
    assert np.array_equal(got, want)


def pin_alpha_beta_cases():
    r = _rng(4)
    A = _f16(r.uniform(-1, 1, (8, 12)))
    B = _f16(r.uniform(-1, 1, (10, 12)))
    C = r.uniform(-1, 1, (8, 10)).astype(np.float32)
    # alpha = 0 leaves beta * C
    assert np.array_equal(oracle.gemm_tn(A, B, 0.0, 0.75, C),
                          0.75 * C.astype(np.float64))
    # beta = 0 never reads C: NaN in C does not leak
    Cn = np.full((8, 10), np.nan, np.float32)
    assert np.isfinite(oracle.gemm_tn(A, B, 1.0, 0.0, Cn)).all()
    # B = 0, beta = 1 gives C
    assert np.array_equal(
        oracle.gemm_tn(A, _f16(np.zeros((10, 12))), 1.0, 1.0, C),
        C.astype(np.float64))
    # power-of-two alpha scales exactly
    base = oracle.gemm_tn(A, B)
    assert np.array_equal(oracle.gemm_tn(A, B, 0.25), 0.25 * base)
    # fp16 C is decoded exactly
    C16 = _f16(r.uniform(-1, 1, (8, 10)))
    assert np.array_equal(oracle.gemm_tn(A, _f16(np.zeros((10, 12))), 1.0,
                                         -2.0, C16),
                          -2.0 * C16.astype(np.float64))


def pin_brute_force_4x4():
    r = _rng(8)
    a = r.integers(-5, 6, (4, 4)).astype(np.float64)
    b = r.integers(-5, 6, (4, 4)).astype(np.float64)
    got = oracle.gemm_tn(_f16(a), _f16(b))
    for i in range(4):
        for j in range(4):
            s = (a[i][0] * b[j][0] + a[i][1] * b[j][1] +
                 a[i][2] * b[j][2] + a[i][3] * b[j][3])
            assert got[i, j] == s, (i, j)


def pin_integer_exact():
    # small-integer operands: int64 arithmetic gives the exact answer
    r = _rng(9)
    batch, M, N, K = 3, 33, 41, 257
    A = r.integers(-3, 4, (batch, M, K))
    B = r.integers(-3, 4, (batch, N, K))
    got = oracle.gemm_tn(_f16(A), _f16(B))
    want = np.einsum("bmk,bnk->bmn", A, B)          # int64, exact
    assert np.array_equal(got, want.astype(np.float64))


def pin_random_vs_library():
    # fp16 inputs, exact products; numpy's float64 matmul sums in another
    # order, so the two agree to within fp64 rounding
    r = _rng(10)
    M, N, K = 45, 29, 300
    A = _f16(r.uniform(-1, 1, (M, K)))
    B = _f16(r.uniform(-1, 1, (N, K)))
    C = r.uniform(-1, 1, (M, N)).astype(np.float32)
    got = oracle.gemm_tn(A, B, 1.5, 0.5, C)
    want = (1.5 * (A.astype(np.float64) @ B.astype(np.float64).T)
            + 0.5 * C.astype(np.float64))
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_batches_are_independent():
    r = _rng(11)
    batch, M, N, K = 4, 7, 5, 9
    A = _f16(r.uniform(-1, 1, (batch, M, K)))
    B = _f16(r.uniform(-1, 1, (batch, N, K)))
    full = oracle.gemm_tn(A, B)
    for b in range(batch):
        assert np.array_equal(full[b], oracle.gemm_tn(A[b], B[b]))
    assert not np.array_equal(full[0], full[1])


def pin_rows_and_points_agree():
    r = _rng(12)
    batch, M, N, K = 2, 11, 13, 17
    A = _f16(r.uniform(-1, 1, (batch, M, K)))
    B = _f16(r.uniform(-1, 1, (batch, N, K)))
    C = r.uniform(-1, 1, (batch, M, N)).astype(np.float32)
    full = oracle.gemm_tn(A, B, 0.5, 2.0, C)
    part = oracle.gemm_tn(A, B, 0.5, 2.0, C, rows=(5, 17))
    assert np.array_equal(part, full.reshape(-1, N)[5:17])
    pts = np.array([[0, 0, 0], [1, 10, 12], [1, 3, 4], [0, 7, 1]])
    got = oracle.gemm_tn_points(A, B, pts, 0.5, 2.0, C)
    assert np.array_equal(got, full[pts[:, 0], pts[:, 1], pts[:, 2]])


def pin_subnormal_operands():
    # products of fp16 subnormals are exact in double and must survive
    a = np.array([[0x0001, 0x03FF]], np.uint16).view(np.float16)
    b = np.array([[0x3C00, 0x4000]], np.uint16).view(np.float16)  # 1, 2
    got = oracle.gemm_tn(a, b)[0, 0]
    assert got == 2.0 ** -24 + 2 * 1023 * 2.0 ** -24


def pin_degenerate_sizes():
    C = np.arange(6, dtype=np.float32).reshape(2, 3)
    got = oracle.gemm_tn(np.zeros((2, 0), np.float16),
                         np.zeros((3, 0), np.float16), 1.0, 3.0, C)
    assert np.array_equal(got, 3.0 * C.astype(np.float64))      # K = 0
    assert oracle.gemm_tn(np.zeros((0, 4), np.float16),
                          np.zeros((3, 4), np.float16)).shape == (0, 3)


def pin_threads_do_not_change_bits():
    r = _rng(13)
    A = _f16(r.uniform(-1, 1, (64, 200)))
    B = _f16(r.uniform(-1, 1, (48, 200)))
    one = oracle.gemm_tn(A, B, threads=1)
    many = oracle.gemm_tn(A, B, threads=7)
    assert np.array_equal(one.view(np.uint64), many.view(np.uint64))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# mutant number -> the mistake planted (oracle.MUTANTS: text substitutions
# applied to a copy of gemm_oracle.c)
MUTANTS = {n: what for n, (what, _) in oracle.MUTANTS.items()}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=list(MUTANTS.values()))
def test_planted_mistake_is_caught(n):
    failed = []
    with oracle.mutant(n):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"no pin rejects planted mistake {n}: {MUTANTS[n]}"


# ---- the acceptance checker -----------------------------------------------------

def test_checker_flags_planted_error():
    r = _rng(20)
    ref = r.uniform(-10, 10, (6, 7))
    K = 400
    tol = oracle.tolerance(ref, K, "f32")
    d = ref.astype(np.float32).copy()
    assert oracle.check(d, ref, K, "f32").ok
    d[3, 4] = ref[3, 4] + 2.0 * tol[3, 4]
    res = oracle.check(d, ref, K, "f32")
    assert not res.ok and res.n_bad == 1 and res.worst_index == (3, 4)
    assert 1.9 < res.worst_ratio < 2.1
    d[3, 4] = ref[3, 4] + 0.5 * tol[3, 4]
    assert oracle.check(d, ref, K, "f32").ok
    d[0, 0] = np.nan
    assert not oracle.check(d, ref, K, "f32").ok


def test_checker_f16_half_ulp_term():
    # ref just below 2048 rounds up to 2048 in fp16: the half-ulp term is
    # taken at rn16(ref) = 2048 (ulp 2), so d = 2048 passes
    ref = np.array([2047.9999])
    tol = oracle.tolerance(ref, 1, "f16")
    assert math.isclose(tol[0], 1e-3 * 2047.9999 + 1e-4 + 1.0)
    assert oracle.check(np.array([2048.0], np.float16), ref, 1, "f16").ok
    # fp16 subnormal range: ulp is 2^-24
    assert oracle.ulp16(np.array([1e-7]))[0] == 2.0 ** -24
    assert oracle.ulp16(np.array([0.0]))[0] == 2.0 ** -24
    assert oracle.ulp16(np.array([1.0]))[0] == 2.0 ** -10


def test_check_exact():
    ref = np.array([[1.0, 2.5], [-3.0, 1e-3]])
    d32 = oracle.rn32(ref)
    assert oracle.check_exact(d32, ref, "f32").ok
    d32[1, 1] = np.nextafter(d32[1, 1], np.float32(1))
    res = oracle.check_exact(d32, ref, "f32")
    assert not res.ok and res.worst_index == (1, 1)
    d16 = oracle.rn16_bits(ref).view(np.float16)
    assert oracle.check_exact(d16, ref, "f16").ok


def test_check_exact_signed_zero():
    """The sign of an exact zero is part of the bit-exact check: the
    oracle's +0 sum times alpha = -2 is -0, and a +0 there fails; the
    smallest subnormal of either sign does not match zero either."""
    ref = oracle.gemm_tn(np.array([[1.0, 1.0]], np.float16),
                         np.array([[1.0, -1.0]], np.float16), alpha=-2.0)
    assert ref[0, 0] == 0.0 and np.signbit(ref[0, 0])       # -2 * (+0)
    ref = np.array([0.0, -0.0, 0.0, 1.0])
    for out, dt, tiny in (("f16", np.float16, 2.0 ** -24),
                          ("f32", np.float32, 2.0 ** -149)):
        d = np.array([0.0, -0.0, 0.0, 1.0], dt)
        assert oracle.check_exact(d, ref, out).ok
        for k, z in ((0, -0.0), (1, 0.0)):
            e = d.copy()
            e[k] = dt(z)
            res = oracle.check_exact(e, ref, out)
            assert not res.ok and res.n_bad == 1, (out, k)
        for bad in (tiny, -tiny):
            e = d.copy()
            e[2] = dt(bad)
            res = oracle.check_exact(e, ref, out)
            assert not res.ok and res.n_bad == 1, (out, bad)
        e = d.copy()
        e[3] = dt(-1.0)
        assert not oracle.check_exact(e, ref, out).ok


def test_oracle_zero_sums_are_positive():
    """IEEE round-to-nearest: a sum that starts at +0 and cancels exactly,
    or whose terms are all zeros of either sign, is +0 (so the sign of a
    zero result is alpha's, unless the beta term decides it)."""
    A = np.array([[0.0, 0.0, 0.0], [3.0, -1.0, -2.0], [-0.0, -0.0, -0.0]],
                 np.float16)
    B = np.array([[-1.0, -2.0, 3.0], [1.0, 1.0, 1.0]], np.float16)
    ref = oracle.gemm_tn(A, B)
    zero = ref == 0.0
    assert zero.sum() == 5 and not np.signbit(ref[zero]).any()
    neg = oracle.gemm_tn(A, B, alpha=-0.5)
    assert np.signbit(neg[zero]).all()
    C = np.full((3, 2), -0.0, np.float32)
    # +0 + beta * (-0): +0 for beta > 0; -0 + (-0) = -0 for negative alpha
    assert not np.signbit(oracle.gemm_tn(A, B, 1.0, 1.0, C)[zero]).any()
    assert np.signbit(oracle.gemm_tn(A, B, -1.0, 1.0, C)[zero]).all()
