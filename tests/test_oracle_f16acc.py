"""Pins of the fp16-accumulating GEMM oracle (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import gemm_f16acc as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "gemm_f16acc_worked_example.json")


def _golden_operands():
    a = np.ones((2, 48), np.float16)
    a[1] = 2
    b = np.zeros((2, 48), np.float16)
    b[0, :15] = 127
    b[0, 15] = 142
    b[0, 16:20] = 1
    b[0, 32:35] = 1
    b[1, :32] = 62.5
    b[1, 32] = 49
    return a, b


def test_worked_example():
    g = json.load(open(GOLDEN))
    a, b = _golden_operands()
    d = F.gemm_tn_f16acc(a, b)
    assert d.dtype == np.float16
    np.testing.assert_array_equal(d.astype(np.float64), g["D"])
    np.testing.assert_array_equal(a.astype(np.float64) @ b.astype(np.float64).T,
                                  g["exact"])


def test_constant_inputs_closed_form():
    # a = b = 3: each 16-deep step adds 144; 144 s is exact in binary16
    # while the spacing divides 144 (below 2^15, spacing <= 16)
    for steps in (1, 7, 100, 227):
        K = 16 * steps
        d = F.gemm_tn_f16acc(np.full((1, K), 3, np.float16),
                             np.full((1, K), 3, np.float16))
        assert float(d[0, 0]) == 144 * steps
    # step 229: 32832 + 144 = 32976 = 32768 + 6.5 * 32, a tie -> 32960
    K = 16 * 229
    d = F.gemm_tn_f16acc(np.full((1, K), 3, np.float16),
                         np.full((1, K), 3, np.float16))
    assert float(d[0, 0]) == 32960


def test_one_step_is_one_rounding_of_the_exact_product():
    r = np.random.default_rng(3)
    for K in (1, 5, 16):
        a = r.standard_normal((7, K)).astype(np.float16)
        b = r.standard_normal((9, K)).astype(np.float16)
        exact = a.astype(np.float64) @ b.astype(np.float64).T
        np.testing.assert_array_equal(F.gemm_tn_f16acc(a, b),
                                      exact.astype(np.float16))


def test_small_integers_are_exact():
    # |partial sums| stay below 2048, where binary16 holds every integer
    r = np.random.default_rng(4)
    a = r.integers(-3, 4, (2, 12, 200)).astype(np.float16)
    b = r.integers(-3, 4, (2, 10, 200)).astype(np.float16)
    exact = np.einsum("bik,bjk->bij", a.astype(np.int64), b.astype(np.int64))
    assert np.abs(exact).max() < 2048
    np.testing.assert_array_equal(F.gemm_tn_f16acc(a, b).astype(np.int64),
                                  exact)


def test_the_step_is_sixteen_deep():
    # the golden case tells 16-deep steps from 1- and 48-deep ones
    a, b = _golden_operands()
    d16 = F.gemm_tn_f16acc(a, b)
    for kstep in (1, 48):
        assert not np.array_equal(F.gemm_tn_f16acc(a, b, kstep=kstep), d16)
    # and this one from 32-deep steps: 16-deep sums 2047, 1, 1, 1 give
    # 2047 -> 2048 -> rn16(2049) = 2048 -> 2048 (ties to even), while the
    # 32-deep sums 2048, 2 give 2050
    a = np.ones((1, 64), np.float16)
    b = np.zeros((1, 64), np.float16)
    b[0, :15] = 127
    b[0, 15] = 142
    b[0, [16, 32, 48]] = 1
    assert float(F.gemm_tn_f16acc(a, b)[0, 0]) == 2048
    assert float(F.gemm_tn_f16acc(a, b, kstep=32)[0, 0]) == 2050


def test_brute_force_tiny():
    r = np.random.default_rng(5)
    a = r.standard_normal((3, 37)).astype(np.float16)
    b = r.standard_normal((2, 37)).astype(np.float16)
    d = F.gemm_tn_f16acc(a, b)
    for i in range(3):
        for j in range(2):
            acc = np.float16(0)
            for k0 in range(0, 37, 16):
                s = sum(float(a[i, k]) * float(b[j, k])
                        for k in range(k0, min(k0 + 16, 37)))
                acc = np.float16(float(acc) + s)
            assert d[i, j] == acc


def test_flip_bound_covers_a_one_ulp_move():
    a, b = _golden_operands()
    d, bound = F.flip_bound(a, b)
    # three steps; the spacing of binary16 is 0.5 in [512, 1024), 1 in
    # [1024, 2048), 2 in [2048, 4096) and 4 in [4096, 8192)
    np.testing.assert_array_equal(d.astype(np.float64),
                                  [[2056, 2048], [4112, 4096]])
    np.testing.assert_array_equal(bound, [[1 + 2 + 2, 0.5 + 1 + 2],
                                          [2 + 4 + 4, 1 + 2 + 4]])
