"""Pins of the transpose oracle (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import transpose as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "transpose_worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    x = np.array(g["x"], dtype=np.float32)
    assert np.array_equal(T.transpose(x), np.array(g["y"], np.float32))


def test_definition_by_brute_force():
    r = np.random.default_rng(5)
    x = r.standard_normal((3, 5, 7)).astype(np.float32)
    y = T.transpose(x)
    assert y.shape == (3, 7, 5)
    for b in range(3):
        for i in range(5):
            for j in range(7):
                assert y[b, j, i] == x[b, i, j]


@pytest.mark.parametrize("shape", [(1, 9), (9, 1), (1, 1), (4, 4), (6, 10)])
def test_involution_and_unit_dims(shape):
    r = np.random.default_rng(6)
    x = r.standard_normal(shape).astype(np.float32)
    y = T.transpose(x)
    assert y.shape == shape[::-1]
    assert np.array_equal(T.transpose(y), x)
    # a row (column) vector keeps its values in order
    if 1 in shape:
        assert np.array_equal(y.reshape(-1), x.reshape(-1))


def test_values_are_copied_bit_for_bit():
    bits = np.array([[0x7FC00001, 0x80000000], [0x00000001, 0xFF800000]],
                    dtype=np.uint32)          # a NaN payload, -0, a denormal, -inf
    x = bits.view(np.float32)
    y = T.transpose(x)
    assert np.array_equal(y.view(np.uint32), bits.T)
