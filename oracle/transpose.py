"""CPU oracle for the fp32 matrix transpose.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this module; the HIP library
never calls it and shares no code with it.

The operation is the one of page "Mat Transpose CuTe 版代码学习"
(chuoer47.github.io, the reg kernel and its host wrappers): x is an M x N
row-major matrix, y the N x M row-major matrix with y[j][i] = x[i][j];
every output element is a copy, so the GPU result must match bit for bit.
A batch of matrices is transposed matrix by matrix.

Pins (tests/test_oracle_transpose.py): a hand-written worked example under
tests/golden/, the element-by-element definition on a tiny brute-force
case, the involution y^T = x, and shapes with a unit dimension.
"""
from __future__ import annotations

import numpy as np


def transpose(x: np.ndarray) -> np.ndarray:
    """y[b, j, i] = x[b, i, j] for a (batch, M, N) or (M, N) array, written
    out one input row at a time: row i of x becomes column i of y."""
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    batch, M, N = x.shape
    y = np.empty((batch, N, M), dtype=x.dtype)
    for b in range(batch):
        for i in range(M):
            y[b, :, i] = x[b, i, :]
    return y[0] if squeeze else y
