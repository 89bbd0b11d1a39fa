"""CPU oracle for the fp16-accumulating TN GEMM  D = A @ B^T.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this module; the HIP library
never calls it and shares no code with it.

What is computed.  Page "cute(8) smem_gemm" (yuyanqi.com, the kernel listing
and section 2.3) builds its GEMM from the MMA atom that takes fp16 A, B and
C and produces fp16 D, 16 deep in K: the accumulator fragment is half_t, so
after every 16-deep step of K the running sum is an fp16 value.  There is no
alpha, beta or C.  Per output element:

    acc_0 = 0
    acc_{s+1} = rn16(acc_s + sum_{k = 16 s}^{16 s + 15} a(i,k) b(j,k))
    d(i,j) = acc_{ceil(K / 16)}

with rn16 round-to-nearest-even to binary16 (overflow to +-inf) and the
16-term sum exact (float64 holds every fp16 product exactly, and the sums
here stay far inside its precision).  A K that is not a multiple of 16 ends
with a shorter step (the missing terms are zero).

Acceptance (`flip_bound`): a kernel may form each 16-term sum in fp32 before
the fp16 rounding; that can move a rounding decision by one fp16 spacing
when the pre-rounding value sits near a midpoint, and such a difference is
carried by the later steps.  The bound per element is the sum over steps of
the fp16 spacing at |acc_{s+1}|.  Integer-valued inputs make every step's
sum exact in fp32, so there the GPU result must equal the oracle bit for
bit.

Pins (tests/test_oracle_f16acc.py): a worked example under tests/golden/
whose partial sums pass 2048 (where fp16 stops holding every integer); a
closed form for constant inputs; a single step equals numpy's binary16
rounding of the exact product; small integer inputs with no rounding equal
the exact product; the step boundary (16 terms, not 1 or 32) decides a case
built to tell them apart; a pure-Python brute force on tiny inputs.
"""
from __future__ import annotations

import numpy as np

KSTEP = 16


def _rn16(x: np.ndarray) -> np.ndarray:
    """float64 -> the nearest binary16 value (ties to even), as float64."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(
            np.float64)


def gemm_tn_f16acc(A, B, kstep: int = KSTEP, with_steps: bool = False):
    """D (float16) for A (M, K) and B (N, K) float16, or batched (batch, M,
    K) and (batch, N, K).  with_steps also returns the list of acc_{s+1}
    arrays (float64), one per step."""
    A = np.asarray(A)
    B = np.asarray(B)
    two_d = A.ndim == 2
    if two_d:
        A, B = A[None], B[None]
    batch, M, K = A.shape
    if B.shape[0] != batch or B.shape[2] != K:
        raise ValueError("B must be (batch, N, K) with A's batch and K")
    a = A.astype(np.float64)
    b = B.astype(np.float64)
    acc = np.zeros((batch, M, B.shape[1]))
    steps = []
    for k0 in range(0, K, kstep):
        part = np.einsum("bik,bjk->bij", a[:, :, k0:k0 + kstep],
                         b[:, :, k0:k0 + kstep])
        acc = _rn16(acc + part)
        if with_steps:
            steps.append(acc.copy())
    d = acc.astype(np.float16)
    if two_d:
        d = d[0]
        steps = [s[0] for s in steps]
    return (d, steps) if with_steps else d


def spacing16(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 at |x| (x a binary16 value): 2^(max(e, -14) - 10)
    for |x| in [2^e, 2^(e+1)); the subnormal spacing 2^-24 below 2^-14."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, e - 1, -14)
    return np.ldexp(1.0, np.maximum(e, -14) - 10)


def flip_bound(A, B, kstep: int = KSTEP):
    """(D, bound): the oracle's D and, per element, the sum over steps of
    the fp16 spacing at the step's result."""
    d, steps = gemm_tn_f16acc(A, B, kstep, with_steps=True)
    bound = np.zeros(np.shape(d))
    for s in steps:
        bound = bound + spacing16(s)
    return d, bound
