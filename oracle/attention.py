"""CPU oracle for the attention forward pass  O = softmax(scale * Q K^T) V.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this module; the HIP library
never calls it and shares no code with it.

What is computed.  Page "为什么 cutlass_cute_tutorial_zh.md 中要用 retile_D"
(blog.qingsen.net, section 1) takes its example from a FlashAttention-style
tutorial: the score product score = Q @ K.T, with Q as the A operand and K
as the B operand of a TN MMA that accumulates in fp32 (section 2), head
dimension 64 (section 3).  The rest of that attention forward is the
textbook one: each row of scores is scaled, turned into probabilities by a
softmax (exponentials shifted by the row maximum, divided by their sum) and
the probabilities weight the rows of V.  Per batch entry (one head):

    S   = scale * Q K^T                     (Lq x Lk)
    P   = exp(S - rowmax S) / rowsum(...)   (Lq x Lk)
    O   = P V                               (Lq x dv)
    lse = rowmax S + log(rowsum(exp(S - rowmax S)))   (log-sum-exp of S)

Everything is float64: the fp16 inputs convert exactly, the matrix
products are library float64 products, exp and log are numpy's.  The
result stands for the exact one: its rounding error is far below the
acceptance bound below.

Acceptance bound (`bounds`): a first-order bound on the error of a kernel
that forms S in fp32 from exact fp16 products, computes the exponentials in
fp32 with a per-row shift, rounds the probabilities to fp16 for the P V
product, accumulates in fp32, and divides at the end by the row sum (an
fp32 sum of the probabilities, taken before or after their fp16 rounding);
doubled for second-order terms.  Its derivation is written out at `bounds`.

Pins (tests/test_oracle_attention.py): a hand-worked example under
tests/golden/, torch's scaled_dot_product_attention and scipy's logsumexp in
float64, closed forms (scale 0 averages V, one key returns its row of V, a
dominant key), invariances (joint key permutation, a shift of every key,
batches independent), a pure-Python brute force on tiny inputs, and scores
large enough to overflow an unshifted exponential.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x).astype(np.float64)


def _batched(Q, K, V):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    two_d = Q.ndim == 2
    if two_d:
        Q, K, V = Q[None], K[None], V[None]
    if K.shape[0] != Q.shape[0] or V.shape[0] != Q.shape[0]:
        raise ValueError("Q, K and V need the same batch")
    if K.shape[2] != Q.shape[2]:
        raise ValueError("Q and K need the same head dimension")
    if V.shape[1] != K.shape[1]:
        raise ValueError("K and V need the same number of keys")
    if K.shape[1] == 0:
        raise ValueError("softmax over zero keys is undefined")
    return Q, K, V, two_d


def attention(Q, K, V, scale: float):
    """(O, lse) in float64 for Q (batch, Lq, d), K (batch, Lk, d),
    V (batch, Lk, dv) (or the 2-D forms without batch).  lse is the natural
    log-sum-exp of each row of scale * Q K^T."""
    Q, K, V, two_d = _batched(Q, K, V)
    batch, Lq, _ = Q.shape
    O = np.empty((batch, Lq, V.shape[2]))
    lse = np.empty((batch, Lq))
    for b in range(batch):
        S = scale * (Q[b] @ K[b].T)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        P = E / l
        O[b] = P @ V[b]
        lse[b] = m[:, 0] + np.log(l[:, 0])
    return (O[0], lse[0]) if two_d else (O, lse)


def bounds(Q, K, V, scale: float):
    """Per-element error bounds (tol_O, tol_lse) for a GPU result, before
    the output rounding (the caller adds half an ulp of the output type).

    Write p_j = exp(S_j - m) / l (the exact probabilities of one row),
    W = sum_j p_j |v_j| (per output column), A_j = sum_i |q_i k_ji|,
    PA = sum_j p_j A_j, WA = sum_j p_j A_j |v_j|, c = |scale| * log2(e),
    u = 2^-24 (fp32 unit roundoff), and Lk, d the key count and head
    dimension.  To first order the kernel's weight of key j is
    p_j (1 + delta_j - delta_bar + theta_j - theta_bar - eta), where
      delta_j : fp16 rounding of the probability, |delta_j| <= 2^-11 (an
                absolute 2^-25 / l below fp16's normal range, l >= 1);
      delta_bar : the same roundings averaged into the row sum, when the
                sum is formed from the rounded probabilities (0 when it is
                formed in fp32 before rounding); sum_j p_j (delta_j -
                delta_bar) v_j = sum_j p_j delta_j (v_j - o), bounded by
                2^-11 (W + |o|) either way (o the exact output);
      theta_j : fp32 score error, |S_j error| <= (d - 1) u A_j, scaled by
                c ln 2 through exp2, plus the exp2 / shift roundings;
      theta_bar : the same errors averaged into the row sum;
      eta     : fp32 summation of the row sum, |eta| <= Lk u;
    and the fp32 P V accumulation adds at most Lk u W, each rescale of the
    accumulator by a new row maximum about 2^-22 (at most Lk / 64 + 8 of
    them).  Summing |weight error| |v_j| over j:
      B = 2^-11 (W + |o|) + W (2 Lk u + (Lk/64 + 8) 2^-22)
          + ln2 c (d - 1) u (WA + PA W) + Lk 2^-25 max|v|.
    tol_O = 2 B covers the second-order terms.  The log-sum-exp carries the
    row sum's relative error (delta_bar, theta_bar, eta) as an absolute one:
    tol_lse = 2 (2^-11 + Lk u + ln2 c (d - 1) u PA + 2^-19) + 2^-22 |lse|."""
    Q, K, V, two_d = _batched(Q, K, V)
    batch, Lq, d = Q.shape
    Lk = K.shape[1]
    u = 2.0 ** -24
    c = abs(scale) / math.log(2.0)
    tol_O = np.empty((batch, Lq, V.shape[2]))
    tol_lse = np.empty((batch, Lq))
    for b in range(batch):
        S = scale * (Q[b] @ K[b].T)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)
        Va = np.abs(V[b])
        A = np.abs(Q[b]) @ np.abs(K[b]).T
        W = P @ Va
        PA = (P * A).sum(axis=1, keepdims=True)
        WA = (P * A) @ Va
        score = math.log(2.0) * c * (d - 1) * u
        O = P @ V[b]
        B = (2.0 ** -11 * (W + np.abs(O))
             + W * (2 * Lk * u + (Lk / 64 + 8) * 2.0 ** -22)
             + score * (WA + PA * W)
             + Lk * 2.0 ** -25 * (Va.max() if Va.size else 0.0))
        tol_O[b] = 2.0 * B
        lse = S.max(axis=1) + np.log(E.sum(axis=1))
        tol_lse[b] = (2.0 * (2.0 ** -11 + Lk * u + score * PA[:, 0]
                             + 2.0 ** -19)
                      + 2.0 ** -22 * np.abs(lse))
    return (tol_O[0], tol_lse[0]) if two_d else (tol_O, tol_lse)


def half_ulp_f16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of binary16 at rn16(x) (the rounding error of a
    round-to-nearest fp16 output), taken at the rounded value so that a
    value rounding up across a binade uses the larger spacing."""
    r = np.abs(np.asarray(x, dtype=np.float64).astype(np.float16)
               .astype(np.float64))
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -14)))
    return 0.5 * 2.0 ** (e - 10)


def check(O_gpu, lse_gpu, Q, K, V, scale: float, out_dtype: str,
          ref=None):
    """Compare a GPU result with the oracle.  Returns a dict with the worst
    ratio |error| / tolerance for O and for lse (<= 1 passes) and the
    number of failing elements.  `ref` = (O, lse) reuses an oracle result."""
    O_ref, lse_ref = attention(Q, K, V, scale) if ref is None else ref
    tol_O, tol_lse = bounds(Q, K, V, scale)
    if out_dtype == "f16":
        tol_O = tol_O + half_ulp_f16(O_ref)
    elif out_dtype == "f32":
        tol_O = tol_O + 2.0 ** -24 * np.abs(O_ref)
    else:
        raise ValueError("out_dtype is 'f16' or 'f32'")
    err_O = np.abs(np.asarray(O_gpu, dtype=np.float64) - O_ref)
    r_O = err_O / tol_O
    out = {"O_ratio": float(np.nanmax(r_O)) if r_O.size else 0.0,
           "O_fail": int(np.count_nonzero(~(err_O <= tol_O)))}
    if lse_gpu is not None:
        err_l = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
        r_l = err_l / tol_lse
        out["lse_ratio"] = float(np.nanmax(r_l)) if r_l.size else 0.0
        out["lse_fail"] = int(np.count_nonzero(~(err_l <= tol_lse)))
    return out
