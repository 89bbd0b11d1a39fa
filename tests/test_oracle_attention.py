"""Pins of the attention-forward oracle and of its acceptance bound (CPU
only).  Each pin is fixed by something other than the oracle itself: hand
arithmetic, torch / scipy float64 routines, closed forms, invariances, and a
pure-Python brute force."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as AT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "attention_worked_examples.json")


def _rand(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal(shape) * scale).astype(np.float16)


def _inputs(batch, Lq, Lk, d, seed, dv=None, scale=1.0):
    return (_rand((batch, Lq, d), seed, scale),
            _rand((batch, Lk, d), seed + 1, scale),
            _rand((batch, Lk, dv or d), seed + 2))


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"],
                         ids=lambda c: c["name"])
def test_worked_examples(case):
    O, lse = AT.attention(np.array(case["Q"], np.float16),
                          np.array(case["K"], np.float16),
                          np.array(case["V"], np.float16), case["scale"])
    np.testing.assert_allclose(O, case["O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, case["lse"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape,scale", [((2, 7, 11, 8), 0.3),
                                         ((3, 64, 100, 64), 0.125),
                                         ((1, 33, 5, 16), -1.7)])
def test_against_torch_sdpa_and_scipy(shape, scale):
    batch, Lq, Lk, d = shape
    Q, K, V = _inputs(batch, Lq, Lk, d, 11, dv=d + 3)
    O, lse = AT.attention(Q, K, V, scale)
    t = [torch.from_numpy(x.astype(np.float64)) for x in (Q, K, V)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], scale=scale).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
    S = scale * np.einsum("bqd,bkd->bqk", Q.astype(np.float64),
                          K.astype(np.float64))
    np.testing.assert_allclose(lse, scipy.special.logsumexp(S, axis=2),
                               rtol=1e-13, atol=1e-12)


def test_scale_zero_averages_the_rows_of_v():
    Q, K, V = _inputs(2, 9, 13, 8, 3)
    O, lse = AT.attention(Q, K, V, 0.0)
    mean = V.astype(np.float64).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(O, np.broadcast_to(mean, O.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(13), atol=1e-13)


def test_one_key_returns_its_value_row():
    Q, K, V = _inputs(2, 6, 1, 8, 4)
    O, lse = AT.attention(Q, K, V, 0.7)
    np.testing.assert_array_equal(O, np.broadcast_to(
        V.astype(np.float64), O.shape))
    s = 0.7 * np.einsum("bqd,bkd->bqk", Q.astype(np.float64),
                        K.astype(np.float64))[..., 0]
    np.testing.assert_allclose(lse, s, atol=1e-13)


def test_dominant_key_wins():
    Q = np.ones((1, 3, 4), np.float16)
    K = np.zeros((1, 5, 4), np.float16)
    K[0, 2] = 8.0                     # score 32 above every other key
    V = _rand((1, 5, 6), 5)
    O, _ = AT.attention(Q, K, V, 4.0)  # scaled gap 128: exp(-128) ~ 3e-56
    np.testing.assert_allclose(O[0], np.broadcast_to(
        V[0, 2].astype(np.float64), (3, 6)), rtol=1e-14, atol=1e-14)


def test_large_scores_do_not_overflow():
    Q, K, V = _inputs(1, 4, 9, 8, 6, scale=8.0)
    O, lse = AT.attention(Q, K, V, 50.0)     # scores in the thousands
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    assert np.abs(lse).max() > 1000
    # the same softmax from the scores shifted by their exact row maximum
    S = 50.0 * np.einsum("bqd,bkd->bqk", Q.astype(np.float64),
                         K.astype(np.float64))
    P = scipy.special.softmax(S, axis=2)
    np.testing.assert_allclose(O, P @ V.astype(np.float64), rtol=1e-12,
                               atol=1e-12)


def test_joint_key_permutation_changes_nothing():
    Q, K, V = _inputs(2, 10, 17, 8, 7)
    perm = np.random.default_rng(1).permutation(17)
    O1, l1 = AT.attention(Q, K, V, 0.4)
    O2, l2 = AT.attention(Q, K[:, perm], V[:, perm], 0.4)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)
    # permuting only V must change the result (V rows are tied to keys)
    O3, _ = AT.attention(Q, K, V[:, perm], 0.4)
    assert np.abs(O3 - O1).max() > 1e-3


def test_shifting_every_key_shifts_only_lse():
    Q, _, V = _inputs(1, 8, 12, 4, 8)
    # keys on a coarse grid (multiples of 1/4), so that K + u is exact
    K = (np.random.default_rng(2).integers(-8, 9, (1, 12, 4)) / 4
         ).astype(np.float16)
    u = np.array([1, -2, 0.5, 3], np.float16)
    Ks = (K.astype(np.float32) + u).astype(np.float16)
    exact = np.abs(Ks.astype(np.float64) - K.astype(np.float64) - u) == 0
    assert exact.all()
    O1, l1 = AT.attention(Q, K, V, 0.5)
    O2, l2 = AT.attention(Q, Ks, V, 0.5)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-12)
    shift = 0.5 * Q[0].astype(np.float64) @ u.astype(np.float64)
    np.testing.assert_allclose(l2[0] - l1[0], shift, atol=1e-12)


def test_batches_are_independent():
    Q, K, V = _inputs(3, 5, 7, 8, 9)
    O, lse = AT.attention(Q, K, V, 0.9)
    for b in range(3):
        Ob, lb = AT.attention(Q[b], K[b], V[b], 0.9)
        np.testing.assert_array_equal(O[b], Ob)
        np.testing.assert_array_equal(lse[b], lb)


def test_brute_force_tiny():
    Q, K, V = _inputs(2, 3, 4, 2, 10, dv=3)
    scale = 0.8
    O, lse = AT.attention(Q, K, V, scale)
    for b in range(2):
        for i in range(3):
            s = [scale * sum(float(Q[b, i, x]) * float(K[b, j, x])
                             for x in range(2)) for j in range(4)]
            e = [math.exp(v) for v in s]
            tot = sum(e)
            assert lse[b, i] == pytest.approx(math.log(tot), abs=1e-13)
            for c in range(3):
                o = sum(e[j] / tot * float(V[b, j, c]) for j in range(4))
                assert O[b, i, c] == pytest.approx(o, abs=1e-13)


def test_zero_keys_is_rejected():
    with pytest.raises(ValueError):
        AT.attention(np.zeros((1, 2, 4), np.float16),
                     np.zeros((1, 0, 4), np.float16),
                     np.zeros((1, 0, 4), np.float16), 1.0)


# ---- the acceptance bound -------------------------------------------------

def _emulate(Q, K, V, scale, block=64, threshold=8.0, skip_rescale=False,
             pad_to_block=False, rounded_sum=False):
    """A float32 model of a blocked kernel: fp32 scores, exp2 with a lazily
    updated per-row shift, fp16 probabilities for P V, fp32 sums (of the
    fp16 probabilities with `rounded_sum`, else of the fp32 ones).  With
    `skip_rescale` the accumulator is not rescaled when the shift moves (a
    planted mistake); with `pad_to_block` the zero keys that pad the last
    block are not masked (another one)."""
    batch, Lq, d = Q.shape
    Lk = K.shape[1]
    c = np.float32(scale / math.log(2.0))
    O = np.zeros((batch, Lq, V.shape[2]), np.float32)
    lse = np.zeros((batch, Lq), np.float32)
    nb = -(-Lk // block)
    for b in range(batch):
        q = Q[b].astype(np.float32)
        m = None
        l = np.zeros(Lq, np.float32)
        acc = np.zeros((Lq, V.shape[2]), np.float32)
        for kb in range(nb):
            k = K[b, kb * block:(kb + 1) * block].astype(np.float32)
            v = V[b, kb * block:(kb + 1) * block].astype(np.float32)
            if pad_to_block and k.shape[0] < block:
                pad = block - k.shape[0]
                k = np.vstack([k, np.zeros((pad, d), np.float32)])
                v = np.vstack([v, np.zeros((pad, v.shape[1]), np.float32)])
            s = (q @ k.T).astype(np.float32) * c
            mb = s.max(axis=1)
            if m is None:
                m = mb
            else:
                grow = mb - m > threshold
                if grow.any():
                    mn = np.maximum(m, mb)
                    f = np.exp2(m - mn).astype(np.float32)
                    if not skip_rescale:
                        acc *= f[:, None]
                    l *= f
                    m = mn
            p = np.exp2(s - m[:, None]).astype(np.float32)
            p16 = p.astype(np.float16).astype(np.float32)
            l += (p16 if rounded_sum else p).sum(axis=1, dtype=np.float32)
            acc += p16 @ v
        O[b] = acc / l[:, None]
        lse[b] = m * np.float32(math.log(2.0)) + np.log(l)
    return O, lse


@pytest.mark.parametrize("shape,scale,mag", [((2, 40, 300, 64), 0.125, 1.0),
                                             ((1, 32, 200, 64), 1.0, 1.0),
                                             ((1, 16, 130, 64), 0.125, 3.0)])
def test_bound_accepts_a_float32_kernel_model(shape, scale, mag):
    batch, Lq, Lk, d = shape
    Q, K, V = _inputs(batch, Lq, Lk, d, 12, scale=mag)
    for rounded in (False, True):
        O, lse = _emulate(Q, K, V, scale, rounded_sum=rounded)
        for out in ("f32", "f16"):
            Oo = O if out == "f32" else O.astype(np.float16)
            r = AT.check(Oo, lse, Q, K, V, scale, out)
            assert r["O_fail"] == 0 and r["lse_fail"] == 0, r
            assert r["O_ratio"] < 0.5, r      # the bound is not tight


def test_bound_rejects_planted_mistakes():
    # scores that grow along the keys, so the shift moves between blocks
    Q, K, V = _inputs(1, 16, 200, 64, 13)
    ramp = np.linspace(0, 3, 200, dtype=np.float32)[None, :, None]
    K = (K.astype(np.float32) + ramp * np.sign(
        Q.astype(np.float32).sum(axis=1, keepdims=True))).astype(np.float16)
    scale = 0.5
    assert AT.check(*_emulate(Q, K, V, scale), Q, K, V, scale,
                    "f32")["O_fail"] == 0
    bad = _emulate(Q, K, V, scale, skip_rescale=True, threshold=0.0)
    assert AT.check(bad[0], None, Q, K, V, scale, "f32")["O_fail"] > 0
    # unmasked zero keys padding a ragged last block
    Q, K, V = _inputs(1, 8, 5, 64, 14)
    bad = _emulate(Q, K, V, 0.125, pad_to_block=True)
    r = AT.check(bad[0], bad[1], Q, K, V, 0.125, "f32")
    assert r["O_fail"] > 0 and r["lse_fail"] > 0
    # a dropped key, and exp taken in the wrong base
    O_drop, _ = AT.attention(Q, K[:, :4], V[:, :4], 0.125)
    assert AT.check(O_drop, None, Q, K, V, 0.125, "f32")["O_fail"] > 0
    O_base, _ = AT.attention(Q, K, V, 0.125 / math.log(2.0))
    assert AT.check(O_base, None, Q, K, V, 0.125, "f32")["O_fail"] > 0


SPACING = os.path.join(os.path.dirname(__file__), "golden",
                       "fp16_half_spacing.json")


@pytest.mark.parametrize("case", json.load(open(SPACING))["cases"],
                         ids=lambda c: c[0])
def test_half_ulp_f16_golden(case):
    """half_ulp_f16 against half-spacings worked by hand from the binary16
    definition, including values that round up across a binade boundary
    and the subnormal range, where the spacing stays 2^-24."""
    _, x, _, half = case
    assert AT.half_ulp_f16(np.array([x]))[0] == half
    assert AT.half_ulp_f16(np.array([-x]))[0] == half


def test_half_ulp_f16_matches_the_gemm_oracle_codec():
    """Across every finite binade (and below the normal range) the
    attention oracle's half spacing equals half of the GEMM oracle's ulp16
    taken at its own RNE encoding (both pinned separately: that codec
    against all 65536 patterns).  Values that round to infinity have no
    spacing and are left out."""
    import oracle
    r = np.random.default_rng(0x5EED0300)
    x = np.ldexp(r.uniform(1.0, 2.0, 20000), r.integers(-30, 16, 20000))
    x = np.concatenate([x, np.ldexp(1.0, np.arange(-30, 16)),
                        np.ldexp(1.0, np.arange(-30, 16)) * (1 - 2.0 ** -12)])
    x = x[x < 65520.0]
    x = np.where(r.integers(0, 2, x.size) == 1, -x, x)
    want = 0.5 * oracle.ulp16(oracle.decode_f16(oracle.rn16_bits(x)))
    np.testing.assert_array_equal(AT.half_ulp_f16(x), want)


def test_half_ulp_f16_pin_catches_an_exponent_off_by_one():
    """A half spacing one binade too large or too small (the kind of slip
    the formula invites) fails the golden table."""
    cases = json.load(open(SPACING))["cases"]
    x = np.array([c[1] for c in cases])
    want = np.array([c[3] for c in cases])
    good = AT.half_ulp_f16(x)
    assert np.array_equal(good, want)
    for wrong in (good * 2, good / 2):
        assert not np.array_equal(wrong, want)
    # the spacing at x instead of at rn16(x): misses the binade crossings
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    assert not np.array_equal(0.5 * 2.0 ** (e - 10), want)
