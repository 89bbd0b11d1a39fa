"""Attention forward on the GPU against the float64 oracle, through the C
ABI: every output element within the oracle's derived bound (O and lse),
on seeded inputs from a few queries and keys up to the 64-head, 1024-query,
1024-key workload and the largest supported key count."""
import math

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as AT

pytestmark = pytest.mark.gpu


def _gpu():
    import dense_gemm_fp16_amd as g
    return g


def _say(msg):
    print(msg, flush=True)


def _qkv(batch, Lq, Lk, seed, mag=1.0, d=64):
    Q = si.make("normal", (batch, Lq, d), seed, si.TENSOR_Q, np.float16, mag)
    K = si.make("normal", (batch, Lk, d), seed, si.TENSOR_K, np.float16, mag)
    V = si.make("normal", (batch, Lk, d), seed, si.TENSOR_V, np.float16)
    return Q, K, V


def _run(Q, K, V, scale, out_dtype="f16"):
    import torch
    g = _gpu()
    t = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (Q, K, V)]
    dt = torch.float16 if out_dtype == "f16" else torch.float32
    O, lse = g.attention_fwd(*t, scale, out_dtype=dt, return_lse=True)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), lse.cpu().numpy()


def _check(Q, K, V, scale, out_dtype, label):
    _say(f"[attention] {label} {Q.shape} x {K.shape[1]} keys, scale {scale},"
         f" out {out_dtype}")
    O, lse = _run(Q, K, V, scale, out_dtype)
    r = AT.check(O, lse, Q, K, V, scale, out_dtype)
    assert r["O_fail"] == 0 and r["lse_fail"] == 0, r
    return O, lse


@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_small_workload(out_dtype):
    w = si.attention_workload("attn_small")
    _check(w.Q, w.K, w.V, w.scale, out_dtype, "attn_small")


@pytest.mark.parametrize("batch,Lq,Lk", [
    (1, 1, 1), (1, 1, 64), (1, 17, 5), (2, 128, 63), (1, 129, 65),
    (3, 200, 130), (1, 64, 1000), (2, 300, 4096), (1, 2, 10007),
])
def test_ragged_shapes(batch, Lq, Lk):
    Q, K, V = _qkv(batch, Lq, Lk, 1000 + Lq + Lk)
    _check(Q, K, V, 0.125, "f32", "ragged")


@pytest.mark.parametrize("scale,mag", [(-0.125, 1.0), (0.0, 1.0),
                                       (1.0, 1.0), (0.125, 3.0),
                                       (2.0, 2.0)])
def test_scales_and_magnitudes(scale, mag):
    # large scale * magnitude: peaked rows whose maximum moves between key
    # blocks; scale 0: every row averages V; negative: reversed order
    Q, K, V = _qkv(2, 150, 700, 2000, mag)
    _check(Q, K, V, scale, "f32", f"mag {mag}")


def test_rising_scores_move_the_row_shift():
    # scores that grow along the keys, so each block's maximum exceeds the
    # shift and the accumulators are rescaled
    Q, K, V = _qkv(1, 64, 512, 3000)
    ramp = np.linspace(0.0, 4.0, 512)[None, :, None]
    K = (K.astype(np.float64) + ramp * np.sign(
        Q.astype(np.float64).sum(axis=1, keepdims=True))).astype(np.float16)
    _check(Q, K, V, 0.5, "f32", "rising")


def test_full_size_workload():
    w = si.attention_workload("attn_64x1024")
    _check(w.Q, w.K, w.V, w.scale, "f16", "attn_64x1024")


def test_largest_key_count():
    # 2^23 keys (1 GiB each for K and V).  All keys zero but the last: query
    # row 0 (zeros) averages V; row 1 (ones) scores 64 on the last key and 0
    # elsewhere, so it returns V's last row up to exp(-64) * 2^23 ~ 1e-21.
    import torch
    g = _gpu()
    Lk, d = 2 ** 23, 64
    _say(f"[attention] largest key count {Lk}")
    q = torch.zeros((1, 2, d), dtype=torch.float16, device="cuda")
    q[0, 1] = 1.0
    k = torch.zeros((1, Lk, d), dtype=torch.float16, device="cuda")
    k[0, Lk - 1] = 8.0
    j = torch.arange(Lk, dtype=torch.int32, device="cuda")[:, None]
    x = torch.arange(d, dtype=torch.int32, device="cuda")[None, :]
    v = (((j + x) % 7) - 3).to(torch.float16)[None]
    del j, x
    O, lse = g.attention_fwd(q, k, v, 0.125, out_dtype=torch.float32,
                             return_lse=True)
    torch.cuda.synchronize()
    O = O.cpu().numpy()[0]
    lse = lse.cpu().numpy()[0]
    # column x of V cycles through -3..3; whole cycles of 7 keys sum to 0,
    # so the column sum is that of the last Lk mod 7 keys
    r = Lk % 7
    mean = np.array([sum(((Lk - r + i + x) % 7) - 3 for i in range(r))
                     for x in range(d)], dtype=np.float64) / Lk
    np.testing.assert_allclose(O[0], mean, rtol=0, atol=2e-4)
    last = (((Lk - 1 + np.arange(d)) % 7) - 3).astype(np.float64)
    np.testing.assert_allclose(O[1], last, rtol=0, atol=2e-4)
    np.testing.assert_allclose(lse[0], math.log(Lk), rtol=2e-6)
    np.testing.assert_allclose(lse[1], 64.0, rtol=2e-6)


def test_heads_are_independent_and_results_repeat():
    import torch
    g = _gpu()
    Q, K, V = _qkv(1, 300, 500, 4000)
    Q3 = np.concatenate([Q, Q * 0, Q])
    K3 = np.concatenate([K, K, K])
    V3 = np.concatenate([V, -V, V])
    t = [torch.from_numpy(x).cuda() for x in (Q3, K3, V3)]
    O1 = g.attention_fwd(*t, 0.125)
    O2 = g.attention_fwd(*t, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    assert torch.equal(O1[0], O1[2])
    # head 1: zero queries -> the mean of -V over the keys
    mean = -V[0].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(O1[1].float().cpu().numpy(),
                               np.broadcast_to(mean, (300, 64)),
                               atol=2e-3)


def test_many_heads_and_guard_bands():
    import torch
    g = _gpu()
    batch, Lq, Lk = 2049, 9, 33
    Q, K, V = _qkv(batch, Lq, Lk, 5000)
    pad = 4096
    buf = torch.full((pad + batch * Lq * 64 + pad,), 7.0, device="cuda")
    out = buf[pad:pad + batch * Lq * 64].view(batch, Lq, 64)
    lbuf = torch.full((pad + batch * Lq + pad,), 7.0, device="cuda")
    lse = lbuf[pad:pad + batch * Lq].view(batch, Lq)
    t = [torch.from_numpy(x).cuda() for x in (Q, K, V)]
    g.attention_fwd(*t, 0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    for b_ in (buf, lbuf):
        assert torch.all(b_[:pad] == 7.0) and torch.all(b_[-pad:] == 7.0)
    r = AT.check(out.cpu().numpy(), lse.cpu().numpy(), Q, K, V, 0.125, "f32")
    assert r["O_fail"] == 0 and r["lse_fail"] == 0, r


def test_2d_inputs_and_errors():
    import torch
    g = _gpu()
    Q, K, V = _qkv(1, 40, 70, 6000)
    t = [torch.from_numpy(x[0]).cuda() for x in (Q, K, V)]
    O = g.attention_fwd(*t, 0.3)
    torch.cuda.synchronize()
    r = AT.check(O.float().cpu().numpy()[None], None, Q, K, V, 0.3, "f16")
    assert r["O_fail"] == 0, r
    with pytest.raises(g.GemmError):
        g.attention_fwd(t[0], t[1][:0], t[2][:0], 0.3)       # no keys
    q128 = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(g.GemmError):
        g.attention_fwd(q128, q128, q128, 0.3)               # d = 128


def test_random_problems_within_the_bound():
    """Seeded random problems: batch, ragged query and key counts, scale
    (either sign), input magnitude and output type, each within the
    oracle's bound."""
    r = np.random.default_rng(0x5EED0089)
    for case in range(24):
        batch = int(r.integers(1, 4))
        Lq = int(r.integers(1, 300))
        Lk = int(r.integers(1, 900))
        scale = float(r.choice([0.125, -0.125, 0.3, 1.0, 0.05]))
        mag = float(r.choice([0.5, 1.0, 2.0]))
        out = "f16" if r.integers(0, 2) else "f32"
        Q, K, V = _qkv(batch, Lq, Lk, 5000 + case, mag)
        _check(Q, K, V, scale, out, f"random {case}")
