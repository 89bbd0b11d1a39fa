"""fp16-accumulating GEMM on the GPU against its oracle, through the C ABI.
Integer-valued inputs make every 16-deep step's sum exact in fp32, so the
result must equal the oracle bit for bit, also once the partial sums pass
2048 and the fp16 roundings start to bite; float inputs must fall within
the oracle's one-spacing-per-step bound and match exactly almost
everywhere."""
import numpy as np
import pytest

from oracle import gemm_f16acc as F

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    import dense_gemm_fp16_amd as g
    return g


def _say(msg):
    print(msg, flush=True)


def _run(A, B):
    g = _gpu()
    a = torch.from_numpy(np.ascontiguousarray(A)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(B)).cuda()
    d = g.gemm_tn_f16acc(a, b)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def _ints(shape, seed, lo=-3, hi=4):
    return np.random.default_rng(seed).integers(lo, hi, shape).astype(
        np.float16)


@pytest.mark.parametrize("shape", [
    (1, 128, 128, 32), (2, 300, 260, 832), (1, 64, 200, 1000),
    (3, 129, 131, 33), (1, 1, 1, 16), (1, 257, 5, 4096), (2, 70, 90, 37),
])
def test_integer_inputs_bit_exact(shape):
    batch, M, N, K = shape
    A, B = _ints((batch, M, K), sum(shape)), _ints((batch, N, K), 7 * M)
    _say(f"[f16acc] ints {shape}")
    np.testing.assert_array_equal(_run(A, B).view(np.uint16),
                                  F.gemm_tn_f16acc(A, B).view(np.uint16))


def test_partial_sums_past_2048_round_as_the_oracle_says():
    # positive integers in 1..3: the sums grow to about 8000, past 4096
    # where fp16 steps are 4
    A = _ints((1, 96, 2048), 11, 1, 4)
    B = _ints((1, 80, 2048), 12, 1, 4)
    ref = F.gemm_tn_f16acc(A, B)
    exact = np.einsum("bik,bjk->bij", A.astype(np.int64), B.astype(np.int64))
    assert np.abs(exact).min() > 4096
    assert np.any(ref.astype(np.int64) != exact)     # roundings happened
    _say("[f16acc] growing sums")
    np.testing.assert_array_equal(_run(A, B).view(np.uint16),
                                  ref.view(np.uint16))


def test_golden_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "gemm_f16acc_worked_example.json")))
    a = np.ones((2, 48), np.float16)
    a[1] = 2
    b = np.zeros((2, 48), np.float16)
    b[0, :15] = 127
    b[0, 15] = 142
    b[0, 16:20] = 1
    b[0, 32:35] = 1
    b[1, :32] = 62.5
    b[1, 32] = 49
    np.testing.assert_array_equal(_run(a, b).astype(np.float64), g["D"])


@pytest.mark.parametrize("shape", [(1, 256, 256, 1024), (2, 200, 300, 520)])
def test_float_inputs_within_the_flip_bound(shape):
    batch, M, N, K = shape
    r = np.random.default_rng(13)
    A = r.uniform(-1, 1, (batch, M, K)).astype(np.float16)
    B = r.uniform(-1, 1, (batch, N, K)).astype(np.float16)
    ref, bound = F.flip_bound(A, B)
    _say(f"[f16acc] floats {shape}")
    d = _run(A, B)
    err = np.abs(d.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bound), float((err / bound).max())
    assert np.mean(d.view(np.uint16) == ref.view(np.uint16)) > 0.99


def test_zero_k_broadcast_and_guard_bands():
    g = _gpu()
    M, N, K = 70, 66, 64
    A = _ints((1, M, K), 21)
    B = _ints((3, N, K), 22)
    a = torch.from_numpy(A).cuda().expand(3, M, K)     # stride 0 broadcast
    b = torch.from_numpy(B).cuda()
    pad = 512
    buf = torch.full((pad + 3 * M * N + pad,), 7.0, dtype=torch.float16,
                     device="cuda")
    out = buf[pad:pad + 3 * M * N].view(3, M, N)
    g.gemm_tn_f16acc(a, b, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 7) and torch.all(buf[-pad:] == 7)
    ref = F.gemm_tn_f16acc(np.broadcast_to(A, (3, M, K)), B)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16),
                                  ref.view(np.uint16))
    z = g.gemm_tn_f16acc(a[:, :, :0].contiguous(), b[:, :, :0].contiguous())
    torch.cuda.synchronize()
    assert torch.all(z == 0)


def test_unaligned_operands_take_the_element_loader():
    g = _gpu()
    M, N, K = 90, 70, 40
    A = _ints((M * K + 1,), 31)
    B = _ints((N * K + 1,), 32)
    a = torch.from_numpy(A).cuda()[1:].view(M, K)      # 2-byte offset
    b = torch.from_numpy(B).cuda()[1:].view(N, K)
    d = g.gemm_tn_f16acc(a, b)
    torch.cuda.synchronize()
    ref = F.gemm_tn_f16acc(A[1:].reshape(M, K), B[1:].reshape(N, K))
    np.testing.assert_array_equal(d.cpu().numpy().view(np.uint16),
                                  ref.view(np.uint16))


def test_overflow_to_infinity_stays_infinite():
    """An fp16 accumulator that passes 65504 becomes +-inf (round to
    nearest) and stays there, per element: row 0 overflows in the first
    16-deep step, row 1 in the fourth (sums 19200, 38400, 57600, 76800),
    row 2 to -inf, row 3 stays finite, and the columns of B flip signs or
    scale.  Both the direct and the element loader run it."""
    K = 64
    A = np.zeros((1, 4, K), np.float16)
    A[0, 0], A[0, 1], A[0, 2], A[0, 3] = 8192, 1200, -8192, 3
    B = np.ones((1, 3, K), np.float16)
    B[0, 1] = -1
    B[0, 2] = 0.5
    ref = F.gemm_tn_f16acc(A, B)
    assert np.isposinf(ref[0, 0, 0]) and np.isneginf(ref[0, 0, 1])
    assert np.isposinf(ref[0, 1, 0]) and ref[0, 1, 2] == 38400
    assert np.isneginf(ref[0, 2, 0]) and np.all(np.isfinite(ref[0, 3]))
    _say("[f16acc] overflow")
    np.testing.assert_array_equal(_run(A, B).view(np.uint16),
                                  ref.view(np.uint16))
    # odd K: the element loader
    A3, B3 = A[:, :, :63], B[:, :, :63]
    ref3 = F.gemm_tn_f16acc(A3, B3)
    np.testing.assert_array_equal(_run(A3, B3).view(np.uint16),
                                  ref3.view(np.uint16))


def test_random_integer_problems_bit_exact():
    """Seeded random shapes, batches and integer ranges (sums past 2048
    where the fp16 roundings act): bit-exact against the oracle."""
    r = np.random.default_rng(0x5EED008B)
    for case in range(24):
        batch = int(r.integers(1, 3))
        M, N = (int(v) for v in r.integers(1, 300, 2))
        K = int(r.integers(1, 1500))
        if case % 2:
            K = -(-K // 8) * 8          # rows that allow 16-byte loads
        hi = int(r.choice([4, 8]))
        A = _ints((batch, M, K), 8000 + case, -hi + 1, hi)
        B = _ints((batch, N, K), 9000 + case, -hi + 1, hi)
        _say(f"[f16acc random {case}] {(batch, M, N, K)} |x| < {hi}")
        np.testing.assert_array_equal(_run(A, B).view(np.uint16),
                                      F.gemm_tn_f16acc(A, B).view(np.uint16))
