"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Floating-point inputs must meet, element by element,
    |d - ref| <= 1e-3*|ref| + 1e-4*sqrt(K)  (+ half an fp16 ulp if D is fp16)
and integer-valued inputs in {-3..3} (exact in fp32 in any summation order)
must match the correctly rounded oracle bit for bit.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import seeded_inputs as si

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_fp16_amd as g
    return g


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dt(out):
    return torch.float16 if out == "f16" else torch.float32


def run_gpu(w, out=None, **kw):
    """Run workload w on the GPU; returns D as numpy (batch, M, N)."""
    g = _gpu()
    A = torch.from_numpy(np.ascontiguousarray(w.A)).cuda()
    B = torch.from_numpy(np.ascontiguousarray(w.B)).cuda()
    C = None
    if w.C is not None:
        C = torch.from_numpy(np.ascontiguousarray(w.C)).cuda()
    D = g.gemm_tn(A, B, w.alpha, w.beta, C, out=out,
                  out_dtype=_dt(w.out_dtype), **kw)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def sample_points(batch, M, N, n_random=4000, seed=0):
    """Whole rows and columns at the edges and inside, plus random points."""
    r = np.random.default_rng(seed)
    pts = []
    for b in sorted({0, batch - 1}):
        for i in sorted({0, M // 2 + 1, M - 1}):
            pts.append(np.stack([np.full(N, b), np.full(N, i), np.arange(N)], 1))
        for j in sorted({0, N // 3, N - 1}):
            pts.append(np.stack([np.full(M, b), np.arange(M), np.full(M, j)], 1))
    pts.append(np.stack([r.integers(0, batch, n_random),
                         r.integers(0, M, n_random),
                         r.integers(0, N, n_random)], 1))
    return np.concatenate(pts).astype(np.int64)


WORKLOADS = ["c1_256", "c2_1024", "c3_4096", "c4a_ragged", "c4b_skinny",
             "c5_qk"]


def full_check(w, d, exact):
    """Every element of d against the oracle, in blocks of at most 1024
    flattened rows (the 4096^3 and 64-batch results would otherwise hold
    several GiB of float64 temporaries).  Returns the first failing block's
    result, or the last block's."""
    flat = d.reshape(w.batch * w.M, w.N)
    step = 1024
    res = None
    for r0 in range(0, w.batch * w.M, step):
        r1 = min(r0 + step, w.batch * w.M)
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C, rows=(r0, r1))
        res = (oracle.check_exact(flat[r0:r1], ref, w.out_dtype) if exact
               else oracle.check(flat[r0:r1], ref, w.K, w.out_dtype))
        if not res.ok:
            res.worst_index = (r0 + res.worst_index[0],) + tuple(
                res.worst_index[1:])
            return res
    return res


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_tolerance(name):
    """Every element of every workload, at its full size, within the
    tolerance."""
    w = si.workload(name)
    _say(f"[parity] {name} {w.batch}x{w.M}x{w.N}x{w.K} out={w.out_dtype}")
    d = run_gpu(w)
    assert np.isfinite(d.astype(np.float64)).all()
    res = full_check(w, d, exact=False)
    _say(f"[parity] {name}: {res}")
    assert res.ok, str(res)


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_integer_bit_exact(name):
    """Every element of every workload's integer-valued variant, at its full
    size, bit for bit."""
    w = si.workload(name, int_values=True)
    _say(f"[exact] {name} {w.batch}x{w.M}x{w.N}x{w.K} out={w.out_dtype}")
    d = run_gpu(w)
    res = full_check(w, d, exact=True)
    _say(f"[exact] {name}: {res}")
    assert res.ok, str(res)


EDGE = [1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257]
EDGE_SHAPES = sorted({(m, n, k) for m, n, k in [
    *[(m, 64, 64) for m in EDGE], *[(64, n, 64) for n in EDGE],
    *[(64, 64, k) for k in EDGE], (1, 1, 1), (257, 255, 129), (129, 257, 65),
    (300, 260, 520), (513, 383, 200), (1, 777, 1024), (777, 1, 1024),
    (96, 80, 1000), (2, 3, 4097)]})


def _int_workload(batch, M, N, K, out, alpha=1.0, beta=0.0, seed=7):
    return si.build(f"edge{M}x{N}x{K}", batch, M, N, K, alpha, beta, out,
                    "int", seed + M * 7919 + N * 104729 + K, c_kind="int")


@pytest.mark.parametrize("out", ["f16", "f32"])
def test_edge_shapes_bit_exact(out):
    for (M, N, K) in EDGE_SHAPES:
        beta = 0.5 if (M + N) % 2 else 0.0
        w = _int_workload(1, M, N, K, out, alpha=1.5, beta=beta)
        _say(f"[edge] {M}x{N}x{K} out={out} beta={beta}")
        d = run_gpu(w)
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(d, ref, out)
        assert res.ok, f"{M}x{N}x{K} {out}: {res}"


CONFIGS = [f"tile={t},loader={l},split={s}" for t in (256, 128, 64)
           for l in (0, 1, 2) for s in (1, 3)] + [
    # the 256 tile of TN operands on eight waves (four is the default where
    # the output rows allow 16-byte stores)
    "tile=256,loader=0,split=1,w4=0", "tile=256,loader=0,split=3,w4=0"]


@pytest.mark.parametrize("spec", CONFIGS)
def test_every_kernel_configuration(spec, monkeypatch):
    """Each tile x loader x split-K instantiation on ragged shapes."""
    monkeypatch.setenv("GEMM_TN_FORCE", spec)
    for (batch, M, N, K, out, beta) in [(1, 300, 260, 832, "f16", 0.0),
                                        (1, 300, 264, 832, "f16", 0.5),
                                        (2, 129, 200, 1000, "f32", -2.0),
                                        (1, 512, 516, 768, "f32", 0.5)]:
        w = _int_workload(batch, M, N, K, out, alpha=0.5, beta=beta)
        _say(f"[config] {spec} {batch}x{M}x{N}x{K} {out}")
        d = run_gpu(w)
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(d, ref, out)
        assert res.ok, f"{spec} {M}x{N}x{K}: {res}"


FOUR_WAVE_SHAPES = [
    # (batch, M, N, K, out, alpha, beta)
    (1, 300, 264, 832, "f16", 1.0, 0.0),     # ragged M and N, alpha = 1
    (1, 257, 520, 1000, "f16", -1.5, 0.5),   # K tail (1000 = 15 x 64 + 40)
    (2, 129, 136, 72, "f32", 0.5, -2.0),     # two k-tiles, the second of 8
    (1, 256, 256, 64, "f16", 1.0, 0.0),      # exactly one k-tile
    (1, 256, 256, 8, "f32", 2.0, 0.0),       # K below one k-tile
    (3, 512, 256, 200, "f32", 1.0, 1.0),     # batches, several tiles
]


@pytest.mark.parametrize("shape", FOUR_WAVE_SHAPES)
def test_four_wave_kernel_bit_exact(shape, monkeypatch):
    """The 256 tile's four-wave kernel on ragged shapes: M and N tails,
    K tails and a single k-tile, batches, with and without C."""
    batch, M, N, K, out, alpha, beta = shape
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=256")
    desc = _gpu().describe(batch, M, N, K, beta, out)
    assert "sched=four-wave" in desc, desc
    w = _int_workload(batch, M, N, K, out, alpha=alpha, beta=beta)
    _say(f"[four-wave] {batch}x{M}x{N}x{K} {out} alpha={alpha} beta={beta}")
    d = run_gpu(w)
    ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
    res = oracle.check_exact(d, ref, out)
    assert res.ok, f"{shape}: {res}"


def test_four_wave_kernel_with_k_zero(monkeypatch):
    """An empty K range multiplies one tile of zeros: D = beta * C."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=256")
    assert "sched=four-wave" in g.describe(1, 300, 260, 0, 0.5, "f32")
    A = torch.empty(300, 0, dtype=torch.float16, device="cuda")
    B = torch.empty(260, 0, dtype=torch.float16, device="cuda")
    C = torch.randn(300, 260, device="cuda")
    D = g.gemm_tn(A, B, 2.0, -0.5, C)
    assert torch.equal(D, -0.5 * C)


def test_unaligned_operands_and_odd_k():
    g = _gpu()
    r = np.random.default_rng(3)
    M, N, K = 70, 90, 37
    A = r.integers(-3, 4, (M * K + 1)).astype(np.float16)
    B = r.integers(-3, 4, (N * K + 1)).astype(np.float16)
    At = torch.from_numpy(A).cuda()[1:].view(M, K)   # 2-byte aligned
    Bt = torch.from_numpy(B).cuda()[1:].view(N, K)
    D = g.gemm_tn(At, Bt, out_dtype=torch.float32)
    ref = oracle.gemm_tn(A[1:].reshape(M, K), B[1:].reshape(N, K))
    assert oracle.check_exact(D.cpu().numpy(), ref, "f32").ok
    # K multiple of 8 but misaligned base pointers
    K = 64
    A = r.integers(-3, 4, (M * K + 8)).astype(np.float16)
    B = r.integers(-3, 4, (N * K)).astype(np.float16)
    At = torch.from_numpy(A).cuda()[4:4 + M * K].view(M, K)  # 8-byte aligned
    Bt = torch.from_numpy(B).cuda().view(N, K)
    Dbuf = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    D = Dbuf[1:].view(M, N)                                  # 4-byte aligned
    g.gemm_tn(At, Bt, out=D)
    ref = oracle.gemm_tn(A[4:4 + M * K].reshape(M, K), B.reshape(N, K))
    assert oracle.check_exact(D.cpu().numpy(), ref, "f32").ok


def test_k_zero_gives_beta_c():
    g = _gpu()
    A = torch.empty(33, 0, dtype=torch.float16, device="cuda")
    B = torch.empty(17, 0, dtype=torch.float16, device="cuda")
    C = torch.randn(33, 17, device="cuda")
    D = g.gemm_tn(A, B, 2.0, -0.5, C)
    assert torch.equal(D, -0.5 * C)


def test_beta_zero_ignores_nan_c_and_overwrites_d():
    g = _gpu()
    w = _int_workload(1, 100, 120, 96, "f32")
    A = torch.from_numpy(w.A[0]).cuda()
    B = torch.from_numpy(w.B[0]).cuda()
    C = torch.full((100, 120), float("nan"), device="cuda")
    D = torch.full((100, 120), float("nan"), device="cuda")
    g.gemm_tn(A, B, 1.0, 0.0, C, out=D)
    d = D.cpu().numpy()
    assert np.isfinite(d).all()
    assert oracle.check_exact(d, oracle.gemm_tn(w.A[0], w.B[0]), "f32").ok


@pytest.mark.parametrize("out", ["f16", "f32"])
def test_c_may_alias_d(out):
    g = _gpu()
    w = _int_workload(1, 200, 136, 256, out, alpha=1.0, beta=-1.0)
    A = torch.from_numpy(w.A[0]).cuda()
    B = torch.from_numpy(w.B[0]).cuda()
    CD = torch.from_numpy(w.C[0].copy()).cuda()
    g.gemm_tn(A, B, 1.0, -1.0, CD, out=CD)
    ref = oracle.gemm_tn(w.A[0], w.B[0], 1.0, -1.0, w.C[0])
    assert oracle.check_exact(CD.cpu().numpy(), ref, out).ok


@pytest.mark.parametrize("shape", [(1, 130, 70, 200), (3, 64, 65, 64),
                                   (1, 128, 4096, 8192)])
def test_guard_bands_untouched(shape):
    """Nothing outside D is written (sentinels before and after it)."""
    g = _gpu()
    batch, M, N, K = shape
    w = _int_workload(batch, M, N, K, "f32")
    A = torch.from_numpy(w.A).cuda()
    B = torch.from_numpy(w.B).cuda()
    pad = 4096
    buf = torch.full((pad + batch * M * N + pad,), 12345.0, device="cuda")
    D = buf[pad:pad + batch * M * N].view(batch, M, N)
    g.gemm_tn(A, B, out=D)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)
    ref = oracle.gemm_tn(w.A, w.B)
    assert oracle.check_exact(D.cpu().numpy(), ref, "f32").ok


@pytest.mark.parametrize("name", ["c4b_skinny", "c3_4096", "c5_qk"])
def test_two_runs_are_bitwise_equal(name):
    w = si.workload(name)
    d1 = run_gpu(w)
    d2 = run_gpu(w)
    assert np.array_equal(d1.view(np.uint8), d2.view(np.uint8))


def test_batched_broadcast_operand():
    g = _gpu()
    batch, M, N, K = 5, 40, 48, 72
    w = _int_workload(batch, M, N, K, "f32")
    A = torch.from_numpy(w.A).cuda()
    B0 = torch.from_numpy(w.B[0]).cuda()
    D = torch.empty(batch, M, N, device="cuda")
    st = g.gemm_tn_strided_batched(
        batch, M, N, K, 1.0, A.data_ptr(), M * K, B0.data_ptr(), 0, 0.0,
        None, 0, D.data_ptr(), M * N, g.GEMM_TN_F32,
        torch.cuda.current_stream().cuda_stream)
    assert st == g.OK
    ref = oracle.gemm_tn(w.A, np.broadcast_to(w.B[0], (batch, N, K)))
    assert oracle.check_exact(D.cpu().numpy(), ref, "f32").ok


def test_fp16_overflow_rounds_to_inf():
    g = _gpu()
    K = 64
    A = torch.full((32, K), 40.0, dtype=torch.float16, device="cuda")
    B = torch.full((32, K), 30.0, dtype=torch.float16, device="cuda")
    D = g.gemm_tn(A, B, out_dtype=torch.float16)   # 76800 > 65504
    assert torch.isinf(D).all() and (D > 0).all()


def test_split_k_workspace_reuse(monkeypatch):
    """The split-K workspace is kept per stream and grown on demand: calls
    with more and fewer tiles, alternating between two streams, with C
    aliasing D, all stay exact."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=64,split=4")
    side = torch.cuda.Stream()
    shapes = [(1, 130, 200, 1024, "f32", 0.0), (2, 256, 320, 1100, "f16", 0.5),
              (1, 64, 64, 2048, "f32", -1.0), (3, 200, 136, 1024, "f32", 2.0),
              (1, 130, 200, 1024, "f32", 0.0)]
    for rep, (batch, M, N, K, out, beta) in enumerate(shapes):
        w = _int_workload(batch, M, N, K, out, alpha=0.5, beta=beta)
        stream = side if rep % 2 else torch.cuda.current_stream()
        _say(f"[split workspace] {batch}x{M}x{N}x{K} {out} beta={beta} "
             f"stream={'side' if rep % 2 else 'current'}")
        A = torch.from_numpy(w.A).cuda()
        B = torch.from_numpy(w.B).cuda()
        dt = torch.float16 if out == "f16" else torch.float32
        CD = (torch.from_numpy(w.C.copy()).cuda() if w.C is not None
              else torch.zeros(batch, M, N, dtype=dt, device="cuda"))
        torch.cuda.synchronize()
        st = g.gemm_tn_strided_batched(
            batch, M, N, K, w.alpha, A.data_ptr(), M * K, B.data_ptr(), N * K,
            w.beta, CD.data_ptr() if beta != 0.0 else None, M * N,
            CD.data_ptr(), M * N,
            g.GEMM_TN_F16 if out == "f16" else g.GEMM_TN_F32,
            stream.cuda_stream)
        assert st == g.OK
        torch.cuda.synchronize()
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(CD.cpu().numpy(), ref, out)
        assert res.ok, f"{batch}x{M}x{N}x{K}: {res}"


def test_split_k_from_several_threads(monkeypatch):
    """Host threads issuing split-K calls on one stream at once, each call
    larger than the last (the workspace keeps growing while other threads
    launch): every result exact.  The workspace lock is held until a call's
    kernels are enqueued, so a growing call's wait on the stream covers
    them before the old buffer is freed."""
    import threading
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=64,split=4")
    stream = torch.cuda.current_stream()
    jobs = []
    for t in range(4):
        for i in range(6):
            M = 64 + 48 * (6 * t + i)          # growing problems
            w = _int_workload(1, M, 96, 512, "f32", seed=100 * t + i)
            A = torch.from_numpy(w.A).cuda()
            B = torch.from_numpy(w.B).cuda()
            D = torch.full((1, M, 96), float("nan"), device="cuda")
            jobs.append((t, w, A, B, D))
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        for (tt, w, A, B, D) in jobs:
            if tt != t:
                continue
            st = g.gemm_tn_strided_batched(
                1, w.M, w.N, w.K, 1.0, A.data_ptr(), 0, B.data_ptr(), 0,
                0.0, None, 0, D.data_ptr(), 0, g.GEMM_TN_F32,
                stream.cuda_stream)
            if st != g.OK:
                errors.append((t, st))

    _say("[split threads] 4 threads x 6 growing split-K calls, one stream")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (t, w, A, B, D) in jobs:
        ref = oracle.gemm_tn(w.A, w.B)
        res = oracle.check_exact(D.cpu().numpy(), ref, "f32")
        assert res.ok, f"thread {t} M={w.M}: {res}"


def _padded(arr, ld, fill):
    """A (batch, rows, cols) array copied into a (batch, rows, ld) buffer
    whose padding columns hold `fill`."""
    batch, rows, cols = arr.shape
    buf = np.full((batch, rows, ld), fill, dtype=arr.dtype)
    buf[:, :, :cols] = arr
    return buf


LD_CASES = [
    # batch, M, N, K, out, beta, (pad_a, pad_b, pad_c, pad_d)
    (2, 300, 260, 832, "f16", 0.0, (8, 16, 0, 24)),      # 16-byte rows kept
    (2, 129, 200, 1000, "f32", -2.0, (8, 8, 4, 12)),
    (1, 70, 90, 37, "f32", 0.5, (3, 1, 5, 7)),           # odd row strides
    (3, 64, 66, 64, "f16", 0.0, (1, 8, 0, 2)),
]


@pytest.mark.parametrize("spec", CONFIGS)
def test_leading_dimensions(spec, monkeypatch):
    """gemm_tn_ex on row-strided sub-matrices: padding of A and B holds NaN
    (a read of it would poison the sums), padding of D holds a sentinel
    that must survive."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", spec)
    for (batch, M, N, K, out, beta, pads) in LD_CASES:
        w = _int_workload(batch, M, N, K, out, alpha=0.5, beta=beta)
        lda, ldb, ldc, ldd = K + pads[0], K + pads[1], N + pads[2], N + pads[3]
        dt = np.float16 if out == "f16" else np.float32
        A = torch.from_numpy(_padded(w.A, lda, np.nan)).cuda()
        B = torch.from_numpy(_padded(w.B, ldb, np.nan)).cuda()
        C = (torch.from_numpy(_padded(w.C, ldc, np.nan)).cuda()
             if w.C is not None else None)
        D = torch.from_numpy(_padded(np.zeros((batch, M, N), dt), ldd,
                                     dt(1234.0))).cuda()
        _say(f"[ld] {spec} {batch}x{M}x{N}x{K} {out} lds={lda},{ldb},{ldc},{ldd}")
        st = g.gemm_tn_ex(
            batch, M, N, K, w.alpha, A.data_ptr(), lda, M * lda, B.data_ptr(),
            ldb, N * ldb, w.beta, C.data_ptr() if C is not None else None, ldc,
            M * ldc, D.data_ptr(), ldd, M * ldd,
            g.GEMM_TN_F16 if out == "f16" else g.GEMM_TN_F32,
            torch.cuda.current_stream().cuda_stream)
        assert st == g.OK
        d = D.cpu().numpy()
        assert np.all(d[:, :, N:] == dt(1234.0)), "D padding was written"
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(np.ascontiguousarray(d[:, :, :N]), ref, out)
        assert res.ok, f"{spec} {M}x{N}x{K} lds {lda},{ldb},{ldc},{ldd}: {res}"


def test_binding_takes_row_slices():
    """The Python binding passes a tensor's row stride through, so column
    slices of wider arrays need no copy."""
    g = _gpu()
    w = _int_workload(1, 96, 80, 200, "f32", alpha=1.0, beta=1.0)
    Abig = torch.full((96, 256), float("nan"), dtype=torch.float16,
                      device="cuda")
    Bbig = torch.full((80, 208), float("nan"), dtype=torch.float16,
                      device="cuda")
    Abig[:, :200] = torch.from_numpy(w.A[0]).cuda()
    Bbig[:, :200] = torch.from_numpy(w.B[0]).cuda()
    Dbig = torch.full((96, 100), 7.0, device="cuda")
    C = torch.from_numpy(w.C[0]).cuda()
    g.gemm_tn(Abig[:, :200], Bbig[:, :200], 1.0, 1.0, C, out=Dbig[:, :80])
    d = Dbig.cpu().numpy()
    assert np.all(d[:, 80:] == 7.0)
    ref = oracle.gemm_tn(w.A[0], w.B[0], 1.0, 1.0, w.C[0])
    assert oracle.check_exact(np.ascontiguousarray(d[:, :80]), ref, "f32").ok


LAYOUT_CASES = [
    # batch, M, N, K, out, beta, row-stride padding of the stored A and B
    # M, N and strides multiples of 8: direct loads, transposing LDS reads
    (2, 256, 192, 320, "f16", 0.0, (8, 16)),
    (1, 520, 392, 1000, "f32", 0.5, (0, 8)),     # K tail, ragged tiles
    (1, 72, 136, 64, "f32", -1.0, (8, 0)),
    # otherwise the element loader
    (2, 300, 260, 832, "f16", 0.0, (8, 3)),
    (1, 129, 200, 1000, "f32", -2.0, (0, 0)),
    (3, 70, 90, 37, "f32", 0.5, (5, 1)),
]


@pytest.mark.parametrize("layouts", [(0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("spec", ["tile=256,split=1", "tile=128,split=3",
                                  "tile=64,split=1", "tile=64,split=3"])
def test_operands_stored_along_m_or_n(layouts, spec, monkeypatch):
    """A stored K x M and/or B stored K x N (gemm_tn_ex layouts), with
    padded row strides whose padding holds NaN."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", spec)
    la, lb = layouts
    for (batch, M, N, K, out, beta, pads) in LAYOUT_CASES:
        w = _int_workload(batch, M, N, K, out, alpha=0.5, beta=beta)
        # stored matrices: rows x row length, then padded
        As = np.ascontiguousarray(w.A.transpose(0, 2, 1)) if la else w.A
        Bs = np.ascontiguousarray(w.B.transpose(0, 2, 1)) if lb else w.B
        lda = As.shape[2] + pads[0]
        ldb = Bs.shape[2] + pads[1]
        A = torch.from_numpy(_padded(As, lda, np.nan)).cuda()
        B = torch.from_numpy(_padded(Bs, ldb, np.nan)).cuda()
        dt = np.float16 if out == "f16" else np.float32
        C = torch.from_numpy(w.C).cuda() if w.C is not None else None
        D = torch.empty((batch, M, N), dtype=torch.float16 if out == "f16"
                        else torch.float32, device="cuda")
        _say(f"[layout] {layouts} {spec} {batch}x{M}x{N}x{K} {out}")
        st = g.gemm_tn_ex(
            batch, M, N, K, w.alpha, A.data_ptr(), lda, As.shape[1] * lda,
            B.data_ptr(), ldb, Bs.shape[1] * ldb, w.beta,
            C.data_ptr() if C is not None else None, N, M * N, D.data_ptr(),
            N, M * N, g.GEMM_TN_F16 if out == "f16" else g.GEMM_TN_F32,
            torch.cuda.current_stream().cuda_stream, la, lb)
        assert st == g.OK
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(D.cpu().numpy().astype(dt), ref, out)
        assert res.ok, f"{layouts} {spec} {M}x{N}x{K}: {res}"


def test_binding_takes_transposed_views():
    """A transposed view (unit stride along M or N) is passed as an operand
    stored along M / N, without a copy."""
    g = _gpu()
    w = _int_workload(2, 96, 80, 200, "f32")
    At = torch.from_numpy(np.ascontiguousarray(
        w.A.transpose(0, 2, 1))).cuda()          # (batch, K, M)
    Bt = torch.from_numpy(np.ascontiguousarray(
        w.B.transpose(0, 2, 1))).cuda()          # (batch, K, N)
    ref = oracle.gemm_tn(w.A, w.B)
    for A, B in [(At.transpose(1, 2), torch.from_numpy(w.B).cuda()),
                 (torch.from_numpy(w.A).cuda(), Bt.transpose(1, 2)),
                 (At.transpose(1, 2), Bt.transpose(1, 2))]:
        D = g.gemm_tn(A, B, out_dtype=torch.float32)
        assert oracle.check_exact(D.cpu().numpy(), ref, "f32").ok


@pytest.mark.parametrize("spec", ["", "tile=64,split=1", "tile=128,split=1",
                                  "tile=256,split=1"])
def test_stored_along_m_or_n_matches_tn_at_scale(spec, monkeypatch):
    """Float operands stored along M / N at 2048 x 1536 x 4096 (64 k-tiles,
    tile loads in flight across every k-tile's fragment reads) give the
    TN kernel's result bit for bit: every storage sums each output in the
    same k order.  The planner's choice and each tile forced (the 64 and
    128 tiles run the interleaved loop, the 256 tile the ping-pong), fp16
    and fp32 D, every call twice.  Regression: the interleaved loop's last
    transposing reads (of a tile past the end) were left in flight into
    registers the epilogue reused; whole wave tiles of fp16 D came out
    wrong, differently from call to call."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", spec)
    gen = torch.Generator(device="cuda").manual_seed(0x5EED0077)
    M, N, K = 2048, 1536, 4096
    A = (torch.rand(M, K, device="cuda", generator=gen) * 2 - 1).half()
    B = (torch.rand(N, K, device="cuda", generator=gen) * 2 - 1).half()
    At, Bt = A.t().contiguous(), B.t().contiguous()     # K x M, K x N
    for dt in (torch.float16, torch.float32):
        ref = g.gemm_tn(A, B, out_dtype=dt)
        for la, lb in [(1, 0), (0, 1), (1, 1)]:
            _say(f"[layout at scale] {spec or 'planner'} {dt} "
                 f"a_mn={la} b_mn={lb}")
            for _ in range(2):
                d = g.gemm_tn(At.t() if la else A, Bt.t() if lb else B,
                              out_dtype=dt)
                torch.cuda.synchronize()
                assert torch.equal(d, ref), (dt, la, lb)


TAIL_SPECS = ["tile=64,tail=2,tail_split=3", "tile=128,tail=1,tail_split=2",
              "tile=256,tail=1,tail_split=4", "tile=64,loader=2,tail=3,tail_split=2"]


@pytest.mark.parametrize("spec", TAIL_SPECS)
def test_tail_split(spec, monkeypatch):
    """The bottom tile rows as a split-K problem of their own, the rows
    above as whole tiles: bit-exact on integer inputs, with C read, both
    output types, a batch, operands stored along M / N and padded rows."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", spec)
    for (batch, M, N, K, out, beta, la, lb, pad) in [
            (2, 600, 260, 1088, "f16", 0.0, 0, 0, 0),
            (1, 520, 200, 1152, "f32", -2.0, 1, 0, 8),
            (3, 300, 136, 1024, "f32", 0.5, 0, 1, 16),
            (1, 517, 133, 1031, "f32", 0.5, 1, 1, 3)]:
        w = _int_workload(batch, M, N, K, out, alpha=0.5, beta=beta)
        As = np.ascontiguousarray(w.A.transpose(0, 2, 1)) if la else w.A
        Bs = np.ascontiguousarray(w.B.transpose(0, 2, 1)) if lb else w.B
        lda, ldb, ldd = As.shape[2] + pad, Bs.shape[2] + pad, N + pad
        dt = np.float16 if out == "f16" else np.float32
        A = torch.from_numpy(_padded(As, lda, np.nan)).cuda()
        B = torch.from_numpy(_padded(Bs, ldb, np.nan)).cuda()
        C = torch.from_numpy(w.C).cuda() if w.C is not None else None
        D = torch.from_numpy(_padded(np.zeros((batch, M, N), dt), ldd,
                                     dt(1234.0))).cuda()
        desc = g.describe(batch, M, N, K, beta, out, pad % 8 == 0,
                          lds=(lda, ldb, N, ldd), layouts=(la, lb),
                          strides=(As.shape[1] * lda, Bs.shape[1] * ldb,
                                   M * N, M * ldd))
        _say(f"[tail] {spec} {batch}x{M}x{N}x{K} {out} layouts {la}{lb} "
             f"pad {pad}: {desc}")
        assert "tail_rows=0" not in desc, desc
        st = g.gemm_tn_ex(
            batch, M, N, K, w.alpha, A.data_ptr(), lda, As.shape[1] * lda,
            B.data_ptr(), ldb, Bs.shape[1] * ldb, w.beta,
            C.data_ptr() if C is not None else None, N, M * N, D.data_ptr(),
            ldd, M * ldd, g.GEMM_TN_F16 if out == "f16" else g.GEMM_TN_F32,
            torch.cuda.current_stream().cuda_stream, la, lb)
        assert st == g.OK
        d = D.cpu().numpy()
        assert np.all(d[:, :, N:] == dt(1234.0)), "D padding was written"
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(np.ascontiguousarray(d[:, :, :N]), ref, out)
        assert res.ok, f"{spec} {batch}x{M}x{N}x{K}: {res}"


# (batch, M, N, K, out, alpha, beta, tile, split the cost model picks)
COST_MODEL_CASES = [
    (1, 768, 768, 4096, "f32", 1.0, 0.0, 64, 3),
    (2, 1000, 1100, 4096, "f16", 0.5, 0.0, 128, 3),     # 16-byte stores off
    (1, 1000, 1000, 16000, "f32", 1.0, -1.0, 128, 8),
    (1, 300, 3000, 8192, "f32", 2.0, 0.0, 128, 7),
    (1, 320, 320, 24576, "f32", 1.0, 0.5, 64, 20),     # 20 slices: 8 + 8 + 3
    (1, 2000, 2100, 8200, "f16", 1.0, 0.5, 256, 3),     # eight waves
    (1, 2000, 2100, 8200, "f32", 1.0, 0.5, 256, 3),     # four waves
    (1, 3072, 3072, 2048, "f16", 1.0, 0.0, 256, 1),     # a partial wave
]


@pytest.mark.parametrize("case", COST_MODEL_CASES)
def test_cost_model_plans_bit_exact(case):
    """The plans the cost model picks for long K (every tile, split and
    unsplit, ragged M, N and K, with and without C), every element bit for
    bit on integer inputs."""
    batch, M, N, K, out, alpha, beta, tile, split = case
    g = _gpu()
    desc = dict(kv.split("=") for kv in
                g.describe(batch, M, N, K, beta, out).split())
    assert desc["tile"].startswith(f"{tile}x") and \
        desc["split"] == str(split), desc
    w = _int_workload(batch, M, N, K, out, alpha=alpha, beta=beta)
    _say(f"[model] {batch}x{M}x{N}x{K} {out}: {desc['tile']} split {split}")
    d = run_gpu(w)
    res = full_check(w, d, exact=True)
    assert res.ok, f"{case}: {res}"


def test_tail_split_chosen_by_the_planner():
    """4352^3 leaves a tail of 33 tiles of 256 after one wave: the planner
    splits the last two tile rows 4 ways; every element checked."""
    g = _gpu()
    M = N = 4352
    K = 4096
    desc = dict(kv.split("=") for kv in g.describe(1, M, N, K, 0.0, "f32").split())
    assert desc["tail_rows"] == "2" and desc["tail_split"] == "4", desc
    w = _int_workload(1, M, N, K, "f32", alpha=1.0, beta=0.0)
    _say(f"[tail] planner {M}x{N}x{K}: {desc}")
    d = run_gpu(w)
    res = full_check(w, d, exact=True)
    assert res.ok, str(res)


@pytest.mark.parametrize("spec", ["", "tile=64,split=1"])
def test_largest_k(spec, monkeypatch):
    """K = 2^21, the largest supported: values in {-1, 0, 1} keep every sum
    exact in fp32 (|sum| <= 2^21 < 2^24).  The planner splits K into many
    slices; the forced single slice walks all 32768 k-tiles in one
    workgroup."""
    if spec:
        monkeypatch.setenv("GEMM_TN_FORCE", spec)
    M, N, K = 16, 24, 2 ** 21
    w = si.build("maxk", 1, M, N, K, 1.0, 0.0, "f32", "int", 0x5EED0A01)
    w.A = (w.A.astype(np.float32) // 2).clip(-1, 1).astype(np.float16)
    w.B = (w.B.astype(np.float32) // 2).clip(-1, 1).astype(np.float16)
    _say(f"[max] K={K} {spec or 'planner'}: {_gpu().describe(1, M, N, K, 0.0, 'f32')}")
    d = run_gpu(w)
    ref = oracle.gemm_tn(w.A, w.B)
    res = oracle.check_exact(d, ref, "f32")
    assert res.ok, str(res)


@pytest.mark.parametrize("K", [2 ** 16, 2 ** 16 + 40])
def test_four_wave_kernel_long_k(K, monkeypatch):
    """The four-wave 256 tile over 1024 k-tiles: whole tiles take the loads
    with the k offset in the scalar offset (K = 2^16), a K tail the per-lane
    form; values in {-1, 0, 1} keep every sum exact."""
    monkeypatch.setenv("GEMM_TN_FORCE", "tile=256,split=1")
    M = N = 256
    desc = _gpu().describe(1, M, N, K, 0.0, "f32")
    assert "sched=four-wave" in desc and "split=1" in desc.split(), desc
    w = si.build("longk", 1, M, N, K, 1.0, 0.0, "f32", "int", 0x5EED0A02)
    w.A = (w.A.astype(np.float32) // 2).clip(-1, 1).astype(np.float16)
    w.B = (w.B.astype(np.float32) // 2).clip(-1, 1).astype(np.float16)
    _say(f"[four-wave] K={K}: {desc}")
    d = run_gpu(w)
    ref = oracle.gemm_tn(w.A, w.B)
    res = oracle.check_exact(d, ref, "f32")
    assert res.ok, str(res)


def test_largest_n_and_a_long_m():
    """N = 2^20, the largest supported, and M past a million rows
    (sampled), on integer values."""
    w = _int_workload(1, 8, 2 ** 20, 64, "f32")
    _say(f"[max] N={w.N}")
    d = run_gpu(w)
    ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
    res = oracle.check_exact(d, ref, "f32")
    assert res.ok, str(res)
    w = _int_workload(1, 2 ** 20 + 5, 24, 16, "f16", alpha=1.0)
    _say(f"[max] M={w.M}")
    d = run_gpu(w)
    res = full_check(w, d, exact=True)
    assert res.ok, str(res)


RANDOM_SPECS = ["", "tile=256,split=1", "tile=128,split=2", "tile=64,split=1",
                "tile=64,split=3", "tile=128,loader=1", "tile=64,loader=2",
                "tile=256,tail=1,tail_split=2", "tile=64,tail=1,tail_split=3"]


def test_random_problems_bit_exact(monkeypatch):
    """Seeded random problems through gemm_tn_ex: batch, ragged M / N / K,
    both storages of A and B, padded row strides (padding of A, B and C
    holds NaN, padding of D a sentinel), pointers off 16-byte alignment,
    alpha / beta, fp16 or fp32 D and a forced kernel configuration (or the
    planner's).  Integer inputs: bit-exact against the oracle, D's padding
    untouched."""
    g = _gpu()
    r = np.random.default_rng(0x5EED0088)
    for case in range(80):
        batch = int(r.integers(1, 4))
        M, N = (int(x) for x in r.integers(1, 400, 2))
        K = int(r.integers(1, 1200))
        la, lb = (int(x) for x in r.integers(0, 2, 2))
        out = "f16" if r.integers(0, 2) else "f32"
        alpha = float(r.choice([1.0, 0.5, 1.5, -2.0]))
        beta = float(r.choice([0.0, 0.0, 0.5, -1.0]))
        pads = [int(x) for x in r.integers(0, 17, 4)]
        shift = [int(x) for x in r.integers(0, 2, 2)]  # elements off alignment
        spec = str(r.choice(RANDOM_SPECS))
        if case % 2:
            # sizes, strides and pointers that allow 16-byte loads: the
            # direct loader, transposing LDS reads and the tail split
            M, N, K = (-(-x // 8) * 8 for x in (M, N, K))
            pads = [8 * (x // 8) for x in pads]
            shift = [0, 0]
        monkeypatch.setenv("GEMM_TN_FORCE", spec)
        w = _int_workload(batch, M, N, K, out, alpha=alpha, beta=beta,
                          seed=case)
        As = np.ascontiguousarray(w.A.transpose(0, 2, 1)) if la else w.A
        Bs = np.ascontiguousarray(w.B.transpose(0, 2, 1)) if lb else w.B
        lda, ldb = As.shape[2] + pads[0], Bs.shape[2] + pads[1]
        ldc, ldd = N + pads[2], N + pads[3]
        dt = np.float16 if out == "f16" else np.float32
        # one element of slack in front of A and B for the shifted pointer
        Ab = _padded(As, lda, np.nan).reshape(-1)
        Bb = _padded(Bs, ldb, np.nan).reshape(-1)
        A = torch.from_numpy(np.concatenate([np.full(shift[0], np.nan,
                                                     np.float16), Ab])).cuda()
        B = torch.from_numpy(np.concatenate([np.full(shift[1], np.nan,
                                                     np.float16), Bb])).cuda()
        C = (torch.from_numpy(_padded(w.C, ldc, np.nan)).cuda()
             if w.C is not None else None)
        D = torch.from_numpy(_padded(np.zeros((batch, M, N), dt), ldd,
                                     dt(1234.0))).cuda()
        _say(f"[random {case}] {spec or 'planner'} {batch}x{M}x{N}x{K} "
             f"lay={la}{lb} out={out} a={alpha} b={beta} pads={pads} "
             f"shift={shift}")
        st = g.gemm_tn_ex(
            batch, M, N, K, alpha, A.data_ptr() + 2 * shift[0], lda,
            As.shape[1] * lda, B.data_ptr() + 2 * shift[1], ldb,
            Bs.shape[1] * ldb, beta, C.data_ptr() if C is not None else None,
            ldc, M * ldc, D.data_ptr(), ldd, M * ldd,
            g.GEMM_TN_F16 if out == "f16" else g.GEMM_TN_F32,
            torch.cuda.current_stream().cuda_stream, la, lb)
        assert st == g.OK, (case, st)
        d = D.cpu().numpy()
        assert np.all(d[:, :, N:] == dt(1234.0)), f"case {case}: D padding"
        ref = oracle.gemm_tn(w.A, w.B, alpha, beta, w.C)
        res = oracle.check_exact(np.ascontiguousarray(d[:, :, :N]), ref, out)
        assert res.ok, f"case {case}: {res}"


def _signed_zero_problem(out):
    """Integer problem whose outputs include exact-zero sums formed every
    way the kernels can form them: all-zero products of either sign, a
    multi-term cancellation inside one MFMA k-step, and cancellations
    across k-steps, across k-tiles and across split-K slices (+260 then
    -260 over K = 520); C holds zeros of both signs."""
    r = np.random.default_rng(0x5EED0A55)
    M, N, K = 96, 80, 520
    A = r.integers(-3, 4, (M, K)).astype(np.float16)
    B = r.integers(-3, 4, (N, K)).astype(np.float16)
    A[0] = 0.0
    A[1] = np.float16(-0.0)
    A[2] = 1.0
    B[0] = -1.0
    B[1, :260], B[1, 260:] = 1.0, -1.0          # slices / k-tiles
    B[2] = 0.0
    B[2, 0], B[2, 1:4] = 3.0, -1.0              # inside one k-step
    B[3] = 0.0
    B[3, 5], B[3, 40] = 2.0, -2.0               # across k-steps
    B[4] = 0.0
    B[4, 10], B[4, 500] = 1.0, -1.0             # across k-tiles
    B[5] = np.float16(-0.0)
    dt = np.float16 if out == "f16" else np.float32
    C = r.integers(-3, 4, (M, N)).astype(dt)
    C[(C == 0) & (r.integers(0, 2, (M, N)) == 1)] = dt(-0.0)
    return A, B, C


SIGNED_ZERO_SPECS = ["", "tile=256,tail=1,tail_split=2",
                     "tile=64,tail=1,tail_split=3"] + CONFIGS


@pytest.mark.parametrize("spec", SIGNED_ZERO_SPECS)
def test_signed_zero_bit_exact(spec, monkeypatch):
    """The sign of every exact zero matches the oracle bit for bit on every
    kernel configuration (tile, loader, split-K, tail split), output type,
    sign of alpha and beta term.  In round-to-nearest a sum that starts at
    +0 and cancels is +0 in any order, so the sign is unique; an earlier
    version of the bit-exact check accepted either sign, which this test
    would now catch."""
    g = _gpu()
    if spec:
        monkeypatch.setenv("GEMM_TN_FORCE", spec)
    for out in ("f16", "f32"):
        A, B, C = _signed_zero_problem(out)
        At, Bt, Ct = (torch.from_numpy(x).cuda() for x in (A, B, C))
        for alpha in (1.0, -1.5):
            for beta in (0.0, 0.5, -1.0):
                _say(f"[signed zero] {spec or 'planner'} out={out} "
                     f"alpha={alpha} beta={beta}")
                D = g.gemm_tn(At, Bt, alpha, beta, Ct if beta else None,
                              out_dtype=_dt(out))
                torch.cuda.synchronize()
                ref = oracle.gemm_tn(A, B, alpha, beta, C if beta else None)
                zeros = int((ref == 0).sum())
                assert zeros > 50
                res = oracle.check_exact(D.cpu().numpy(), ref, out)
                assert res.ok, f"{spec} {out} a={alpha} b={beta}: {res}"


def _cancelling_problem(batch, M, N, K, seed):
    """Integer A = [X, X] and B = [Y, -Y] (halves along K): every output is
    an exact zero, reached from the nonzero partial sum X Y^T of the first
    half, and an exact zero at every position of every wave's sub-tile.
    (N a multiple of 8 keeps fp16 rows 16-byte aligned: the staged
    epilogue with 16-byte stores.)"""
    r = np.random.default_rng(seed)
    vals = np.array([-3, -2, -1, 1, 2, 3])
    X = r.choice(vals, (batch, M, K // 2))
    Y = r.choice(vals, (batch, N, K // 2))
    A = np.concatenate([X, X], axis=2).astype(np.float16)
    B = np.concatenate([Y, -Y], axis=2).astype(np.float16)
    return A, B


CANCEL_CASES = ([(spec, (1, 300, 296, 520)) for spec in
                 ["", "tile=256,tail=1,tail_split=2",
                  "tile=64,tail=1,tail_split=3"] + CONFIGS]
                + [("onek=1", (2, 300, 296, 64)), ("onek=0", (2, 300, 296, 64))]
                # rows of 300 fp16 elements rule out 16-byte stores: the
                # element-wise epilogues
                + [(spec, (1, 300, 300, 520)) for spec in
                   ["", "tile=256,loader=0,split=1", "tile=128,loader=0,split=1",
                    "tile=64,loader=0,split=1", "tile=64,loader=0,split=3"]])


@pytest.mark.parametrize("spec,shape", CANCEL_CASES)
def test_cancelling_sums_keep_the_sign_of_zero(spec, shape, monkeypatch):
    """alpha * (an exactly cancelling sum) is alpha * (+0): -0 for negative
    alpha, at every output position, fp16 and fp32, with and without a
    beta term on zeros of both signs.  Regression: hipcc selected the fp16
    epilogue's (half)(x * alpha) of one accumulator per 256-tile wave as a
    mixed FMA with a +0 addend, which gave +0 where -0 is the result."""
    g = _gpu()
    if spec:
        monkeypatch.setenv("GEMM_TN_FORCE", spec)
    batch, M, N, K = shape
    A, B = _cancelling_problem(batch, M, N, K, 0x5EED0C0 + K)
    At, Bt = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    r = np.random.default_rng(0x5EED0C1)
    for out in ("f16", "f32"):
        dt = np.float16 if out == "f16" else np.float32
        C = np.where(r.integers(0, 2, (batch, M, N)) == 1, dt(-0.0), dt(0.0))
        Ct = torch.from_numpy(C).cuda()
        for alpha in (1.0, -1.5):
            for beta in (0.0, 0.5):
                _say(f"[cancelling] {spec or 'planner'} {shape} out={out} "
                     f"alpha={alpha} beta={beta}")
                D = g.gemm_tn(At, Bt, alpha, beta, Ct if beta else None,
                              out_dtype=_dt(out))
                torch.cuda.synchronize()
                ref = oracle.gemm_tn(A, B, alpha, beta, C if beta else None)
                assert not ref.any()
                res = oracle.check_exact(D.cpu().numpy(), ref, out)
                assert res.ok, f"{spec} {out} a={alpha} b={beta}: {res}"


ONEK_SHAPES = [(1, 300, 260, 64), (3, 129, 250, 8), (2, 1024, 1024, 64),
               (1, 4000, 136, 24), (5, 64, 64, 40), (1, 1, 1, 8)]


@pytest.mark.parametrize("out", ["f16", "f32"])
def test_onek_kernel_bit_exact(out, monkeypatch):
    """The persistent kernel for K <= 64 (a workgroup walks a run of tiles,
    loading the next tile's operands while the current one's results are
    written) forced onto ragged shapes: M and N tails, K below one
    k-tile, batches, fewer tiles than XCDs, with and without C."""
    g = _gpu()
    monkeypatch.setenv("GEMM_TN_FORCE", "onek=1")
    for i, (batch, M, N, K) in enumerate(ONEK_SHAPES):
        beta = -0.5 if i % 2 else 0.0
        w = _int_workload(batch, M, N, K, out, alpha=1.5, beta=beta)
        desc = g.describe(batch, M, N, K, beta, out)
        # 16-byte output rows: N a multiple of 8 (fp16) or 4 (fp32)
        if (N * (2 if out == "f16" else 4)) % 16:
            assert "persistent-onek" not in desc, desc
            continue
        assert "persistent-onek" in desc, desc
        _say(f"[onek] {batch}x{M}x{N}x{K} {out} beta={beta}: {desc}")
        d = run_gpu(w)
        ref = oracle.gemm_tn(w.A, w.B, w.alpha, w.beta, w.C)
        res = oracle.check_exact(d, ref, out)
        assert res.ok, f"{batch}x{M}x{N}x{K} {out}: {res}"


def test_onek_kernel_is_planned_for_the_score_product():
    g = _gpu()
    assert "persistent-onek" in g.describe(64, 1024, 1024, 64, 0.0, "f32")
