"""gemm_tn_ex_noalloc against gemm_tn_ex on the GPU: the same kernels with
the split-K partials in the library's fixed per-GPU scratch instead of the
allocated workspace must give the same bits.  Two calls in a row (the
second smaller), then a tail-split problem and two splits of the cost
model (the last filling the whole scratch), each compared bit for bit with
gemm_tn_ex on the same inputs."""
import numpy as np
import pytest

import seeded_inputs as si

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_fp16_amd as g
    return g


def _run(g, fn, w, D):
    A = torch.from_numpy(np.ascontiguousarray(w.A)).cuda()
    B = torch.from_numpy(np.ascontiguousarray(w.B)).cuda()
    st = fn(w.batch, w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, w.M * w.K,
            B.data_ptr(), w.K, w.N * w.K, 0.0, None, w.N, w.M * w.N,
            D.data_ptr(), w.N, w.M * w.N, g.GEMM_TN_F32,
            torch.cuda.current_stream().cuda_stream)
    assert st == g.OK, g.status_string(st)


# (M, N, K, plan the planner must choose): the skinny workload (4 slices,
# 8 MiB of partials), a smaller split (8 slices, 4 MiB), a tail split
# (the bottom tile row in 4 slices, 16.8 MB), and splits of the cost model
# (3 slices of 1536^2, 27 MiB; 16 slices of 1024^2, the whole 64 MiB)
CASES = [(128, 4096, 8192, "split=4"), (64, 2048, 4096, "split=8"),
         (4352, 4096, 2048, "tail_split=4"), (1536, 1536, 8192, "split=3"),
         (1024, 1024, 32768, "split=16")]


def test_noalloc_matches_gemm_tn_ex():
    g = _gpu()
    outs = []
    for M, N, K, plan in CASES:
        desc = g.describe(1, M, N, K, 0.0, "f32")
        print(f"[noalloc] {M}x{N}x{K}: {desc}", flush=True)
        assert plan in desc.split(), desc
        w = si.build(f"noalloc{M}", 1, M, N, K, 1.0, 0.0, "f32", "normal",
                     0x5EED0B00 + M)
        D_ref = torch.full((M, N), float("nan"), device="cuda")
        D_new = torch.full((M, N), float("nan"), device="cuda")
        _run(g, g.gemm_tn_ex, w, D_ref)
        _run(g, g.gemm_tn_ex_noalloc, w, D_new)
        torch.cuda.synchronize()
        ref = D_ref.cpu().numpy()
        assert np.isfinite(ref).all()
        assert np.array_equal(D_new.cpu().numpy().view(np.uint32),
                              ref.view(np.uint32)), (M, N, K)
        outs.append(ref)
    # the first problem again, after the others left their partials in the
    # shared scratch
    M, N, K, _ = CASES[0]
    w = si.build(f"noalloc{M}", 1, M, N, K, 1.0, 0.0, "f32", "normal",
                 0x5EED0B00 + M)
    D = torch.empty((M, N), device="cuda")
    _run(g, g.gemm_tn_ex_noalloc, w, D)
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy().view(np.uint32),
                          outs[0].view(np.uint32))
