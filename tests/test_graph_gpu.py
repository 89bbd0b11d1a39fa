"""Library calls captured into a HIP graph (torch.cuda.CUDAGraph) replay
correctly: every replay, with the program's own eager work and
synchronisations between replays, gives the eager result bit for bit.
Covers a plain call, one that reads C, a split-K call (tile kernel and
reduction through the per-stream workspace) and the same split-K problem
through gemm_tn_ex_noalloc (the fixed scratch)."""
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


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("name", ["c1_256", "c2_1024", "c4b_skinny"])
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager(name, noalloc):
    g = _gpu()
    w = si.workload(name)
    A, B, C = _dev(w.A[0]), _dev(w.B[0]), _dev(None if w.C is None else w.C[0])
    dt = torch.float16 if w.out_dtype == "f16" else torch.float32
    code = g.GEMM_TN_F16 if w.out_dtype == "f16" else g.GEMM_TN_F32
    M, N, K = w.M, w.N, w.K
    fn = g.gemm_tn_ex_noalloc if noalloc else g.gemm_tn_ex

    def call(D):
        st = fn(1, M, N, K, w.alpha, A.data_ptr(), K, M * K, B.data_ptr(), K,
                N * K, w.beta, C.data_ptr() if C is not None else None, N,
                M * N, D.data_ptr(), N, M * N, code,
                torch.cuda.current_stream().cuda_stream)
        assert st == g.OK, g.status_string(st)

    print(f"[graph] {name} noalloc={noalloc}: {g.describe(1, M, N, K, w.beta, w.out_dtype)}",
          flush=True)
    stream = torch.cuda.Stream()
    eager = torch.empty((M, N), dtype=dt, device="cuda")
    with torch.cuda.stream(stream):
        call(eager)                      # workspaces exist before capture
    stream.synchronize()
    want = eager.cpu().numpy()
    outs = [torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            for _ in range(2)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for D in outs:
            call(D)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for D in outs:
            D.fill_(float("nan"))
        junk.mul_(1.5).add_(1.0)         # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, D in enumerate(outs):
            got = D.cpu().numpy()
            assert np.array_equal(got.view(np.uint16 if dt == torch.float16
                                           else np.uint32),
                                  want.view(np.uint16 if dt == torch.float16
                                            else np.uint32)), (name, rep, i)
