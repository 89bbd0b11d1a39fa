"""The seeded generator: SplitMix64 known answers and value ranges."""
import numpy as np

import seeded_inputs as si


def test_splitmix64_known_answer():
    # Published SplitMix64 sequence for start state 1234567 (the reference
    # C implementation by Vigna, counter form: mix64(s + i * GAMMA)).
    seed = np.uint64(1234567)
    with np.errstate(over="ignore"):
        ctr = seed + np.arange(1, 6, dtype=np.uint64) * si.GAMMA
    got = [int(v) for v in si.mix64(ctr)]
    assert got == [6457827717110365317, 3203168211198807973,
                   9817491932198370423, 4593380528125082431,
                   16408922859458223821]


def test_streams_differ_and_repeat():
    a = si.stream(7, si.TENSOR_A, 1000)
    b = si.stream(7, si.TENSOR_B, 1000)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, si.stream(7, si.TENSOR_A, 1000))
    # a prefix of a longer stream is the shorter stream
    assert np.array_equal(a[:10], si.stream(7, si.TENSOR_A, 10))


def test_value_maps():
    u = si.uniform_pm1(1, 0, 100000)
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 0.02
    z = si.normal01(1, 0, 100000)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1.0) < 0.02
    i = si.small_ints(1, 0, 10000)
    assert set(np.unique(i)) == set(range(-3, 4))


def test_workload_shapes():
    w = si.workload("c4a_ragged")
    assert w.A.shape == (1, 1000, 1000) and w.B.shape == (1, 1030, 1000)
    assert w.A.dtype == np.float16 and w.C is None
    w = si.workload("c2_1024")
    assert w.C.dtype == np.float32 and w.C.shape == (1, 1024, 1024)
    assert w.alpha == 1.5 and w.beta == 0.5
    wi = si.workload("c2_1024", int_values=True)
    assert set(np.unique(wi.A.astype(np.float64))) <= set(range(-3, 4))
    assert wi.flops == 2 * 1024 ** 3


def test_attention_workloads_are_seeded_and_shaped():
    import seeded_inputs as si
    w1 = si.attention_workload("attn_small")
    w2 = si.attention_workload("attn_small")
    assert w1.Q.shape == (2, 200, 64) and w1.K.shape == (2, 300, 64)
    assert w1.V.shape == (2, 300, 64) and w1.Q.dtype == np.float16
    for x, y in ((w1.Q, w2.Q), (w1.K, w2.K), (w1.V, w2.V)):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    # Q, K and V come from distinct streams
    assert not np.array_equal(w1.K, w1.V)
    assert abs(float(w1.V.astype(np.float64).std()) - 1.0) < 0.05
    assert w1.flops == 4 * 2 * 200 * 300 * 64
