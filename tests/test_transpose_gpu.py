"""fp32 transpose on the GPU against the oracle: every output word must
equal the oracle's bit for bit."""
import numpy as np
import pytest

from oracle import transpose as T

pytestmark = pytest.mark.gpu


def _gpu():
    import dense_gemm_fp16_amd as g
    return g


def _say(msg):
    print(msg, flush=True)


def _x(shape, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("shape", [
    (1, 64, 64), (2, 256, 512), (1, 1024, 1024),   # 16-byte path
    (1, 1000, 1030), (3, 130, 68), (1, 63, 65),     # ragged: element path
    (1, 1, 4097), (1, 4097, 1), (5, 8, 12), (1, 4096, 2052),
])
def test_matches_oracle(shape):
    import torch
    g = _gpu()
    x = _x(shape, sum(shape))
    _say(f"[transpose] {shape}")
    y = g.transpose_f32(torch.from_numpy(x).cuda())
    ref = T.transpose(x)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_special_values_and_guard_bands():
    import torch
    g = _gpu()
    M, N = 96, 132
    bits = np.random.default_rng(1).integers(0, 2 ** 32, (M, N),
                                             dtype=np.uint64).astype(np.uint32)
    bits[0, :4] = [0x7FC00001, 0x80000000, 0x00000001, 0xFF800000]
    x = bits.view(np.float32)
    pad = 1024
    buf = torch.full((pad + M * N + pad,), 7.0, device="cuda")
    y = buf[pad:pad + M * N].view(N, M)
    g.transpose_f32(torch.from_numpy(x).cuda(), out=y)
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)
    assert np.array_equal(y.cpu().numpy().view(np.uint32),
                          T.transpose(x).view(np.uint32))


def test_misaligned_pointers_take_the_element_path():
    import torch
    g = _gpu()
    M, N = 200, 256
    x = _x((M, N), 3)
    xbuf = torch.zeros(M * N + 1, device="cuda")
    xbuf[1:] = torch.from_numpy(x.reshape(-1)).cuda()
    ybuf = torch.full((M * N + 1,), -1.0, device="cuda")
    st = g.transpose_f32_raw(1, M, N, xbuf[1:].data_ptr(),
                             ybuf[1:].data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == g.OK
    assert ybuf[0].item() == -1.0
    assert np.array_equal(ybuf[1:].cpu().numpy().reshape(N, M),
                          T.transpose(x))


def test_largest_supported_dimension():
    # N = 2^23, the largest supported: x is 2 x 2^23, y is 2^23 x 2
    import torch
    g = _gpu()
    x = _x((2, 2 ** 23), 77)
    _say("[transpose] 2 x 2^23")
    y = g.transpose_f32(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32),
                          T.transpose(x).view(np.uint32))


def test_random_shapes():
    """Seeded random shapes (half of them multiples of 4, the 16-byte
    path): bit-exact against the oracle."""
    import torch
    g = _gpu()
    r = np.random.default_rng(0x5EED008A)
    for case in range(30):
        batch = int(r.integers(1, 4))
        M, N = (int(v) for v in r.integers(1, 700, 2))
        if case % 2:
            M, N = -(-M // 4) * 4, -(-N // 4) * 4
        x = _x((batch, M, N), 7000 + case)
        _say(f"[transpose random {case}] {(batch, M, N)}")
        y = g.transpose_f32(torch.from_numpy(x).cuda())
        ref = T.transpose(x)
        assert np.array_equal(y.cpu().numpy().view(np.uint32),
                              ref.view(np.uint32)), case
