"""The measurement probes of libmoe_probe.so on the GPU: the copy probe copies exactly, the
read probe reads every word once (the XOR of its per-thread results equals the XOR of the
buffer), and the MFMA probe's results are linear in its iteration count and equal to the
closed form of its constant operands."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def test_copy_and_read_probes():
    import torch
    from grouped_gemm_top_amd import probe
    n = (3 << 20) + 4  # words: a ragged tail for the grid-stride loop (16-byte multiple)
    g = torch.Generator().manual_seed(5)
    src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int64, generator=g).to(torch.int32).cuda()
    dst = torch.zeros_like(src)
    probe.copy(src, dst, 37)
    sink = torch.zeros(64 * 256, dtype=torch.int32, device="cuda")
    probe.read(src, 64, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def _mfma_expected(shape, iters):
    # a[i] = (t + i) & 3, b[i] = (3 t + i) & 3 on every lane t (t = threadIdx.x), as bf16 x8.
    # Each MFMA adds the same product to every accumulator, so each thread's sum is iters times
    # the sum over its accumulator elements of one product; computed here from the MFMA's
    # documented lane layout.
    t = np.arange(256)
    A = np.stack([(t + i) & 3 for i in range(8)], 1).astype(np.float64)      # [lane, 8]
    B = np.stack([(3 * t + i) & 3 for i in range(8)], 1).astype(np.float64)
    out = np.zeros(256)
    for w in range(4):
        lanes = np.arange(64) + 64 * w
        a, b = A[lanes], B[lanes]
        if shape == 0:
            # 16x16x32: lane l holds A[m = l % 16][k = 8 (l // 16) + j], B[k = 8 (l // 16) + j][n = l % 16];
            # it receives C[m = 4 (l // 16) + v][n = l % 16], v < 4
            Am = np.zeros((16, 32)); Bm = np.zeros((32, 16))
            for l in range(64):
                Am[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a[l]
                Bm[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b[l]
            C = Am @ Bm
            for l in range(64):
                out[64 * w + l] = 8 * sum(C[4 * (l // 16) + v, l % 16] for v in range(4))
        else:
            # 32x32x16: lane l holds A[m = l % 32][k = 8 (l // 32) + j], B[k][n = l % 32]; it
            # receives C[m = 8 (v // 4) + 4 (l // 32) + v % 4][n = l % 32], v < 16
            Am = np.zeros((32, 16)); Bm = np.zeros((16, 32))
            for l in range(64):
                Am[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = a[l]
                Bm[8 * (l // 32):8 * (l // 32) + 8, l % 32] = b[l]
            C = Am @ Bm
            for l in range(64):
                out[64 * w + l] = 4 * sum(C[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32] for v in range(16))
    return out * iters


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_probe_values(shape):
    import torch
    from grouped_gemm_top_amd import probe
    blocks = 3
    s1 = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    s7 = torch.zeros_like(s1)
    probe.mfma_bf16(shape, blocks, 1, s1)
    probe.mfma_bf16(shape, blocks, 7, s7)
    torch.cuda.synchronize()
    a, b = s1.cpu().numpy().astype(np.float64), s7.cpu().numpy().astype(np.float64)
    assert np.array_equal(b, 7 * a)                 # linear in the iteration count
    want = _mfma_expected(shape, 1)
    assert np.array_equal(a, np.tile(want, blocks))  # the MFMA's closed form on these operands
