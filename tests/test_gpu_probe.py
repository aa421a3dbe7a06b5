"""The measurement probes of libmoe_probe.so on the GPU: the copy probe copies exactly, the
read probe reads every word once (the XOR of its per-thread results equals the XOR of the
buffer), and the MFMA probe's results are linear in its iteration count and equal to the
closed form of its constant operands.  Two probes pin behaviour the fp8 kernels rely on: the
lane layout of the scaled fp8 matrix instruction and the rounding of the fp8 conversion."""
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


def test_reread_probe():
    """The re-read probe reads every kilobyte once per pass: one pass in register mode XORs to
    the buffer's XOR, two passes to zero; the LDS modes complete."""
    import torch
    from grouped_gemm_top_amd import probe
    g = torch.Generator().manual_seed(6)
    src = torch.randint(-2**31, 2**31 - 1, (37 * 256,), dtype=torch.int64, generator=g).to(torch.int32).cuda()
    sink = torch.zeros(8 * 256, dtype=torch.int32, device="cuda")
    assert probe.reread(src, 1, 0, 8, sink) == 37 * 1024
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
    probe.reread(src, 2, 0, 8, sink)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == 0
    for mode in (1, 2):
        probe.reread(src, 3, mode, 8, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


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


def _e4m3(code):
    """Value of an OCP e4m3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
    field 0 is subnormal; 0x7F / 0xFF are NaN)."""
    code = np.asarray(code, np.int64)
    e, m = (code >> 3) & 0xF, code & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))
    v = np.where((code & 0x7F) == 0x7F, np.nan, v)
    return np.where(code & 0x80, -v, v)


def test_fp8_scaled_mfma_lane_layout():
    """The scaled fp8 matrix instruction the fp8 grouped GEMMs use
    (v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 operands), checked on random exact-valued cases:
    lane L holds, for row L % 16 of its operand, k = 16 (L / 16) + j in byte j < 16 and
    k = 64 + 16 (L / 16) + (j - 16) in bytes 16..31; the block scale of (row L % 16, k block
    L / 16 of 32) is byte 0 of lane L's scale register (2^(byte - 127)); the result row
    4 (L / 16) + v (of the first operand) and column L % 16 (of the second) is float v of
    lane L (up to the fp32 rounding of the instruction's accumulation).  The kernels' LDS fragment reads and scale placement rely on exactly this."""
    import torch
    from grouped_gemm_top_amd import probe
    rng = np.random.default_rng(11)
    C = 16
    codes = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C, 0xB0, 0xB8, 0xBC, 0xC0, 0xC8], np.uint8)
    a = codes[rng.integers(0, len(codes), (C, 64, 32))]
    b = codes[rng.integers(0, len(codes), (C, 64, 32))]
    sa = rng.integers(122, 133, (C, 64)).astype(np.int64) | (rng.integers(0, 1 << 24, (C, 64)) << 8)
    sb = rng.integers(122, 133, (C, 64)).astype(np.int64) | (rng.integers(0, 1 << 24, (C, 64)) << 8)
    sa, sb = sa.astype(np.uint32).view(np.int32), sb.astype(np.uint32).view(np.int32)
    d = torch.zeros((C, 64, 4), dtype=torch.float32, device="cuda")
    probe.mfma_fp8_layout(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(sa).cuda(),
                          torch.from_numpy(sb).cuda(), d)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    L = np.arange(64)[:, None]
    j = np.arange(32)[None, :]
    k = np.where(j < 16, 16 * (L // 16) + j, 64 + 16 * (L // 16) + (j - 16))
    for c in range(C):
        A = np.zeros((16, 128))
        B = np.zeros((16, 128))
        A[np.broadcast_to(L % 16, k.shape), k] = _e4m3(a[c])
        B[np.broadcast_to(L % 16, k.shape), k] = _e4m3(b[c])
        SA = np.zeros((16, 4))
        SB = np.zeros((16, 4))
        SA[np.arange(64) % 16, np.arange(64) // 16] = 2.0 ** ((sa[c].view(np.uint32) & 0xFF).astype(np.float64) - 127)
        SB[np.arange(64) % 16, np.arange(64) // 16] = 2.0 ** ((sb[c].view(np.uint32) & 0xFF).astype(np.float64) - 127)
        As, Bs = A * np.repeat(SA, 32, axis=1), B * np.repeat(SB, 32, axis=1)
        D, Dabs = As @ Bs.T, np.abs(As) @ np.abs(Bs).T
        pick = lambda X: np.array([[X[4 * (l // 16) + v, l % 16] for v in range(4)] for l in range(64)])  # noqa: E731
        want, mag = pick(D), pick(Dabs)
        # the instruction accumulates 128 products in fp32 in its own order: within 2^-20 of the
        # sum of their magnitudes (a misplaced byte, block or scale moves results by O(mag))
        bad = np.abs(got[c] - want) > 2.0 ** -20 * mag
        assert not bad.any(), (c, np.argwhere(bad)[:5], got[c][bad][:5], want[bad][:5])


def test_fp8_conversion_matches_rne():
    """v_cvt_pk_fp8_f32, the conversion the fp8 kernels quantize with, rounds fp32 to e4m3 to
    nearest, ties to even, like torch's float8_e4m3fn cast: every code, every midpoint and
    its two neighbours, subnormals, signed zeros and random values in [-448, 448]."""
    import torch
    from grouped_gemm_top_amd import probe
    rng = np.random.default_rng(12)
    grid = _e4m3(np.arange(0, 0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    xs = np.concatenate([grid, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(1000)), rng.uniform(-448, 448, 30000),
                         rng.uniform(-0.02, 0.02, 30000), [0.0, 2.0 ** -10, 2.0 ** -11, 448.0]])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    src = torch.from_numpy(xs).cuda()
    dst = torch.zeros(len(xs), dtype=torch.uint8, device="cuda")
    probe.cvt_fp8(src, dst)
    torch.cuda.synchronize()
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(dst.cpu().numpy(), ref)
