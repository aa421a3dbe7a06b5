"""moe_permute_noalloc, the permute on the library's fixed scratch, against moe_permute, the
same kernels on a caller workspace, through the C ABI: bit-identical plans on calls in a row
(the headline routing, then a smaller ragged one, then the headline again over the scratch
the smaller call left), and the size limit refused before anything is queued."""
import ctypes

import numpy as np
import pytest

from grouped_gemm_top_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()


def _compare(idx, w, E):
    import torch
    import grouped_gemm_top_amd as G
    N, k = idx.shape
    ref = G.permute(idx, w, E)
    got = G.Plan(N, E, k)
    for t in (got.counts, got.offsets, got.row_token, got.row_pair, got.tok_ptr, got.tok_rows):
        t.fill_(-5)  # a slot the call fails to write shows up
    got.row_w.fill_(float("nan"))
    G.permute_noalloc(idx, w, E, got)
    torch.cuda.synchronize()
    m = int(ref.offsets[-1].item())
    assert m == N * k
    for n in ("counts", "offsets", "tok_ptr"):
        np.testing.assert_array_equal(getattr(got, n).cpu().numpy(), getattr(ref, n).cpu().numpy(), err_msg=n)
    for n in ("row_token", "row_pair", "tok_rows"):
        np.testing.assert_array_equal(getattr(got, n)[:m].cpu().numpy(), getattr(ref, n)[:m].cpu().numpy(),
                                      err_msg=n)
    np.testing.assert_array_equal(got.row_w[:m].view(torch.int32).cpu().numpy(),
                                  ref.row_w[:m].view(torch.int32).cpu().numpy())
    return m


def _routing(wl):
    import torch
    import grouped_gemm_top_amd as G
    T = W.generate(wl, weights=False)
    idx, w, _ = G.route_topk(torch.from_numpy(T.logits).cuda(), wl.k,
                             bias=None if T.bias is None else torch.from_numpy(T.bias).cuda())
    return idx, w


def test_noalloc_matches_workspace_permute():
    big = W.WORKLOADS[2]                      # N = 4096, E = 128, k = 8
    small = W.custom("noalloc-small", N=300, H=8, I=8, E=12, k=4, bias="normal", bias_std=0.7, seed=31)
    bi, bw = _routing(big)
    si, sw = _routing(small)
    assert _compare(bi, bw, big.E) == 4096 * 8
    assert _compare(si, sw, small.E) == 300 * 4
    assert _compare(bi, bw, big.E) == 4096 * 8


def test_noalloc_rejects_oversize_before_queueing():
    import grouped_gemm_top_amd as G
    L = G.lib()
    f = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    for N, E, ok in ((131008, 256, True), (131072, 256, False), (32704, 1024, True), (32768, 1024, False)):
        need = G.workspace_bytes(G.OP_PERMUTE, G.MOE_BF16, N, E, 8)
        assert (need <= 4 << 20) == ok, (N, E, need)
        if not ok:
            p = G.CPlan(G.PLAN_TOPK, N, E, 8, N * 8, 0, *([0x10000] * 7))
            assert L.moe_permute_noalloc(f, f, N, E, 8, ctypes.byref(p), None) == G.MOE_EUNSUPPORTED
            assert "scratch" in L.moe_last_error().decode()
