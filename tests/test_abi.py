"""C-ABI contract of libmoe.so, checked on the host: the library loads, exports every entry
point that include/moe.h declares, and rejects bad arguments with the documented status
before anything is queued.  No test here launches a kernel (every call fails validation),
so the suite runs without a GPU."""
import ctypes
import os
import re

import pytest

import grouped_gemm_top_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 0x10000  # a non-NULL, 16-byte aligned address; never dereferenced by these calls


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    # MOE_ABI_TEST_LIB: another build of the same sources to run these checks on (the
    # host-AddressSanitizer build of tests/test_asan.py)
    other = os.environ.get("MOE_ABI_TEST_LIB")
    if other:
        return G.load_library(other)
    if not os.path.exists(G.lib_path()):
        import grouped_gemm_top_amd.build as B
        B.build()
    return G.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(G.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def test_plan_struct_layout():
    assert ctypes.sizeof(G.CPlan) == 6 * 4 + 7 * 8


def test_rows_cap(L):
    assert L.moe_plan_rows_cap(G.PLAN_TOPK, 4096, 128, 8, 0) == 4096 * 8
    assert L.moe_plan_rows_cap(G.PLAN_TR, 16384, 256, 8, 128) == 16384 * 8 + 256 * 64
    assert L.moe_plan_rows_cap(G.PLAN_TOPK, 10, 4, 5, 0) == -1      # k > E
    assert L.moe_plan_rows_cap(G.PLAN_TR, 10, 4, 2, 0) == -1         # mtile < 1
    assert L.moe_plan_rows_cap(7, 10, 4, 2, 0) == -1                 # unknown kind
    assert L.moe_plan_rows_cap(G.PLAN_TOPK, 0, 4, 2, 0) == 0         # empty input is valid


def test_workspace_bytes(L):
    for op in (G.OP_PERMUTE, G.OP_ROUTE_TR, G.OP_GEMM_FWD, G.OP_LAYER_BWD):
        assert L.moe_workspace_bytes(op, G.MOE_BF16, 4096, 128, 8, 2048, 512, 32768) > 0
        assert L.moe_workspace_bytes(op, G.MOE_BF16, 4096, 128, 0, 2048, 512, 32768) == 0  # k = 0
    assert L.moe_workspace_bytes(G.OP_GEMM_FWD, G.MOE_BF16, 64, 8, 2, 60, 32, 128) == 0     # H % 8
    assert L.moe_workspace_bytes(G.OP_LAYER_BWD, 9, 64, 8, 2, 64, 32, 128) == 0            # dtype
    # the router backward's workspace holds the operand planes (three bf16 parts of dlogits
    # and W_r, x^T with a row of ones, dlogits^T) and the sliced dW_r / dbias partial sums
    need = (3 * 4096 * 128 + 3 * 2048 * 128 + 2049 * 4096 + 3 * 128 * 4096) * 2 + 2049 * 128 * 4
    assert L.moe_workspace_bytes(G.OP_ROUTER_BWD, G.MOE_BF16, 4096, 128, 8, 2048, 0, 0) >= need
    # the logits' workspace holds W_r^T's three parts (and x's for fp32 x)
    assert L.moe_workspace_bytes(G.OP_ROUTER_LOGITS, G.MOE_BF16, 4096, 128, 1, 2048, 8, 0) >= 3 * 128 * 2048 * 2
    assert (L.moe_workspace_bytes(G.OP_ROUTER_LOGITS, G.MOE_F32, 4096, 128, 1, 2048, 8, 0)
            >= 3 * 128 * 2048 * 2 + 3 * 4096 * 2048 * 2)
    assert L.moe_workspace_bytes(G.OP_ROUTER_BWD, 9, 4096, 128, 8, 2048, 0, 0) == 0         # dtype
    # no tokens: still a valid query (the sizing must not divide by the empty tile count)
    for op in (G.OP_ROUTER_BWD, G.OP_ROUTER_LOGITS):
        for dt in (G.MOE_BF16, G.MOE_F32):
            assert L.moe_workspace_bytes(op, dt, 0, 128, 8, 2048, 8, 0) > 0
    # forward workspace holds the activation A [M_cap, I]
    assert L.moe_workspace_bytes(G.OP_GEMM_FWD, G.MOE_BF16, 4096, 128, 8, 2048, 512, 32768) >= 32768 * 512 * 2


def _plan(N=64, E=8, k=2, kind=G.PLAN_TOPK, mtile=0, M_cap=None):
    mc = M_cap if M_cap is not None else (N * k if kind == G.PLAN_TOPK else N * k + E * (mtile // 2))
    return G.CPlan(kind, N, E, k, mc, mtile, *([FAKE] * 7))


def _err(L):
    return L.moe_last_error().decode()


def test_route_topk_errors(L):
    f = ctypes.c_void_p(FAKE)
    assert L.moe_route_topk(f, None, 64, 8, 9, f, f, None, None) == G.MOE_EINVAL     # k > E
    assert "k must be" in _err(L)
    assert L.moe_route_topk(f, None, 64, 2000, 2, f, f, None, None) == G.MOE_EINVAL  # E > 1024
    assert L.moe_route_topk(f, None, -1, 8, 2, f, f, None, None) == G.MOE_EINVAL     # N < 0
    assert L.moe_route_topk(None, None, 64, 8, 2, f, f, None, None) == G.MOE_EINVAL  # NULL logits


def test_permute_errors(L):
    f = ctypes.c_void_p(FAKE)
    p = _plan()
    need = L.moe_workspace_bytes(G.OP_PERMUTE, G.MOE_BF16, 64, 8, 2, 8, 8, 0)
    assert L.moe_permute(f, f, 64, 8, 2, ctypes.byref(p), f, need - 1, None) == G.MOE_EWORKSPACE
    assert L.moe_permute(f, f, 64, 8, 2, None, f, need, None) == G.MOE_EINVAL
    small = _plan(M_cap=100)
    assert L.moe_permute(f, f, 64, 8, 2, ctypes.byref(small), f, need, None) == G.MOE_EINVAL
    other = _plan(N=32)
    assert L.moe_permute(f, f, 64, 8, 2, ctypes.byref(other), f, need, None) == G.MOE_EINVAL
    tr = _plan(kind=G.PLAN_TR, mtile=16)
    assert L.moe_permute(f, f, 64, 8, 2, ctypes.byref(tr), f, need, None) == G.MOE_EINVAL
    nullrows = _plan()
    nullrows.row_token = None
    assert L.moe_permute(f, f, 64, 8, 2, ctypes.byref(nullrows), f, need, None) == G.MOE_EINVAL
    assert L.moe_permute(None, f, 64, 8, 2, ctypes.byref(p), f, need, None) == G.MOE_EINVAL


def test_permute_noalloc_errors(L):
    """The no-allocation permute validates like moe_permute and refuses shapes whose histogram
    would not fit its fixed 4 MiB scratch, before anything is queued."""
    f = ctypes.c_void_p(FAKE)
    p = _plan()
    assert L.moe_permute_noalloc(f, f, 64, 8, 2, None, None) == G.MOE_EINVAL
    assert L.moe_permute_noalloc(None, f, 64, 8, 2, ctypes.byref(p), None) == G.MOE_EINVAL
    assert L.moe_permute_noalloc(f, f, 64, 8, 2, ctypes.byref(_plan(kind=G.PLAN_TR, mtile=16)), None) == G.MOE_EINVAL
    big = _plan(N=131072, E=256, k=8)
    assert L.moe_permute_noalloc(f, f, 131072, 256, 8, ctypes.byref(big), None) == G.MOE_EUNSUPPORTED
    assert "scratch" in _err(L)


def test_token_rounding_errors(L):
    f = ctypes.c_void_p(FAKE)
    p = _plan(kind=G.PLAN_TR, mtile=16)
    need = L.moe_workspace_bytes(G.OP_ROUTE_TR, G.MOE_BF16, 64, 8, 2, 8, 8, 0)
    args = lambda plan, mt, ws, probs=f: L.moe_route_token_rounding(f, None, 64, 8, 2, mt, f, f, probs,
                                                                    ctypes.byref(plan), f, ws, None)
    assert args(p, 16, need - 1) == G.MOE_EWORKSPACE
    assert args(p, 0, need) == G.MOE_EINVAL
    assert args(p, 32, need) == G.MOE_EINVAL           # mtile differs from the plan's
    assert args(_plan(), 16, need) == G.MOE_EINVAL     # top-k plan
    assert args(p, 16, need, probs=None) == G.MOE_EINVAL


def test_gemm_fwd_errors(L):
    f = ctypes.c_void_p(FAKE)
    p = _plan()
    need = L.moe_workspace_bytes(G.OP_GEMM_FWD, G.MOE_BF16, 64, 8, 2, 64, 32, p.M_cap)
    call = lambda dt, x, H, I, ws: L.moe_grouped_gemm_fwd(dt, x, f, f, f, H, I, ctypes.byref(p), f, f, f, ws, None)
    assert call(G.MOE_BF16, f, 60, 32, need) == G.MOE_EUNSUPPORTED      # H % 8
    assert call(G.MOE_BF16, f, 64, 36, need) == G.MOE_EUNSUPPORTED      # I % 8
    assert call(G.MOE_BF16, f, 0, 32, need) == G.MOE_EINVAL
    assert call(5, f, 64, 32, need) == G.MOE_EUNSUPPORTED               # dtype
    assert call(G.MOE_BF16, ctypes.c_void_p(FAKE + 2), 64, 32, need) == G.MOE_EUNSUPPORTED  # misaligned
    assert call(G.MOE_BF16, None, 64, 32, need) == G.MOE_EINVAL         # NULL x
    assert call(G.MOE_BF16, f, 64, 32, need - 1) == G.MOE_EWORKSPACE


def test_combine_errors(L):
    f = ctypes.c_void_p(FAKE)
    p = _plan()
    assert L.moe_unpermute_combine(G.MOE_BF16, f, 60, ctypes.byref(p), None, f, None) == G.MOE_EUNSUPPORTED
    assert L.moe_unpermute_combine(G.MOE_BF16, f, 64, ctypes.byref(p), None, None, None) == G.MOE_EINVAL
    assert L.moe_unpermute_combine(G.MOE_BF16, ctypes.c_void_p(FAKE + 8), 64, ctypes.byref(p), None, f,
                                   None) == G.MOE_EUNSUPPORTED
    assert L.moe_unpermute_combine(3, f, 64, ctypes.byref(p), None, f, None) == G.MOE_EUNSUPPORTED


def test_layer_bwd_errors(L):
    f = ctypes.c_void_p(FAKE)
    p = _plan()
    need = L.moe_workspace_bytes(G.OP_LAYER_BWD, G.MOE_BF16, 64, 8, 2, 64, 32, p.M_cap)

    def call(ws=need, dx=f, H=64, ds=f, plan=p):
        return L.moe_layer_bwd(G.MOE_BF16, f, f, f, f, f, H, 32, ctypes.byref(plan), f, dx, f, f, f, ds, f, ws,
                               None)
    assert call(ws=need - 1) == G.MOE_EWORKSPACE
    assert call(dx=None) == G.MOE_EINVAL
    assert call(ds=None) == G.MOE_EINVAL
    assert call(H=12) == G.MOE_EUNSUPPORTED
    assert call(plan=_plan(M_cap=3)) == G.MOE_EINVAL


def test_descriptor_size_limits(L):
    """Every tensor one kernel buffer descriptor covers must stay below 2 GiB (32-bit byte
    offsets); larger shapes are refused with MOE_EUNSUPPORTED before anything is queued, by
    both grouped-GEMM calls, and shapes just inside the limit pass this check (the calls then
    stop at the workspace check, since the fake workspace is too small)."""
    f = ctypes.c_void_p(FAKE)

    def calls(dt, N, H, I, E=8, k=2):
        p = _plan(N=N, E=E, k=k)
        fwd = L.moe_grouped_gemm_fwd(dt, f, f, f, f, H, I, ctypes.byref(p), f, f, f, 1, None)
        bwd = L.moe_layer_bwd(dt, f, f, f, f, f, H, I, ctypes.byref(p), f, f, f, f, f, f, f, 1, None)
        return fwd, bwd

    E2 = G.MOE_EUNSUPPORTED
    # x / dout [N, H]: 2^31 bytes exactly (N * H * 2)
    assert calls(G.MOE_BF16, 65536, 16384, 8) == (E2, E2)
    assert "x/dout" in _err(L)
    assert calls(G.MOE_BF16, 65535, 16384, 8) == (G.MOE_EWORKSPACE, G.MOE_EWORKSPACE)
    # the same N*H is over the limit in fp32 (4-byte elements)
    assert calls(G.MOE_F32, 32768, 16384, 8) == (E2, E2)
    # one expert's weight matrix [I, H]
    assert calls(G.MOE_BF16, 8, 32768, 32768) == (E2, E2)
    assert "weight matrix" in _err(L)
    # row activations [M_cap, 2I]: M_cap = N k = 2^20 rows, 2I = 1024 -> 2^31 bytes
    assert calls(G.MOE_BF16, 1 << 19, 8, 512) == (E2, E2)
    assert "row activations" in _err(L)
    assert calls(G.MOE_BF16, 1 << 19, 8, 504) == (G.MOE_EWORKSPACE, G.MOE_EWORKSPACE)
    # (the plan's row arrays, 4 M_cap bytes, stay below the limit whenever [M_cap, 2I] does)


def test_probe_library_exports_and_validation():
    """libmoe_probe.so (the measurement probes): exports what include/moe_probe.h declares and
    rejects bad arguments with status 1 before queueing anything."""
    from grouped_gemm_top_amd import probe
    if not os.path.exists(probe.lib_path()):
        import grouped_gemm_top_amd.build as B
        B.build()
    P = probe.lib()
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))
    assert set(names) == set(probe.PROBE_SYMBOLS)
    for n in names:
        assert hasattr(P, n), n
    f = ctypes.c_void_p(FAKE)
    assert P.moe_probe_mfma_bf16(2, 8, 10, f, None) == 1        # unknown shape
    assert P.moe_probe_mfma_bf16(0, 0, 10, f, None) == 1        # no blocks
    assert P.moe_probe_mfma_bf16(0, 8, 0, f, None) == 1         # no iterations
    assert P.moe_probe_mfma_bf16(0, 8, 10, None, None) == 1     # NULL sink
    assert P.moe_probe_copy(f, f, 24, 8, None) == 1             # not a multiple of 16
    assert P.moe_probe_copy(ctypes.c_void_p(FAKE + 4), f, 32, 8, None) == 1  # misaligned
    assert P.moe_probe_copy(f, None, 32, 8, None) == 1
    assert P.moe_probe_copy(f, f, 0, 8, None) == 0              # empty: nothing to queue
    assert P.moe_probe_read(f, 32, 8, None, None) == 1
    assert P.moe_probe_read(f, 32, 70000, f, None) == 1         # too many blocks


def test_mxfp8_dx_errors(L):
    """moe_quantize_dx_weights_mxfp8 and moe_layer_bwd_mxfp8 refuse bad arguments before
    anything is queued (H and I multiples of 32, weight codes given and aligned, workspace)."""
    f = ctypes.c_void_p(FAKE)
    qd = L.moe_quantize_dx_weights_mxfp8
    assert qd(G.MOE_BF16, f, f, 8, 64, 48, f, f, None) == G.MOE_EUNSUPPORTED   # I % 32
    assert qd(G.MOE_BF16, f, f, 8, 80, 32, f, f, None) == G.MOE_EUNSUPPORTED   # H % 32
    assert qd(G.MOE_BF16, f, f, 0, 64, 32, f, f, None) == G.MOE_EINVAL         # E
    assert qd(G.MOE_BF16, f, None, 8, 64, 32, f, f, None) == G.MOE_EINVAL      # NULL w_up
    assert qd(G.MOE_BF16, f, f, 8, 64, 32, ctypes.c_void_p(FAKE + 4), f, None) == G.MOE_EUNSUPPORTED
    assert qd(7, f, f, 8, 64, 32, f, f, None) == G.MOE_EUNSUPPORTED            # dtype
    p = _plan()
    need = L.moe_workspace_bytes(G.OP_LAYER_BWD_MXFP8, G.MOE_BF16, 64, 8, 2, 64, 32, p.M_cap)
    assert need > L.moe_workspace_bytes(G.OP_LAYER_BWD, G.MOE_BF16, 64, 8, 2, 64, 32, p.M_cap)
    assert L.moe_workspace_bytes(G.OP_LAYER_BWD_MXFP8, G.MOE_BF16, 64, 8, 2, 64, 40, p.M_cap) == 0

    def call(ws=need, H=64, I=32, wq=f, wsc=f):
        return L.moe_layer_bwd_mxfp8(f, f, f, f, f, wq, wsc, H, I, ctypes.byref(p), f, f, f, f, f, f, f, ws, None)
    assert call(ws=need - 1) == G.MOE_EWORKSPACE
    assert call(I=40) == G.MOE_EUNSUPPORTED
    assert call(H=72) == G.MOE_EUNSUPPORTED
    assert call(wq=None) == G.MOE_EINVAL
    assert call(wsc=ctypes.c_void_p(FAKE + 2)) == G.MOE_EUNSUPPORTED          # scale codes 4-byte aligned
