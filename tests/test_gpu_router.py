"""GPU parity of the router's logits product and backward (through the C ABI) against the
fp64 CPU oracle.

* logits, dlogits, dW_r, dbias (fp32): max|diff|/max|ref| <= 1e-5;
* dx_out = dx_in + the router's share: <= 1e-5 (fp32 workloads) or <= 1e-2 (bf16, where dx
  is stored in bf16);
* two runs are bitwise identical.
The backward is compared given the same dS (the layer backward's output, whose own parity is
covered by test_gpu_parity.py) and the same plan (bit-exact against the oracle's)."""
import numpy as np
import pytest

import oracle
from grouped_gemm_top_amd import workloads as W
from harness import TOL, check_routing, log, rel_err, run_gpu, to_np, upload

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()  # fails loudly when the HIP library is missing


def _router_case(T, tag):
    """The layer on the GPU, then the router backward from its dS; both checked."""
    import torch
    import grouped_gemm_top_amd as G
    wl = T.wl
    D = upload(T)
    wr = torch.from_numpy(T.wr).to("cuda")
    bias = D["bias"]
    # forward product
    lg = G.router_logits(D["x"], wr, bias)
    lg2 = G.router_logits(D["x"], wr, bias)
    torch.cuda.synchronize()
    ref_lg = oracle.router_logits(T.x, T.wr, T.bias)
    e_lg = rel_err(lg.cpu().numpy(), ref_lg)
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), lg2.cpu().numpy().view(np.uint32)), "logits not reproducible"
    # the layer (routing from the workload's logits, as everywhere else)
    res = run_gpu(T, D)
    check_routing(T, res)
    if wl.routing == "tr":
        plan, idx, w, probs = G.route_token_rounding(D["logits"], wl.k, wl.mtile, bias=D["bias"])
        ds = torch.from_numpy(res["ds"]).to("cuda")
    elif wl.routing == "cap":
        plan, idx, w, probs = G.route_capacity(D["logits"], wl.k, wl.mtile, wl.cap_policy, bias=D["bias"])
        ds = torch.from_numpy(res["ds"]).to("cuda")
    else:
        idx, w, probs = G.route_topk(D["logits"], wl.k, bias=D["bias"], want_probs=True)
        plan = G.permute(idx, w, wl.E)
        ds = torch.from_numpy(res["ds"]).to("cuda")
    dx_in = torch.from_numpy(res["dx"]).to("cuda").to(D["x"].dtype)
    r1 = G.router_bwd(D["logits"], idx, plan, ds, D["x"], wr, bias=bias, dx_in=dx_in)
    r2 = G.router_bwd(D["logits"], idx, plan, ds, D["x"], wr, bias=bias, dx_in=dx_in)
    torch.cuda.synchronize()
    for n in ("dlogits", "dx", "dw_r", "dbias"):
        a, b = r1[n], r2[n]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), f"{n} not reproducible"
    # oracle, given the GPU's dS per final pair (pairs in row order)
    pl = res["plan"]
    pt, pe, _ = oracle.pairs_from_plan(pl, wl.E)
    if wl.routing in ("tr", "cap"):
        pds = res["ds"][:len(pt)]
    else:
        pds = res["ds"].reshape(-1)[pl["row_pair"]]
    ref = oracle.router_bwd(T.logits, T.bias, res["idx"], pt, pe, pds, T.x, T.wr)
    errs = dict(logits=e_lg,
                dlogits=rel_err(r1["dlogits"].cpu().numpy(), ref["dz"]),
                dw_r=rel_err(r1["dw_r"].cpu().numpy(), ref["dwr"]),
                dbias=rel_err(r1["dbias"].cpu().numpy(), ref["dbias"]),
                dx=rel_err(to_np(r1["dx"]), res["dx"].astype(np.float64) + ref["dx"]))
    log(f"[router {tag}] {errs}")
    tol = dict(logits=F32_TOL, dlogits=F32_TOL, dw_r=F32_TOL, dbias=F32_TOL, dx=TOL[wl.dtype])
    bad = {n: v for n, v in errs.items() if not v <= tol[n]}
    assert not bad, bad
    return res, r1, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_ragged(dtype):
    wl = W.custom("ragged", N=512, H=320, I=200, E=12, k=3, dtype=dtype, bias="normal", bias_std=0.3, seed=11)
    _router_case(W.generate(wl), f"ragged {dtype}")


def test_router_token_rounding():
    # padded rows (outside the top-k set) and dropped pairs (inside it, without a row)
    wl = W.custom("tr", N=600, H=64, I=32, E=10, k=2, dtype="bf16", routing="tr", mtile=32, seed=13)
    T = W.generate(wl)
    res, r1, ref = _router_case(T, "token rounding")
    assert np.any(res["plan"]["row_pair"] < 0), "the case needs padded rows"


def test_router_k1_has_no_gradient():
    # with k = 1 the combine weight is identically 1: dlogits, dW_r, dbias vanish, dx is dx_in
    wl = W.custom("k1", N=256, H=64, I=32, E=8, k=1, dtype="f32", seed=14)
    res, r1, ref = _router_case(W.generate(wl), "k=1")
    assert float(r1["dlogits"].abs().max()) == 0.0
    assert float(r1["dw_r"].abs().max()) == 0.0 and float(r1["dbias"].abs().max()) == 0.0


def test_router_empty_input():
    import torch
    import grouped_gemm_top_amd as G
    H, E, k = 64, 8, 2
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    wr = torch.randn((H, E), device="cuda")
    lg = G.router_logits(x, wr)
    idx, w, _ = G.route_topk(lg, k)
    plan = G.permute(idx, w, E)
    ds = torch.empty((0, k), dtype=torch.float32, device="cuda")
    dw = torch.full((H, E), 7.0, device="cuda")
    db = torch.full((E,), 7.0, device="cuda")
    r = G.router_bwd(lg, idx, plan, ds, x, wr, dw_r=dw, dbias=db)
    torch.cuda.synchronize()
    assert lg.shape == (0, E)
    assert float(r["dw_r"].abs().max()) == 0.0 and float(r["dbias"].abs().max()) == 0.0


@pytest.mark.parametrize("cfg", [2])
def test_router_config(cfg):
    # the full-size layer the benchmark times (E=128, H=2048, I=512, k=8, N=4096), in full
    _router_case(W.generate(W.WORKLOADS[cfg]), f"config {cfg}")


def test_router_capacity_plan():
    # dropped pairs (inside the top-k set, without a row) enter only through the normaliser
    wl = W.custom("cap", N=600, H=64, I=32, E=10, k=2, dtype="bf16", routing="cap", mtile=96, cap_policy=1,
                  seed=15)
    res, r1, ref = _router_case(W.generate(wl), "capacity")
    assert int(res["plan"]["offsets"][-1]) < 600 * 2, "the case needs dropped pairs"
