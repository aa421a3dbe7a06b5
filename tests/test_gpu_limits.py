"""Layers whose tensors reach the 2 GiB a buffer descriptor may cover (the largest the C ABI
accepts), so the kernels' 32-bit byte offsets run up to just below 2^31:

* gathers: x and dOut [N, H] of 2^31 - 8192 bytes (N = 262143, H = 4096: one more token is
  refused), with the last tokens routed to a small expert, so the gathered rows sit at the
  highest offsets in every GEMM that gathers them (gate/up, dH, dW_d, dW_g/u);
* rows: hcache and dH [M_cap, 2I] of 2.143e9 bytes (N = 16384, k = E = 8, I = 4088), the last
  expert's rows at the top.

The oracle is run on samples (rows are independent given the weights): a sampled token's out,
dx and dS and the small expert's dW are exact comparisons, routed end to end by the oracle
from the sampled logits.  Inputs are drawn on the GPU (bf16), and only the sampled rows are
copied to the host."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()


def _run(N, H, I, E, k, lg, seed):
    import torch
    import grouped_gemm_top_amd as G
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((N, H), generator=g, device="cuda").bfloat16()
    dout = torch.randn((N, H), generator=g, device="cuda").bfloat16()
    wg = (0.02 * torch.randn((E, I, H), generator=g, device="cuda")).bfloat16()
    wu = (0.02 * torch.randn((E, I, H), generator=g, device="cuda")).bfloat16()
    wd = (0.02 * torch.randn((E, H, I), generator=g, device="cuda")).bfloat16()
    idx, w, _ = G.route_topk(lg, k)
    plan = G.permute(idx, w, E)
    hc, y = G.grouped_gemm_fwd(x, wg, wu, wd, plan)
    out = G.unpermute_combine(y, plan)
    r = G.layer_bwd(dout, x, wg, wu, wd, plan, hc)
    torch.cuda.synchronize()
    return dict(x=x, dout=dout, wg=wg, wu=wu, wd=wd, idx=idx, w=w, plan=plan, out=out, **r)


def _check(res, lg_host, toks, k, E, small=None):
    """Oracle on the sampled tokens; `small`: an expert all of whose tokens are in toks."""
    import oracle
    from harness import TOL, log, rel_err
    h = lambda t: t.float().cpu().numpy()  # noqa: E731
    sel = np.asarray(toks, np.int64)
    oi, ow, _ = oracle.route_topk(lg_host[sel], None, k)
    np.testing.assert_array_equal(res["idx"][sel].cpu().numpy(), oi)
    xs, ds_ = h(res["x"][sel]), h(res["dout"][sel])
    wg, wu, wd = h(res["wg"]), h(res["wu"]), h(res["wd"])
    pt = np.repeat(np.arange(len(sel), dtype=np.int32), k)
    pe, pw = oi.reshape(-1), ow.reshape(-1)
    want = ("dx", "ds") + (("dwg", "dwu", "dwd") if small is not None else ())
    ref_out = oracle.layer_fwd(xs, wg, wu, wd, pt, pe, pw)
    ref = oracle.layer_bwd(ds_, xs, wg, wu, wd, pt, pe, pw, want=want)
    errs = dict(out=rel_err(h(res["out"][sel]), ref_out), dx=rel_err(h(res["dx"][sel]), ref["dx"]),
                ds=rel_err(res["ds"][sel].cpu().numpy().reshape(-1), ref["ds"]))
    if small is not None:
        for n, m in (("dwg", "dw_gate"), ("dwu", "dw_up"), ("dwd", "dw_down")):
            errs[n] = rel_err(h(res[m][small]), ref[n][small])
    log(f"[limits] {errs}")
    tol = TOL["bf16"]
    assert all(v <= tol for v in errs.values()), errs


def test_gathers_near_2gib():
    import torch
    N, H, I, E, k = 262143, 4096, 64, 2, 1
    assert N * H * 2 <= 0x7FFFFFFF < (N + 1) * H * 2  # the largest N the C ABI accepts here
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    lg[:, 1] -= 30.0  # expert 1 takes only the chosen tokens: the last 16 and 32 others
    small = np.concatenate([rng.choice(N - 16, 32, replace=False), np.arange(N - 16, N)])
    lg[small, 1] += 60.0
    res = _run(N, H, I, E, k, torch.from_numpy(lg).cuda(), seed=21)
    counts = res["plan"].counts.cpu().numpy()
    assert counts[1] == len(small), counts
    toks = np.unique(np.concatenate([small, rng.choice(N, 48, replace=False)]))
    _check(res, lg, toks, k, E, small=1)


def test_rows_near_2gib():
    import torch
    N, H, I, E, k = 16384, 64, 4088, 8, 8
    assert N * k * 2 * I * 2 <= 0x7FFFFFFF
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    res = _run(N, H, I, E, k, torch.from_numpy(lg).cuda(), seed=22)
    # k = E: every token has a row in every expert, the last expert's rows at the top
    toks = np.unique(np.concatenate([np.arange(N - 24, N), rng.choice(N, 40, replace=False)]))
    _check(res, lg, toks, k, E)
