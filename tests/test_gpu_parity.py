"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

* routing indices, counts, offsets and every row list: bit-exact;
* route / row weights and probabilities (fp32): max|diff|/max|ref| <= 1e-5;
* out, dx, dW_gate, dW_up, dW_down, dS: max|diff|/max|ref| <= 1e-5 for fp32 workloads and
  <= 1e-2 for bf16 workloads;
* two runs are bitwise identical.
The five workloads run at full size; configurations 1 and 2 are compared in full, the
larger ones on a sample (rows are independent given the weights, so a sampled token's out,
dx and dS and a sampled expert's dW are exact comparisons)."""
import numpy as np
import pytest

from grouped_gemm_top_amd import workloads as W
from harness import bitwise_equal, check_layer, check_routing, log, run_gpu, sample, upload

pytestmark = pytest.mark.gpu

SAMPLES = {3: (256, 6), 4: (1024, 16), 5: (512, 8)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()  # fails loudly when the HIP library is missing


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_tiles(dtype):
    """Several tiles in every dimension with ragged tails (H=320: 2.5 N-tiles of 128; I=200:
    3.1 gate/up tiles of 64 and 1.6 of 128; ~128 rows per expert +- a tail)."""
    wl = W.custom("ragged", N=512, H=320, I=200, E=12, k=3, dtype=dtype, bias="normal", bias_std=0.3, seed=11)
    T = W.generate(wl)
    log(f"[ragged {dtype}] running")
    res = run_gpu(T)
    check_routing(T, res)
    errs, bad = check_layer(T, res)
    log(f"[ragged {dtype}] {errs}")
    assert not bad, bad


def _run_choice(choice, E, H=64, I=32, dtype="bf16", seed=3, k=None):
    """Routing forced through the logits: token t prefers the experts in choice[t] in order."""
    N = len(choice)
    k = k or len(choice[0])
    wl = W.custom("forced", N=N, H=H, I=I, E=E, k=k, dtype=dtype, seed=seed)
    T = W.generate(wl)
    lg = np.full((N, E), -4.0, np.float32)
    for t, es in enumerate(choice):
        for r, e in enumerate(es):
            lg[t, e] = 2.0 - 0.25 * r
    T.logits = lg
    res = run_gpu(T)
    check_routing(T, res)
    errs, bad = check_layer(T, res)
    return res, errs, bad


def test_edge_empty_experts_and_single_row_expert():
    E = 9
    choice = [(0, 1)] * 150 + [(2, 0)] + [(1, 0)] * 40   # expert 2 has one row, 3..8 none
    res, errs, bad = _run_choice(choice, E, H=128, I=64)
    c = res["plan"]["counts"]
    assert c[2] == 1 and np.all(c[3:] == 0)
    assert np.all(res["dwg"][3:] == 0) and np.all(res["dwd"][3:] == 0)
    assert not bad, (errs, bad)


def test_edge_one_expert_gets_every_token():
    choice = [(5,)] * 700  # 700 rows: six 128-row tiles, ragged last tile
    res, errs, bad = _run_choice(choice, 8, H=192, I=96)
    assert res["plan"]["counts"][5] == 700
    assert not bad, (errs, bad)


def test_edge_k_equals_E_and_N_1():
    res, errs, bad = _run_choice([(3, 1, 0, 2)], 4, H=64, I=32, dtype="f32")
    assert res["plan"]["counts"].tolist() == [1, 1, 1, 1]
    assert not bad, (errs, bad)


def test_edge_single_expert_dense():
    wl = W.custom("dense", N=300, H=256, I=128, E=1, k=1, dtype="bf16", seed=5)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    assert np.all(res["w"] == 1.0)
    errs, bad = check_layer(T, res)
    assert not bad, (errs, bad)


def test_edge_wide_hidden_2880():
    """H = I = 2880 (45 k-tiles of 64, 22.5 n-tiles of 128), the shape of configuration 3."""
    wl = W.custom("h2880", N=48, H=2880, I=2880, E=4, k=2, dtype="bf16", seed=6)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    errs, bad = check_layer(T, res)
    log(f"[h2880] {errs}")
    assert not bad, (errs, bad)


def test_edge_ties_and_many_experts():
    """E = 1024 (16 values per lane) with quantised logits full of ties, incl. signed zeros."""
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    rng = np.random.default_rng(8)
    lg = (rng.integers(-2, 3, size=(300, 1024)) * 0.5).astype(np.float32)
    lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    for k in (1, 7, 64):
        idx, w, probs = G.route_topk(torch.from_numpy(lg).cuda(), k, want_probs=True)
        oi, ow, op = oracle.route_topk(lg, None, k, want_probs=True)
        np.testing.assert_array_equal(idx.cpu().numpy(), oi)
        assert np.abs(w.cpu().numpy() - ow).max() <= 1e-5 * np.abs(ow).max()


def test_edge_empty_input():
    import torch
    import grouped_gemm_top_amd as G
    E, k, H, I = 4, 2, 64, 32
    x = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((0, E), dtype=torch.float32, device="cuda")
    wg = torch.randn((E, I, H), device="cuda").bfloat16()
    wu = torch.randn((E, I, H), device="cuda").bfloat16()
    wd = torch.randn((E, H, I), device="cuda").bfloat16()
    idx, w, _ = G.route_topk(lg, k)
    plan = G.permute(idx, w, E)
    hc, y = G.grouped_gemm_fwd(x, wg, wu, wd, plan)
    out = G.unpermute_combine(y, plan)
    g = G.layer_bwd(x, x, wg, wu, wd, plan, hc)
    torch.cuda.synchronize()
    assert plan.counts.cpu().tolist() == [0] * E and plan.offsets.cpu().tolist() == [0] * (E + 1)
    assert out.shape == (0, H)
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert torch.count_nonzero(g[n]).item() == 0


def test_token_rounding_small_mtile():
    """Token rounding with a small granule on a skewed router, compared in full."""
    wl = W.custom("tr-small", N=400, H=128, I=64, E=16, k=4, dtype="bf16", bias="normal", bias_std=0.8,
                  routing="tr", mtile=32, seed=9)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    c = res["plan"]["counts"]
    assert np.all(c % 32 == 0)
    errs, bad = check_layer(T, res)
    assert not bad, (errs, bad)


@pytest.mark.parametrize("policy", [0, 1])
def test_capacity_plan(policy):
    """Capacity plans with drops (C below the busiest experts' counts), compared in full."""
    wl = W.custom("cap-small", N=500, H=128, I=64, E=10, k=2, dtype="bf16",
                  routing="cap", mtile=90, cap_policy=policy, seed=12)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    c = res["plan"]["counts"]
    assert c.max() == 90 and int(c.sum()) < 500 * 2
    errs, bad = check_layer(T, res)
    log(f"[capacity policy {policy}] {errs}")
    assert not bad, (errs, bad)


def test_capacity_zero_drops_everything():
    """C = 0: no rows; out, dx and every dW are zero."""
    wl = W.custom("cap-zero", N=64, H=64, I=32, E=4, k=2, dtype="bf16", routing="cap", mtile=0, seed=16)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    assert int(res["plan"]["offsets"][-1]) == 0
    for n in ("out", "dx", "dwg", "dwu", "dwd"):
        assert not np.any(res[n]), n


@pytest.mark.parametrize("policy", [0, 1])
def test_capacity_headline_layer(policy):
    """The headline layer (E=128, H=2048, I=512, k=8, N=4096) with capacity factor 1
    (C = N k / E = 256), on a sample of tokens and experts."""
    import dataclasses
    wl = dataclasses.replace(W.CONFIGS[2], name="headline-cap", routing="cap", mtile=256, cap_policy=policy)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    toks, exps = sample(T, res, 256, 6)
    errs, bad = check_layer(T, res, toks, exps)
    log(f"[capacity headline policy {policy}] {errs}")
    assert not bad, (errs, bad)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config(cfg):
    wl = W.CONFIGS[cfg]
    log(f"[config {cfg}] {wl.name}: generating inputs")
    T = W.generate(wl)
    D = upload(T)
    log(f"[config {cfg}] running the HIP path")
    res = run_gpu(T, D)
    log(f"[config {cfg}] second run for determinism")
    res2 = run_gpu(T, D)
    assert bitwise_equal(res, res2) is None, bitwise_equal(res, res2)
    del res2, D
    log(f"[config {cfg}] routing parity")
    check_routing(T, res)
    counts = res["plan"]["counts"]
    log(f"[config {cfg}] rows {int(counts.sum())}, per-expert min {counts.min()} max {counts.max()} "
        f"empty {(counts == 0).sum()}")
    if cfg in SAMPLES:
        toks, exps = sample(T, res, *SAMPLES[cfg], seed=cfg)
    else:
        toks = exps = None
    log(f"[config {cfg}] oracle layer fwd/bwd")
    errs, bad = check_layer(T, res, toks, exps)
    log(f"[config {cfg}] max rel errors {errs}")
    assert not bad, bad
