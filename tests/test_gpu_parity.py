"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

* routing indices, counts, offsets and every row list: bit-exact;
* route / row weights and probabilities (fp32): max|diff|/max|ref| <= 1e-5;
* out, dx, dW_gate, dW_up, dW_down, dS: max|diff|/max|ref| <= 1e-5 for fp32 workloads and
  <= 1e-2 for bf16 workloads;
* two runs are bitwise identical.
The five workloads run at full size; configurations 1 and 2 are compared in full, the
larger ones on a sample (rows are independent given the weights, so a sampled token's out,
dx and dS and a sampled expert's dW are exact comparisons): 1024 tokens, every token of the
two lightest non-empty experts among them, and dW of 16 experts (the heaviest, the lightest
non-empty, up to two empty ones, the rest random).  Top-k workloads are compared end to end
against the oracle's own routing plan and weights from the logits; token-rounding and
capacity plans against the oracle run on the GPU plan, which is first checked bit-exact given
the GPU's probabilities.  Every buffer of a run carries guard bands that are checked after
each call."""
import numpy as np
import pytest

from grouped_gemm_top_amd import workloads as W
from harness import Guards, bitwise_equal, check_layer, check_routing, log, rel_err, run_gpu, sample, upload

pytestmark = pytest.mark.gpu

SAMPLES = {3: (1024, 16), 4: (1024, 16), 5: (1024, 16)}


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


@pytest.mark.parametrize("dtype,H", [("f32", 2048), ("bf16", 4096)])
def test_wide_rows_combine(dtype, H):
    """Rows of 512 16-byte vectors (fp32 H = 2048, bf16 H = 4096): the combines' two-vector
    kernel instance, forward and dX, with ragged row counts; compared in full."""
    wl = W.custom(f"wide-{dtype}", N=96, H=H, I=64, E=6, k=2, dtype=dtype, bias="normal", bias_std=0.5, seed=31)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    errs, bad = check_layer(T, res)
    log(f"[wide rows {dtype} H={H}] {errs}")
    assert not bad, bad


def test_ragged_k_tails_bf16():
    """bf16 with H and I not multiples of 64 (H = 200, I = 72): the K tails of every kernel
    (the last k-step of gate/up and dH over H, of down over I, of dX over 2I) and ragged N
    tails, with several experts and ragged row counts; compared in full."""
    wl = W.custom("ktails", N=300, H=200, I=72, E=6, k=2, dtype="bf16", bias="normal", bias_std=0.4, seed=21)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    errs, bad = check_layer(T, res)
    log(f"[k tails] {errs}")
    assert not bad, bad


def _plan_model(idx, w, E):
    """CPU model of the top-k plan moe_permute documents for any topk_idx: pair (t, j) makes a
    row only if its id is in [0, E) and no earlier slot of the token names it; rows by expert,
    then token; token t's rows ascending in tok_rows[t k ..], then -1."""
    N, k = idx.shape
    valid = np.zeros((N, k), bool)
    for t in range(N):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < E and e not in seen:
                valid[t, j] = True
                seen.add(e)
    rows = [(int(idx[t, j]), t, j) for t in range(N) for j in range(k) if valid[t, j]]
    rows.sort()
    counts = np.bincount([r[0] for r in rows], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tok_rows = np.full(N * k, -1, np.int32)
    fill = np.zeros(N, np.int64)
    for r, (e, t, j) in enumerate(rows):
        tok_rows[t * k + fill[t]] = r
        fill[t] += 1
    return dict(counts=counts, offsets=offsets, row_token=np.array([t for _, t, _ in rows], np.int32),
                row_w=np.array([w[t, j] for _, t, j in rows], np.float32),
                row_pair=np.array([t * k + j for _, t, j in rows], np.int32),
                tok_ptr=(np.arange(N + 1) * k).astype(np.int32), tok_rows=tok_rows)


def test_permute_skips_invalid_pairs():
    """topk_idx with repeated and out-of-range expert ids (which the router never produces):
    the plan matches the documented skipping rule exactly, and the layer run on it matches the
    oracle on the pairs that made rows.  Guard bands around every buffer stay intact."""
    import torch
    import grouped_gemm_top_amd as G
    wl = W.custom("invalid-idx", N=300, H=128, I=64, E=12, k=4, dtype="bf16", seed=23)
    T = W.generate(wl)
    N, E, k, H, I = wl.N, wl.E, wl.k, wl.H, wl.I
    rng = np.random.default_rng(5)
    idx = rng.integers(-2, E + 2, size=(N, k)).astype(np.int32)
    idx[::7, 1] = idx[::7, 0]                      # repeats inside a token
    idx[::11] = rng.integers(0, E, size=(len(idx[::11]), 1))  # a token with one expert in every slot
    idx[5] = np.arange(k)                          # a token with k valid distinct experts
    idx[6] = -1                                    # a token with no valid slot
    w = rng.random((N, k)).astype(np.float32)
    ref = _plan_model(idx, w, E)
    assert 0 < ref["offsets"][-1] < N * k
    g = Guards()
    D = upload(T, g)
    didx = g.upload("topk_idx", idx)
    dw = g.upload("topk_w", w)
    plan = G.Plan(N, E, k, alloc=lambda name, n, dt: g.alloc("plan." + name, (n,), dt))
    ws = g.alloc("ws_permute", (G.workspace_bytes(G.OP_PERMUTE, G.MOE_BF16, N, E, k),), torch.uint8)
    # fill the plan's rows with a pattern, so rows past M that the call must not write are seen
    for t in (plan.row_token, plan.row_pair, plan.tok_rows):
        t.fill_(-7)
    G.permute(didx, dw, E, plan=plan, ws=ws)
    g.check("permute")
    m = int(ref["offsets"][-1])
    for n in ("counts", "offsets", "tok_ptr"):
        np.testing.assert_array_equal(getattr(plan, n).cpu().numpy(), ref[n], err_msg=n)
    for n in ("row_token", "row_w", "row_pair"):
        got = getattr(plan, n).cpu().numpy()
        np.testing.assert_array_equal(got[:m], ref[n], err_msg=n)
    assert np.all(plan.row_token.cpu().numpy()[m:] == -7)
    np.testing.assert_array_equal(plan.tok_rows.cpu().numpy(), ref["tok_rows"])
    hc = g.alloc("hcache", (N * k, 2 * I), torch.bfloat16)
    y = g.alloc("y", (N * k, H), torch.bfloat16)
    wsf = g.alloc("ws_fwd", (G.workspace_bytes(G.OP_GEMM_FWD, G.MOE_BF16, N, E, k, H, I, N * k),), torch.uint8)
    G.grouped_gemm_fwd(D["x"], D["wg"], D["wu"], D["wd"], plan, hcache=hc, y=y, ws=wsf)
    out = g.alloc("out", (N, H), torch.bfloat16)
    G.unpermute_combine(y, plan, out=out)
    g.check("forward")
    ds = g.alloc("ds", (N, k), torch.float32)
    ds.fill_(123.0)
    wsb = g.alloc("ws_bwd", (G.workspace_bytes(G.OP_LAYER_BWD, G.MOE_BF16, N, E, k, H, I, N * k),), torch.uint8)
    bw = dict(dx=g.alloc("dx", (N, H), torch.bfloat16), dw_gate=g.alloc("dwg", (E, I, H), torch.bfloat16),
              dw_up=g.alloc("dwu", (E, I, H), torch.bfloat16), dw_down=g.alloc("dwd", (E, H, I), torch.bfloat16))
    G.layer_bwd(D["dout"], D["x"], D["wg"], D["wu"], D["wd"], plan, hc, ds=ds, ws=wsb, **bw)
    g.check("layer_bwd")
    import oracle
    pt, pe, pw = oracle.pairs_from_plan(ref, E)
    o = oracle.layer_fwd(T.x, T.wg, T.wu, T.wd, pt, pe, pw)
    gr = oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt, pe, pw)
    dsg = ds.cpu().numpy().reshape(-1)
    errs = {"out": rel_err(out.float().cpu().numpy(), o), "dx": rel_err(bw["dx"].float().cpu().numpy(), gr["dx"]),
            "dwg": rel_err(bw["dw_gate"].float().cpu().numpy(), gr["dwg"]),
            "dwu": rel_err(bw["dw_up"].float().cpu().numpy(), gr["dwu"]),
            "dwd": rel_err(bw["dw_down"].float().cpu().numpy(), gr["dwd"]),
            "ds": rel_err(dsg[ref["row_pair"]], gr["ds"])}
    log(f"[invalid idx] rows {m} of {N * k}: {errs}")
    assert all(v <= 1e-2 for v in errs.values()), errs
    # ds of a skipped pair is left unwritten
    skipped = np.setdiff1d(np.arange(N * k), ref["row_pair"])
    assert np.all(dsg[skipped] == 123.0)


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
    wl = dataclasses.replace(W.WORKLOADS[2], name="headline-cap", routing="cap", mtile=256, cap_policy=policy)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    toks, exps = sample(T, res, 256, 6)
    errs, bad = check_layer(T, res, toks, exps)
    log(f"[capacity headline policy {policy}] {errs}")
    assert not bad, (errs, bad)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config(cfg):
    wl = W.WORKLOADS[cfg]
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



@pytest.mark.parametrize("H,I,E", [(512, 256, 16), (640, 200, 16), (1024, 256, 32)])
def test_heavy_skew_full(H, I, E):
    """Zipf-skewed groups (s = 1.5, k = 2): two experts hold nearly every row, several get a
    handful, the rest none, so the weight-gradient kernels run tiles of 100+ k-steps beside
    single-step and empty ones.  Compared in full, every expert's dW included (the Zipf
    workload itself is compared on a sample); H = 640, I = 200 puts tile edges inside the
    matrices.  Two runs bitwise identical."""
    wl = W.custom(f"skew-{H}-{I}-{E}", N=4096, H=H, I=I, E=E, k=2, dtype="bf16", bias="zipf", zipf_s=1.5, seed=41)
    T = W.generate(wl)
    res = run_gpu(T)
    check_routing(T, res)
    log(f"[skew H={H} I={I} E={E}] counts top {np.sort(res['plan']['counts'])[::-1][:4]}")
    errs, bad = check_layer(T, res)
    log(f"[skew H={H} I={I} E={E}] {errs}")
    assert not bad, bad
    res2 = run_gpu(T)
    assert bitwise_equal(res, res2) is None
