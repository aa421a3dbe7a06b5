"""The token-rounding and capacity plans' select against the oracle, on the shapes that take
its less common paths: scores full of ties (every key of an expert in the first pass's
threshold bin, so the radix passes read the keys from memory), quantised scores (ties inside
the threshold bin), more than 1024 token blocks of 64 (the token-major lists then use the
separate scan), and small or ragged token counts (fewer tokens than one tile, a partial token
block, one expert, E = 1024).  Given the GPU's own probabilities and indices the plan is bit-exact; the row
weights within 1e-5."""
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


def _check(plan, probs, idx, ref):
    gp = plan.host()
    for n in ("counts", "offsets", "row_token", "row_pair", "tok_ptr", "tok_rows"):
        np.testing.assert_array_equal(gp[n], ref[n], err_msg=n)
    scale = max(float(np.abs(ref["row_w"]).max()), 1e-30) if len(ref["row_w"]) else 1.0
    assert np.abs(gp["row_w"] - ref["row_w"]).max(initial=0.0) <= 1e-5 * scale


CASES = [
    # (name, N, E, k, mtile, logits)
    ("constant", 10000, 8, 2, 128, "zero"),       # P equal everywhere: one bin holds every key
    ("quantised", 9000, 64, 4, 96, "quant"),      # few distinct scores: ties at the threshold
    ("many-blocks", 70000, 8, 2, 64, "normal"),   # 1094 token blocks: the separate scan
]


@pytest.mark.parametrize("name,N,E,k,mtile,kind", CASES)
def test_token_rounding_select_paths(name, N, E, k, mtile, kind):
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    from harness import log
    log(f"[token rounding] {name}: N={N} E={E} k={k} mtile={mtile}")
    rng = np.random.default_rng(N + E)
    if kind == "zero":
        lg = np.zeros((N, E), np.float32)
    elif kind == "quant":
        lg = (rng.integers(-3, 4, size=(N, E)) * 0.25).astype(np.float32)
    else:
        lg = rng.standard_normal((N, E)).astype(np.float32)
    plan, idx, w, probs = G.route_token_rounding(torch.from_numpy(lg).cuda(), k, mtile)
    torch.cuda.synchronize()
    pr, ix = probs.cpu().numpy(), idx.cpu().numpy()
    ref = oracle.token_round(pr, ix, mtile)
    _check(plan, pr, ix, ref)
    c = plan.counts.cpu().numpy()
    assert np.all(c % mtile == 0)


@pytest.mark.parametrize("policy", [0, 1])
def test_capacity_select_ties(policy):
    """Capacity plans on constant scores: every routed token ties, the token order decides."""
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    N, E, k, C = 6000, 8, 2, 1000
    lg = np.zeros((N, E), np.float32)
    plan, idx, w, probs = G.route_capacity(torch.from_numpy(lg).cuda(), k, C, policy)
    torch.cuda.synchronize()
    ref = oracle.capacity_plan(idx.cpu().numpy(), w.cpu().numpy(), E, C, policy, probs.cpu().numpy())
    _check(plan, probs.cpu().numpy(), idx.cpu().numpy(), ref)


SMALL = [
    # (N, E, k, mtile): token counts below, at and just past the 64-token block and the
    # 16-token wavefront runs of the select, one expert, k = E, and E = 1024
    (1, 8, 2, 16),
    (2, 4, 4, 16),
    (15, 16, 1, 16),
    (63, 8, 2, 32),
    (64, 8, 3, 16),
    (65, 32, 4, 16),
    (127, 1, 1, 16),
    (300, 256, 8, 64),
    (777, 1024, 2, 16),
]


@pytest.mark.parametrize("N,E,k,mtile", SMALL)
def test_token_rounding_small_shapes(N, E, k, mtile):
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    from harness import log
    log(f"[token rounding] small: N={N} E={E} k={k} mtile={mtile}")
    rng = np.random.default_rng(1000 * N + E)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    plan, idx, w, probs = G.route_token_rounding(torch.from_numpy(lg).cuda(), k, mtile)
    torch.cuda.synchronize()
    pr, ix = probs.cpu().numpy(), idx.cpu().numpy()
    _check(plan, pr, ix, oracle.token_round(pr, ix, mtile))


@pytest.mark.parametrize("N,E,k,mtile", SMALL)
@pytest.mark.parametrize("policy", [0, 1])
def test_capacity_small_shapes(N, E, k, mtile, policy):
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    from harness import log
    C = max(1, (N * k) // (2 * E))  # about half of an even share: most experts drop
    log(f"[capacity] small: N={N} E={E} k={k} C={C} policy={policy}")
    rng = np.random.default_rng(1000 * N + E + 7)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    plan, idx, w, probs = G.route_capacity(torch.from_numpy(lg).cuda(), k, C, policy)
    torch.cuda.synchronize()
    ref = oracle.capacity_plan(idx.cpu().numpy(), w.cpu().numpy(), E, C, policy, probs.cpu().numpy())
    _check(plan, probs.cpu().numpy(), idx.cpu().numpy(), ref)
