"""The top-k router and both launch shapes of the permute against the oracle: the router's
indices bit for bit and weights to 1e-5 (ties included: the lowest expert id wins); the plan
bit for bit, on shapes that take the two-launch permute (histogram, then scan and scatter in
one kernel whose every block sums the whole histogram) and the three-launch one (histogram,
scan, scatter), with ragged token blocks, one expert, k = E, k > 64 and E = 1024."""
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


CASES = [
    # (N, E, k, ties, launches of the permute)
    (1, 1, 1, False, 2),
    (63, 8, 2, False, 2),
    (4097, 128, 8, True, 2),
    (200, 16, 16, False, 2),        # k = E
    (300, 32, 32, False, 2),
    (1000, 1024, 8, True, 2),
    (300, 128, 100, True, 2),       # k > 64: the router keeps its choices in LDS
    (16384, 256, 8, False, 2),
    (65536, 64, 4, False, 3),       # nb^2 E > 2^25
]


def _launches(N, E, k):
    nb = -(-N // 64)
    return 2 if nb * nb * E <= 1 << 25 else 3


@pytest.mark.parametrize("N,E,k,ties,launches", CASES)
def test_route_and_permute_against_oracle(N, E, k, ties, launches):
    import torch
    import grouped_gemm_top_amd as G
    import oracle
    from harness import log
    assert _launches(N, E, k) == launches
    log(f"[route_permute] N={N} E={E} k={k} ties={ties} permute launches={launches}")
    rng = np.random.default_rng(N * 7 + E)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    if ties:
        lg = np.round(lg * 2) / 2  # many equal logits: the expert-id tie break decides
    b = (0.5 * rng.standard_normal(E)).astype(np.float32)
    idx, w, _ = G.route_topk(torch.from_numpy(lg).cuda(), k, bias=torch.from_numpy(b).cuda())
    plan = G.permute(idx, w, E)
    torch.cuda.synchronize()
    oi, ow, _ = oracle.route_topk(lg, b, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-7)
    # the plan from the GPU's own selection and weights: exact
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    op = oracle.permute(gi, gw, E)
    h = plan.host()
    for name in ("counts", "offsets", "row_token", "row_pair", "tok_ptr", "tok_rows"):
        np.testing.assert_array_equal(h[name], np.asarray(op[name]), err_msg=name)
    np.testing.assert_array_equal(h["row_w"].view(np.int32), np.asarray(op["row_w"]).view(np.int32))
