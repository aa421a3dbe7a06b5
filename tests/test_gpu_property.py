"""Property test: the whole path through the C ABI against the fp64 oracle on random small
layers (N, H, I, E, k, dtype, routing), every buffer guarded.  H and I are multiples of 8 (the
ABI's rule); the draws include k = E, experts left empty on purpose, E up to 1024, fp32 and
bf16 storage, and token rounding with small granules.  Examples are drawn deterministically,
and the run stops at the first failing example (no shrinking: each example is a GPU run)."""
import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, example, given, settings
from hypothesis import strategies as st

from grouped_gemm_top_amd import workloads as W
from harness import check_layer, check_routing, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()


@st.composite
def layers(draw):
    E = draw(st.sampled_from([1, 2, 3, 5, 8, 13, 32, 128, 257, 1024]))
    k = E if (E <= 16 and draw(st.booleans())) else draw(st.integers(1, min(E, 8)))
    big_e = E > 128
    H = 8 * draw(st.integers(1, 8 if big_e else 48))
    I = 8 * draw(st.integers(1, 8 if big_e else 48))
    N = draw(st.integers(1, 320))
    dtype = draw(st.sampled_from(["bf16", "f32"]))
    routing = draw(st.sampled_from(["topk", "topk", "tr"]))
    mtile = draw(st.sampled_from([1, 8, 16, 32, 128]))
    bias_std = draw(st.sampled_from([0.0, 0.5, 2.0]))
    n_empty = draw(st.integers(0, E - k))  # experts pushed out of every token's top-k
    seed = draw(st.integers(0, 1 << 16))
    return dict(N=N, H=H, I=I, E=E, k=k, dtype=dtype, routing=routing, mtile=mtile, bias_std=bias_std,
                n_empty=n_empty, seed=seed)


@settings(max_examples=40, deadline=None, derandomize=True, database=None, phases=[Phase.explicit, Phase.generate],
          suppress_health_check=list(HealthCheck), print_blob=True)
@given(layers())
@example(dict(N=3, H=16, I=8, E=4, k=4, dtype="bf16", routing="topk", mtile=8, bias_std=0.0, n_empty=0, seed=1))
@example(dict(N=40, H=64, I=24, E=1024, k=8, dtype="bf16", routing="topk", mtile=8, bias_std=0.0, n_empty=1000,
              seed=2))
@example(dict(N=17, H=8, I=8, E=5, k=2, dtype="f32", routing="tr", mtile=4, bias_std=2.0, n_empty=2, seed=3))
def test_random_layers(p):
    wl = W.custom("prop", N=p["N"], H=p["H"], I=p["I"], E=p["E"], k=p["k"], dtype=p["dtype"],
                  bias="normal" if p["bias_std"] > 0 else "none", bias_std=p["bias_std"], routing=p["routing"],
                  mtile=p["mtile"], seed=p["seed"])
    T = W.generate(wl)
    if p["n_empty"]:
        # the last n_empty experts lose every comparison (top-k never needs them, since
        # n_empty <= E - k), so they get no rows from top-k routing
        T.logits = T.logits.copy()
        T.logits[:, wl.E - p["n_empty"]:] -= np.float32(60.0)
    log(f"[property] {p}")
    res = run_gpu(T)
    check_routing(T, res)
    if p["routing"] == "topk" and p["n_empty"]:
        assert np.all(res["plan"]["counts"][wl.E - p["n_empty"]:] == 0)
    errs, bad = check_layer(T, res)
    assert not bad, (p, errs, bad)
