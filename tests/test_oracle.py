"""Pins for the CPU oracle against facts that do not come from the oracle itself: the pages'
worked examples, closed forms, library routines on special cases, brute force on tiny
inputs and finite differences.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_top_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits_for_choice(choice, E, hi=1.0):
    lg = np.zeros((len(choice), E), np.float32)
    for t, e in enumerate(choice):
        lg[t, e] = hi
    return lg


# ----------------------------------------------------------------------------- routing

def _brute_topk(z, k):
    """Independent top-k: Python sort with the key (value descending, id ascending)."""
    out = []
    for row in z:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, np.int32)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    # coarse quantisation creates many ties; include signed zeros (they must tie)
    lg = (rng.integers(-3, 4, size=(200, 16)) * 0.5).astype(np.float32)
    lg[lg == 0] = np.where(rng.random((lg == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    for k in (1, 3, 16):
        idx, w, _ = oracle.route_topk(lg, None, k)
        np.testing.assert_array_equal(idx, _brute_topk(lg, k))


def test_topk_bias_enters_selection_and_weights():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    b = rng.standard_normal(12).astype(np.float32)
    idx, w, _ = oracle.route_topk(lg, b, 4)
    z = lg + b  # one fp32 add
    np.testing.assert_array_equal(idx, _brute_topk(z, 4))
    # weights = softmax over the chosen logits only (the full-E denominator cancels)
    zc = np.take_along_axis(z.astype(np.float64), idx, 1)
    ref = np.exp(zc - zc.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=2e-7, atol=0)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_topk_all_configs_vs_numpy(cfg):
    wl = W.WORKLOADS[cfg]
    T = W.generate(wl, weights=False)
    idx, w, probs = oracle.route_topk(T.logits, T.bias, wl.k, want_probs=True)
    z = T.logits if T.bias is None else T.logits + T.bias
    # numpy lexsort: primary key -z, secondary key expert id
    ids = np.broadcast_to(np.arange(wl.E), z.shape)
    order = np.lexsort((ids, -z), axis=1)[:, : wl.k]
    np.testing.assert_array_equal(idx, order)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=wl.k * 6e-8)
    # the full softmax against scipy's implementation
    from scipy.special import softmax
    np.testing.assert_allclose(probs, softmax(z.astype(np.float64), axis=1), rtol=1e-6, atol=1e-12)


def test_topk_k1_weight_is_exactly_one():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((30, 7)).astype(np.float32)
    _, w, _ = oracle.route_topk(lg, None, 1)
    assert np.all(w == 1.0)


def test_golden_ep_dispatch_top1():
    g = _golden("ep_dispatch_top1.json")
    lg = _logits_for_choice(g["choice"], g["E"])
    idx, w, _ = oracle.route_topk(lg, None, g["k"])
    np.testing.assert_array_equal(idx[:, 0], g["choice"])
    pl = oracle.permute(idx, w, g["E"])
    ex = g["expected"]
    np.testing.assert_array_equal(pl["counts"], ex["counts"])
    np.testing.assert_array_equal(pl["offsets"], ex["offsets"])
    np.testing.assert_array_equal(pl["row_token"], ex["row_token"])
    np.testing.assert_array_equal(pl["row_w"], ex["weights"])


def test_golden_ep_imbalance_top1():
    g = _golden("ep_imbalance_top1.json")
    lg = _logits_for_choice(g["choice"], g["E"])
    idx, w, _ = oracle.route_topk(lg, None, g["k"])
    pl = oracle.permute(idx, w, g["E"])
    np.testing.assert_array_equal(pl["counts"], g["expected"]["counts"])
    c = pl["counts"]
    assert [int(c[0] + c[1]), int(c[2] + c[3])] == g["expected"]["rows_per_gpu_of_two_experts"]


def test_golden_ep_combine_top2():
    g = _golden("ep_combine_top2.json")
    E = g["E"]
    lg = np.full((1, E), -30.0, np.float32)
    for e, wt in zip(g["experts"], g["weights"]):
        lg[0, e] = math.log(wt)
    idx, w, _ = oracle.route_topk(lg, None, g["k"])
    np.testing.assert_array_equal(idx[0], g["experts"])
    np.testing.assert_allclose(w[0], g["weights"], rtol=1e-6)
    # y(A2) = 0.7 u0 + 0.3 u2, with u_e the expert's output at weight 1
    rng = np.random.default_rng(3)
    H, I = 16, 8
    x = rng.standard_normal((1, H)).astype(np.float32)
    wg = (0.3 * rng.standard_normal((E, I, H))).astype(np.float32)
    wu = (0.3 * rng.standard_normal((E, I, H))).astype(np.float32)
    wd = (0.3 * rng.standard_normal((E, H, I))).astype(np.float32)
    u = [oracle.layer_fwd(x, wg, wu, wd, [0], [e], [1.0])[0] for e in g["experts"]]
    y = oracle.layer_fwd(x, wg, wu, wd, [0, 0], g["experts"], g["weights"])[0]
    ref = sum(float(np.float32(a)) * b for a, b in zip(g["weights"], u))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- plan

def _check_plan_invariants(idx, w, pl, E):
    N, k = idx.shape
    M = N * k
    counts, off = pl["counts"], pl["offsets"]
    assert counts.sum() == M and off[-1] == M and off[0] == 0
    assert np.all(np.diff(off) == counts)
    np.testing.assert_array_equal(np.bincount(idx.reshape(-1), minlength=E), counts)
    # (t, j) <-> row is a bijection, and each row holds its pair's token, expert and weight
    rp = pl["row_pair"]
    assert sorted(rp.tolist()) == list(range(M))
    np.testing.assert_array_equal(pl["row_token"], rp // k)
    np.testing.assert_array_equal(pl["row_w"], w.reshape(-1)[rp])
    row_e = np.repeat(np.arange(E), counts)
    np.testing.assert_array_equal(idx.reshape(-1)[rp], row_e)
    # stable: within an expert the tokens ascend
    for e in range(E):
        seg = pl["row_token"][off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # token-major lists: rows of token t, ascending
    np.testing.assert_array_equal(pl["tok_ptr"], np.arange(N + 1) * k)
    for t in range(N):
        rows = pl["tok_rows"][t * k:(t + 1) * k]
        assert np.all(np.diff(rows) > 0)
        assert np.all(pl["row_token"][rows] == t)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_plan_invariants(cfg):
    wl = W.WORKLOADS[cfg]
    T = W.generate(wl, weights=False)
    idx, w, _ = oracle.route_topk(T.logits, T.bias, wl.k)
    pl = oracle.permute(idx, w, wl.E)
    _check_plan_invariants(idx, w, pl, wl.E)


def test_permute_unpermute_identity():
    wl = W.WORKLOADS[1]
    T = W.generate(wl)
    idx, w, _ = oracle.route_topk(T.logits, T.bias, wl.k)
    pl = oracle.permute(idx, w, wl.E)
    gathered = T.x[pl["row_token"]]               # expert order
    inv = np.empty_like(pl["row_pair"])
    inv[pl["row_pair"]] = np.arange(len(inv))     # pair -> row
    back = gathered[inv].reshape(wl.N, wl.k, wl.H)
    for j in range(wl.k):
        assert np.array_equal(back[:, j].view(np.uint32), T.x.view(np.uint32))


# ----------------------------------------------------------------------------- forward

def _silu_mlp_torch(x, wg, wu, wd):
    """Dense SwiGLU MLP with library routines (torch matmul + F.silu) in fp64."""
    xt = torch.from_numpy(x.astype(np.float64))
    g = xt @ torch.from_numpy(wg.astype(np.float64)).T
    u = xt @ torch.from_numpy(wu.astype(np.float64)).T
    return (torch.nn.functional.silu(g) * u) @ torch.from_numpy(wd.astype(np.float64)).T


def _small(E=4, N=24, H=32, I=16, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H)).astype(np.float32)
    wg = (0.2 * rng.standard_normal((E, I, H))).astype(np.float32)
    wu = (0.2 * rng.standard_normal((E, I, H))).astype(np.float32)
    wd = (0.2 * rng.standard_normal((E, H, I))).astype(np.float32)
    dout = rng.standard_normal((N, H)).astype(np.float32)
    return x, wg, wu, wd, dout


def test_fwd_single_expert_is_dense_mlp():
    x, wg, wu, wd, _ = _small(E=1)
    N = x.shape[0]
    out = oracle.layer_fwd(x, wg, wu, wd, np.arange(N), np.zeros(N), np.ones(N))
    ref = _silu_mlp_torch(x, wg[0], wu[0], wd[0]).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_fwd_top1_weight1_is_per_token_expert_mlp():
    x, wg, wu, wd, _ = _small(E=5)
    N = x.shape[0]
    e = np.arange(N) % 5
    out = oracle.layer_fwd(x, wg, wu, wd, np.arange(N), e, np.ones(N))
    for t in range(N):
        ref = _silu_mlp_torch(x[t:t + 1], wg[e[t]], wu[e[t]], wd[e[t]]).numpy()[0]
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-13)


def test_fwd_equal_groups_is_batched_matmul():
    """idx[t,j] = (t + j*E/k) mod E gives every expert N*k/E rows; the grouped layer then
    equals a batched dense matmul over [E, N*k/E, .] (torch.bmm)."""
    E, k = 4, 2
    x, wg, wu, wd, _ = _small(E=E, N=16)
    N, H = x.shape
    idx = np.array([[(t + j * E // k) % E for j in range(k)] for t in range(N)], np.int32)
    rng = np.random.default_rng(9)
    w = rng.random((N, k)).astype(np.float32)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    out = oracle.layer_fwd(x, wg, wu, wd, pt, pe, pw)
    pl = oracle.permute(idx, w, E)
    assert np.all(pl["counts"] == N * k // E)
    xs = torch.from_numpy(x.astype(np.float64)[pl["row_token"]].reshape(E, N * k // E, H))
    g = torch.bmm(xs, torch.from_numpy(wg.astype(np.float64)).transpose(1, 2).contiguous())
    u = torch.bmm(xs, torch.from_numpy(wu.astype(np.float64)).transpose(1, 2).contiguous())
    y = torch.bmm(torch.nn.functional.silu(g) * u,
                  torch.from_numpy(wd.astype(np.float64)).transpose(1, 2).contiguous())
    y = y.reshape(N * k, H).numpy() * pl["row_w"].astype(np.float64)[:, None]
    ref = np.zeros((N, H))
    np.add.at(ref, pl["row_token"], y)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_fwd_linear_in_w_and_f32_agrees():
    x, wg, wu, wd, _ = _small(E=3)
    N = x.shape[0]
    pt = np.repeat(np.arange(N), 2)
    pe = np.tile([0, 2], N)
    pw = np.tile([0.25, 0.75], N).astype(np.float32)
    a = oracle.layer_fwd(x, wg, wu, wd, pt, pe, pw)
    b = oracle.layer_fwd(x, wg, wu, wd, pt, pe, 2 * pw)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-14, atol=1e-15)
    c = oracle.layer_fwd(x, wg, wu, wd, pt, pe, pw, real="f32")
    assert np.abs(c - a).max() / np.abs(a).max() < 1e-5


def test_fwd_token_without_pairs_is_zero():
    x, wg, wu, wd, _ = _small(E=2, N=6)
    out = oracle.layer_fwd(x, wg, wu, wd, [0, 2], [1, 0], [1.0, 1.0])
    assert np.all(out[[1, 3, 4, 5]] == 0)


# ----------------------------------------------------------------------------- backward

def _autograd_ref(x, wg, wu, wd, dout, pt, pe, pw):
    """fp64 torch autograd through the dense per-pair definition."""
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tg = torch.tensor(wg, dtype=torch.float64, requires_grad=True)
    tu = torch.tensor(wu, dtype=torch.float64, requires_grad=True)
    td = torch.tensor(wd, dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(pw, dtype=torch.float64, requires_grad=True)
    out = torch.zeros(x.shape, dtype=torch.float64)
    for p in range(len(pt)):
        t, e = int(pt[p]), int(pe[p])
        xt = tx[t]
        a = torch.nn.functional.silu(tg[e] @ xt) * (tu[e] @ xt)
        out = out.index_add(0, torch.tensor([t]), (tw[p] * (td[e] @ a))[None])
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return dict(dx=tx.grad.numpy(), dwg=tg.grad.numpy(), dwu=tu.grad.numpy(),
                dwd=td.grad.numpy(), ds=tw.grad.numpy())


def test_bwd_matches_autograd_config1_shape():
    wl = W.WORKLOADS[1]
    T = W.generate(wl)
    idx, w, _ = oracle.route_topk(T.logits, T.bias, wl.k)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    got = oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt, pe, pw)
    ref = _autograd_ref(T.x, T.wg, T.wu, T.wd, T.dout, pt, pe, pw)
    for n in ("dx", "dwg", "dwu", "dwd", "ds"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-10, atol=1e-13, err_msg=n)


def test_bwd_central_finite_differences():
    """Loss L = <dOut, out>.  Perturb single fp32 inputs by an exactly known step and compare
    the fp64 central difference with each gradient."""
    x, wg, wu, wd, dout = _small(E=3, N=10, H=12, I=8, seed=11)
    N = x.shape[0]
    pt = np.repeat(np.arange(N), 2).astype(np.int32)
    pe = np.array([(t + j) % 3 for t in range(N) for j in range(2)], np.int32)
    pw = np.random.default_rng(12).random(2 * N).astype(np.float32)
    g = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw)

    def loss(x_, wg_, wu_, wd_, pw_):
        return float((oracle.layer_fwd(x_, wg_, wu_, wd_, pt, pe, pw_) * dout.astype(np.float64)).sum())

    rng = np.random.default_rng(13)
    args = dict(x=x, wg=wg, wu=wu, wd=wd, pw=pw)
    gname = dict(x="dx", wg="dwg", wu="dwu", wd="dwd", pw="ds")
    for name in args:
        arr = args[name]
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            base = arr[pos]
            hp = np.float32(base + np.float32(1e-2 * max(1.0, abs(base))))
            hm = np.float32(base - np.float32(1e-2 * max(1.0, abs(base))))
            vals = []
            for v in (hp, hm):
                a2 = arr.copy()
                a2[pos] = v
                kw = dict(args)
                kw[name] = a2
                vals.append(loss(kw["x"], kw["wg"], kw["wu"], kw["wd"], kw["pw"]))
            fd = (vals[0] - vals[1]) / (float(hp) - float(hm))
            an = g[gname[name]][pos]
            assert abs(fd - an) <= 2e-4 * max(1.0, abs(an)), (name, pos, fd, an)


def test_ds_identity_fused_form():
    """<dOut_t, Y_r> equals <dA'_r, A_r> with dA'_r = W_down[e]^T dOut_t (the fused form of
    the router-score gradient) and equals the oracle's dS."""
    x, wg, wu, wd, dout = _small(E=3, N=8, seed=21)
    N = x.shape[0]
    pt = np.arange(N).astype(np.int32)
    pe = (np.arange(N) % 3).astype(np.int32)
    pw = np.full(N, 0.6, np.float32)
    ds = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw, want=("ds",))["ds"]
    for p in range(N):
        e, t = pe[p], pt[p]
        xt = x[t].astype(np.float64)
        g = wg[e].astype(np.float64) @ xt
        u = wu[e].astype(np.float64) @ xt
        a = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
        y = wd[e].astype(np.float64) @ a
        dap = wd[e].astype(np.float64).T @ dout[t].astype(np.float64)
        assert abs(dap @ a - dout[t].astype(np.float64) @ y) < 1e-12 * max(1, abs(ds[p]))
        assert abs(dap @ a - ds[p]) < 1e-11 * max(1, abs(ds[p]))


def test_bwd_linear_in_dout_and_empty_expert_zero():
    x, wg, wu, wd, dout = _small(E=4, seed=31)
    N = x.shape[0]
    pt = np.arange(N).astype(np.int32)
    pe = (np.arange(N) % 3).astype(np.int32)  # expert 3 is empty
    pw = np.ones(N, np.float32)
    a = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw)
    b = oracle.layer_bwd(2 * dout, x, wg, wu, wd, pt, pe, pw)  # exact fp32 scaling
    for n in a:
        np.testing.assert_allclose(b[n], 2 * a[n], rtol=1e-12, atol=1e-14)
    for n in ("dwg", "dwu", "dwd"):
        assert np.all(a[n][3] == 0)


# ----------------------------------------------------------------------------- token rounding

def _brute_tr(probs, idx, mtile):
    """Independent token rounding on tiny inputs: per expert, Python-sort all tokens by
    (routed first, score descending, token ascending) and keep the first r_e."""
    N, E = probs.shape
    k = idx.shape[1]
    routed = [set() for _ in range(E)]
    for t in range(N):
        for j in range(k):
            routed[idx[t, j]].add(t)
    sel = []
    for e in range(E):
        c = len(routed[e])
        r = mtile * ((c + mtile // 2) // mtile)
        r = min(r, mtile * (N // mtile))
        order = sorted(range(N), key=lambda t: (t not in routed[e], -float(probs[t, e]), t))
        sel.append(sorted(order[:r]))
    return sel


def test_token_round_brute_force():
    rng = np.random.default_rng(41)
    for trial in range(20):
        N, E, k, mt = int(rng.integers(5, 40)), int(rng.integers(2, 9)), 0, int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        lg = (rng.integers(-4, 5, size=(N, E)) * 0.25).astype(np.float32)  # ties in P
        idx, w, probs = oracle.route_topk(lg, None, k, want_probs=True)
        pl = oracle.token_round(probs, idx, mt)
        sel = _brute_tr(probs, idx, mt)
        off = pl["offsets"]
        c = np.bincount(idx.reshape(-1), minlength=E)
        for e in range(E):
            rows = pl["row_token"][off[e]:off[e + 1]]
            assert rows.tolist() == sel[e], (trial, e)
            r = off[e + 1] - off[e]
            assert r % mt == 0
            assert abs(r - c[e]) <= mt // 2 or r == mt * (N // mt)
            for q, t in zip(range(off[e], off[e + 1]), rows):
                js = np.nonzero(idx[t] == e)[0]
                assert pl["row_pair"][q] == (t * k + js[0] if len(js) else -1)
                st = sum(float(probs[t, idx[t, j]]) for j in range(k))
                ref = float(probs[t, e]) / st
                assert abs(float(pl["row_w"][q]) - ref) <= 6e-8 * abs(ref)  # one fp32 rounding
        # token-major lists are consistent
        for t in range(N):
            rows = pl["tok_rows"][pl["tok_ptr"][t]:pl["tok_ptr"][t + 1]]
            assert np.all(np.diff(rows) > 0) and np.all(pl["row_token"][rows] == t)


def test_token_round_identity_when_counts_are_multiples():
    """Each expert already holds exactly Mtile rows, so rounding changes nothing and the
    weights equal the top-k weights."""
    E, k, mt = 4, 2, 4
    N = E * mt // k
    choice = [(t % E, (t + 1) % E) for t in range(N)]
    lg = np.full((N, E), -2.0, np.float32)
    for t, (a, b) in enumerate(choice):
        lg[t, a] = 1.0
        lg[t, b] = 0.5
    idx, w, probs = oracle.route_topk(lg, None, k, want_probs=True)
    top = oracle.permute(idx, w, E)
    assert np.all(top["counts"] == mt)
    tr = oracle.token_round(probs, idx, mt)
    for n in ("counts", "offsets", "row_token", "row_pair", "tok_ptr", "tok_rows"):
        np.testing.assert_array_equal(tr[n], top[n], err_msg=n)
    np.testing.assert_allclose(tr["row_w"], top["row_w"], rtol=1e-6)


def test_token_round_config5_counts():
    wl = W.WORKLOADS[5]
    T = W.generate(wl, weights=False)
    idx, w, probs = oracle.route_topk(T.logits, T.bias, wl.k, want_probs=True)
    pl = oracle.token_round(probs, idx, wl.mtile)
    c = np.bincount(idx.reshape(-1), minlength=wl.E)
    r = pl["counts"]
    assert np.all(r % wl.mtile == 0)
    assert np.all(np.abs(r - c) <= wl.mtile // 2)
    assert pl["offsets"][-1] <= wl.N * wl.k + wl.E * wl.mtile // 2


# ----------------------------------------------------------------------------- router
# The router's forward weights, written in float64 numpy for finite differences: for a token
# with top-k set K and logits z, the final pair (t, e) weighs exp(z_e) / sum_{j in K} exp(z_j).
# The oracle's backward is pinned against central differences of this forward; the forward
# itself is pinned against the oracle's routing outputs (route_topk's weights, and the
# token-rounding plan's row weights).

def _pair_weights(z, K, pe):
    zmax = max(z[j] for j in K)
    sk = sum(math.exp(z[j] - zmax) for j in K)
    return np.array([math.exp(z[e] - zmax) / sk for e in pe])


def _loss(z_rows, idx, pt, pe, ds):
    """sum over final pairs of dS_f * w_f(z)"""
    tot = 0.0
    for t in range(z_rows.shape[0]):
        sel = np.nonzero(pt == t)[0]
        if len(sel) == 0:
            continue
        w = _pair_weights(z_rows[t], list(idx[t]), pe[sel])
        tot += float(np.dot(ds[sel].astype(np.float64), w))
    return tot


def _fd_dz(z, idx, pt, pe, ds, eps=1e-6):
    N, E = z.shape
    g = np.zeros((N, E))
    for t in range(N):
        for m in range(E):
            zp = z.astype(np.float64).copy()
            zm = zp.copy()
            zp[t, m] += eps
            zm[t, m] -= eps
            g[t, m] = (_loss(zp, idx, pt, pe, ds) - _loss(zm, idx, pt, pe, ds)) / (2 * eps)
    return g


def test_router_logits_matmul_and_one_hot():
    rng = np.random.default_rng(21)
    N, H, E = 9, 13, 7
    x = rng.standard_normal((N, H)).astype(np.float32)
    wr = rng.standard_normal((H, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    lg = oracle.router_logits(x, wr, b)
    ref = (x.astype(np.float64) @ wr.astype(np.float64) + b).astype(np.float32)
    np.testing.assert_array_equal(lg, ref)
    # one-hot rows select rows of W_r exactly
    xo = np.zeros((H, H), np.float32)
    xo[np.arange(H), np.arange(H)] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(xo, wr), wr)


def test_router_bwd_worked_example_top2():
    # weights 0.7 and 0.3 on experts 0 and 2 ('EP: Expert를 나누고 토큰 보내기', section '여러
    # Expert의 결과도 같은 토큰으로 돌아오기'); with dS = (1, 0) the closed form of the
    # renormalised softmax gives dz_0 = 0.7 (1 - 0.7) = 0.21 and dz_2 = 0.3 (0 - 0.7) = -0.21
    g = _golden("ep_combine_top2.json")
    E = g["E"]
    lg = np.full((1, E), -30.0, np.float32)
    for e, wt in zip(g["experts"], g["weights"]):
        lg[0, e] = math.log(wt)
    idx, w, _ = oracle.route_topk(lg, None, g["k"])
    pt, pe, _ = oracle.pairs_from_topk(idx, w)
    r = oracle.router_bwd(lg, None, idx, pt, pe, np.array([1.0, 0.0], np.float32))
    np.testing.assert_allclose(r["dz"][0], [0.21, 0.0, -0.21, 0.0], atol=1e-7)
    # dS = (0, 1): dz_0 = 0.7 (0 - 0.3), dz_2 = 0.3 (1 - 0.3)
    r = oracle.router_bwd(lg, None, idx, pt, pe, np.array([0.0, 1.0], np.float32))
    np.testing.assert_allclose(r["dz"][0], [-0.21, 0.0, 0.21, 0.0], atol=1e-7)
    # k = 1: the weight is identically one, so no gradient reaches z
    idx1, w1, _ = oracle.route_topk(lg, None, 1)
    pt1, pe1, _ = oracle.pairs_from_topk(idx1, w1)
    r = oracle.router_bwd(lg, None, idx1, pt1, pe1, np.array([5.0], np.float32))
    np.testing.assert_array_equal(r["dz"], 0.0)


def test_router_bwd_topk_finite_differences():
    rng = np.random.default_rng(22)
    N, E, k = 5, 6, 3
    lg = rng.standard_normal((N, E)).astype(np.float32)
    idx, w, _ = oracle.route_topk(lg, None, k)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    # the numpy forward reproduces the oracle's routing weights
    for t in range(N):
        np.testing.assert_allclose(_pair_weights(lg[t].astype(np.float64), list(idx[t]), idx[t]), w[t], rtol=2e-7)
    ds = rng.standard_normal(len(pt)).astype(np.float32)
    r = oracle.router_bwd(lg, None, idx, pt, pe, ds)
    np.testing.assert_allclose(r["dz"], _fd_dz(lg, idx, pt, pe, ds), rtol=1e-6, atol=1e-8)
    # shift invariance: the weights do not change when every z of a token moves together
    np.testing.assert_allclose(r["dz"].sum(axis=1), 0.0, atol=1e-12)
    # zero outside the chosen experts
    mask = np.zeros((N, E), bool)
    mask[np.repeat(np.arange(N), k), idx.reshape(-1)] = True
    assert np.all(r["dz"][~mask] == 0.0)


def test_router_bwd_token_rounding_finite_differences():
    # a token-rounding plan has padded pairs (outside K, weight P_e / S_t) and dropped pairs
    # (in K, no final pair): both enter only through the normaliser over K
    rng = np.random.default_rng(23)
    N, E, k, mtile = 12, 4, 2, 4
    lg = rng.standard_normal((N, E)).astype(np.float32)
    idx, w, probs = oracle.route_topk(lg, None, k, want_probs=True)
    pl = oracle.token_round(probs, idx, mtile)
    pt, pe, pw = oracle.pairs_from_plan(pl, E)
    assert np.any(pl["row_pair"] < 0), "the case needs a padded pair"
    routed = {(t, e) for t in range(N) for e in idx[t]}
    assert len(routed - set(zip(pt.tolist(), pe.tolist()))) > 0, "the case needs a dropped pair"
    # the plan's weights are this forward's values
    for f in range(len(pt)):
        wf = _pair_weights(lg[pt[f]].astype(np.float64), list(idx[pt[f]]), [pe[f]])[0]
        np.testing.assert_allclose(pw[f], wf, rtol=1e-6)
    ds = rng.standard_normal(len(pt)).astype(np.float32)
    r = oracle.router_bwd(lg, None, idx, pt, pe, ds)
    np.testing.assert_allclose(r["dz"], _fd_dz(lg, idx, pt, pe, ds), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(r["dz"].sum(axis=1), 0.0, atol=1e-12)


def test_router_bwd_parameter_gradients_finite_differences():
    # end to end: z = x W_r + b, L = sum_f dS_f w_f(z); differences in x, W_r and b
    rng = np.random.default_rng(24)
    N, H, E, k = 4, 5, 6, 2
    x = rng.standard_normal((N, H)).astype(np.float32)
    wr = rng.standard_normal((H, E)).astype(np.float32)
    b = (0.5 * rng.standard_normal(E)).astype(np.float32)
    lg = oracle.router_logits(x, wr)
    idx, w, _ = oracle.route_topk(lg, b, k)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    ds = rng.standard_normal(len(pt)).astype(np.float32)
    r = oracle.router_bwd(lg, b, idx, pt, pe, ds, x, wr)

    def loss(xx, ww, bb):
        z = xx @ ww + bb
        # the selection stays the one the gradient was taken at
        assert all(set(np.argsort(-z[t], kind="stable")[:k]) == set(idx[t]) for t in range(N))
        return _loss(z, idx, pt, pe, ds)

    X, Wr, B = x.astype(np.float64), wr.astype(np.float64), b.astype(np.float64)
    eps = 1e-6
    for (name, arr, shape) in (("dx", X, (N, H)), ("dwr", Wr, (H, E)), ("dbias", B, (E,))):
        g = np.zeros(shape)
        for ix in np.ndindex(*shape):
            ap, am = arr.copy(), arr.copy()
            ap[ix] += eps
            am[ix] -= eps
            args_p = [X, Wr, B]
            args_m = [X, Wr, B]
            pos = {"dx": 0, "dwr": 1, "dbias": 2}[name]
            args_p[pos], args_m[pos] = ap, am
            g[ix] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(r[name], g, rtol=2e-5, atol=1e-7)


# ----------------------------------------------------------------------------- capacity plan

def _brute_capacity(idx, w, E, C, policy, probs):
    """Independent: per expert, Python sort of its (t, j) pairs by the policy key, keep C."""
    N, k = idx.shape
    rows = []
    counts = []
    for e in range(E):
        pairs = [(t, j) for t in range(N) for j in range(k) if idx[t, j] == e]
        key = (lambda tj: tj[0]) if policy == 0 else (lambda tj: (-float(probs[tj[0], e]), tj[0]))
        kept = sorted(sorted(pairs, key=key)[:C])
        counts.append(len(kept))
        rows += [(t, j, float(w[t, j])) for t, j in kept]
    return np.array(counts), rows


def test_golden_ep_imbalance_capacity():
    g = _golden("ep_imbalance_capacity2.json")
    lg = _logits_for_choice(g["choice"], g["E"])
    idx, w, _ = oracle.route_topk(lg, None, g["k"])
    pl = oracle.capacity_plan(idx, w, g["E"], g["capacity"], 0)
    ex = g["expected"]
    np.testing.assert_array_equal(pl["counts"], ex["counts"])
    np.testing.assert_array_equal(pl["offsets"], ex["offsets"])
    np.testing.assert_array_equal(pl["row_token"], ex["row_token"])
    kept = set(pl["row_token"].tolist())
    assert sorted(set(range(len(g["choice"]))) - kept) == ex["dropped_tokens"]


@pytest.mark.parametrize("policy", [0, 1])
def test_capacity_brute_force(policy):
    rng = np.random.default_rng(31 + policy)
    for N, E, k, C in ((40, 6, 2, 9), (64, 8, 3, 20), (17, 5, 5, 3), (30, 4, 1, 0)):
        lg = rng.standard_normal((N, E)).astype(np.float32)
        if policy == 1:
            lg[: N // 3] = np.round(lg[: N // 3])  # ties in P: token order decides
        idx, w, probs = oracle.route_topk(lg, None, k, want_probs=True)
        pl = oracle.capacity_plan(idx, w, E, C, policy, probs)
        counts, rows = _brute_capacity(idx, w, E, C, policy, probs)
        np.testing.assert_array_equal(pl["counts"], counts)
        np.testing.assert_array_equal(pl["counts"], np.minimum(np.bincount(idx.reshape(-1), minlength=E), C))
        np.testing.assert_array_equal(pl["row_token"], [r[0] for r in rows])
        np.testing.assert_array_equal(pl["row_pair"], [r[0] * k + r[1] for r in rows])
        np.testing.assert_array_equal(pl["row_w"], np.array([r[2] for r in rows], np.float32))
        # token lists: the kept rows of each token, ascending
        for t in range(N):
            rs = pl["tok_rows"][pl["tok_ptr"][t]:pl["tok_ptr"][t + 1]]
            assert np.all(np.diff(rs) > 0) and np.all(pl["row_token"][rs] == t)
        assert pl["tok_ptr"][-1] == len(rows)


def test_capacity_without_drops_is_the_topk_plan():
    rng = np.random.default_rng(33)
    N, E, k = 50, 7, 3
    idx, w, probs = oracle.route_topk(rng.standard_normal((N, E)).astype(np.float32), None, k, want_probs=True)
    cmax = int(np.bincount(idx.reshape(-1), minlength=E).max())
    ref = oracle.permute(idx, w, E)
    for policy in (0, 1):
        pl = oracle.capacity_plan(idx, w, E, cmax, policy, probs)
        for n in ref:
            np.testing.assert_array_equal(pl[n], ref[n], err_msg=n)
