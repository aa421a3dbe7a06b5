"""Shared helpers for the GPU parity tests: upload a workload, run the HIP path through the
C ABI, run the oracle (in full or on a sample), compare.  Imported by tests only."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from grouped_gemm_top_amd import workloads as W

TOL = {"f32": 1e-5, "bf16": 1e-2}
W_TOL = 1e-5  # route weights and row weights are fp32 in every workload


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    if den == 0:
        return float(num)
    return float(num / den)


def upload(T: W.Tensors):
    import torch
    dev = "cuda"
    out = {}
    if T.wl.dtype == "bf16":
        for n in ("x", "wg", "wu", "wd", "dout"):
            out[n] = torch.from_numpy(T.bits[n].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        for n in ("x", "wg", "wu", "wd", "dout"):
            out[n] = torch.from_numpy(getattr(T, n)).to(dev)
    out["logits"] = torch.from_numpy(T.logits).to(dev)
    out["bias"] = None if T.bias is None else torch.from_numpy(T.bias).to(dev)
    return out


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def run_gpu(T: W.Tensors, D=None):
    """The whole hot path through the C ABI; returns host copies of every output."""
    import torch
    import grouped_gemm_top_amd as G
    wl = T.wl
    D = D or upload(T)
    if wl.routing == "tr":
        plan, idx, w, probs = G.route_token_rounding(D["logits"], wl.k, wl.mtile, bias=D["bias"])
    elif wl.routing == "cap":
        plan, idx, w, probs = G.route_capacity(D["logits"], wl.k, wl.mtile, wl.cap_policy, bias=D["bias"])
    else:
        idx, w, probs = G.route_topk(D["logits"], wl.k, bias=D["bias"], want_probs=True)
        plan = G.permute(idx, w, wl.E)
    hcache, y = G.grouped_gemm_fwd(D["x"], D["wg"], D["wu"], D["wd"], plan)
    out = G.unpermute_combine(y, plan)
    g = G.layer_bwd(D["dout"], D["x"], D["wg"], D["wu"], D["wd"], plan, hcache)
    torch.cuda.synchronize()
    res = dict(idx=idx.cpu().numpy(), w=w.cpu().numpy(), probs=probs.cpu().numpy(), plan=plan.host(),
               out=to_np(out), dx=to_np(g["dx"]), dwg=to_np(g["dw_gate"]), dwu=to_np(g["dw_up"]),
               dwd=to_np(g["dw_down"]), ds=g["ds"].cpu().numpy())
    m = int(res["plan"]["offsets"][-1])
    res["hcache"] = to_np(hcache[:m]) if m > 0 else np.zeros((0, 2 * wl.I))
    res["y"] = to_np(y[:m]) if m > 0 else np.zeros((0, wl.H))
    return res


def bitwise_equal(a: dict, b: dict):
    for n in ("idx", "w", "probs", "out", "dx", "dwg", "dwu", "dwd", "ds", "hcache", "y"):
        if not np.array_equal(np.asarray(a[n]).view(np.uint8), np.asarray(b[n]).view(np.uint8)):
            return n
    for n in a["plan"]:
        if not np.array_equal(a["plan"][n], b["plan"][n]):
            return "plan." + n
    return None


def check_routing(T: W.Tensors, res: dict):
    """Bit-exact indices and plan, fp32 weights within W_TOL."""
    wl = T.wl
    idx, w, probs = oracle.route_topk(T.logits, T.bias, wl.k, want_probs=True)
    np.testing.assert_array_equal(res["idx"], idx)
    assert rel_err(res["w"], w) <= W_TOL, rel_err(res["w"], w)
    assert rel_err(res["probs"], probs) <= W_TOL, rel_err(res["probs"], probs)
    gp = res["plan"]
    if wl.routing == "tr":
        # bit-exact given the GPU's own probabilities and indices
        op = oracle.token_round(res["probs"], res["idx"], wl.mtile)
    elif wl.routing == "cap":
        # bit-exact given the GPU's own indices, weights (copied bitwise) and probabilities
        op = oracle.capacity_plan(res["idx"], res["w"], wl.E, wl.mtile, wl.cap_policy, res["probs"])
    else:
        op = oracle.permute(idx, w, wl.E)
        # row weights are bitwise copies of the GPU's route weights
        np.testing.assert_array_equal(gp["row_w"], res["w"].reshape(-1)[gp["row_pair"]])
    for n in ("counts", "offsets", "row_token", "row_pair", "tok_ptr", "tok_rows"):
        np.testing.assert_array_equal(gp[n], op[n], err_msg=n)
    assert rel_err(gp["row_w"], op["row_w"]) <= W_TOL
    return op


def sample(T: W.Tensors, res: dict, n_tok: int, n_exp: int, seed: int = 0):
    """Tokens: every token of the two lightest non-empty experts plus random ones.
    Experts: heaviest, lightest non-empty, up to two empty, then random."""
    wl = T.wl
    rng = np.random.default_rng(seed)
    pl = res["plan"]
    counts = pl["counts"]
    nz = np.nonzero(counts)[0]
    light = nz[np.argsort(counts[nz], kind="stable")][:2]
    toks = set()
    for e in light:
        toks.update(pl["row_token"][pl["offsets"][e]:pl["offsets"][e + 1]].tolist())
    rest = rng.permutation(wl.N)
    for t in rest:
        if len(toks) >= n_tok:
            break
        toks.add(int(t))
    toks = np.array(sorted(toks), np.int64)
    exps = []
    if len(nz):
        exps += [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    exps += [int(e) for e in np.nonzero(counts == 0)[0][:2]]
    for e in rng.permutation(wl.E):
        if len(exps) >= n_exp:
            break
        if int(e) not in exps:
            exps.append(int(e))
    return toks, np.array(sorted(set(exps)), np.int64)


def check_layer(T: W.Tensors, res: dict, toks=None, exps=None):
    """Forward/backward against the fp64 oracle on the pairs of the GPU plan (verified
    bit-exact beforehand).  toks/exps select a sample (None = everything)."""
    wl = T.wl
    tol = TOL[wl.dtype]
    pt, pe, pw = oracle.pairs_from_plan(res["plan"], wl.E)
    rows = np.arange(len(pt))
    if toks is not None:
        keep = np.isin(pt, toks)
        tr, tt, te, tw = rows[keep], pt[keep], pe[keep], pw[keep]
    else:
        toks = np.arange(wl.N)
        tr, tt, te, tw = rows, pt, pe, pw
    errs = {}
    out = oracle.layer_fwd(T.x, T.wg, T.wu, T.wd, tt, te, tw)
    errs["out"] = rel_err(res["out"][toks], out[toks])
    g = oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, tt, te, tw, want=("dx", "ds"))
    errs["dx"] = rel_err(res["dx"][toks], g["dx"][toks])
    if wl.routing in ("tr", "cap"):
        gds = res["ds"][tr]
    else:
        gds = res["ds"].reshape(-1)[res["plan"]["row_pair"][tr]]
    errs["ds"] = rel_err(gds, g["ds"])
    if exps is None:
        exps = np.arange(wl.E)
        ke = np.ones(len(pt), bool)
    else:
        ke = np.isin(pe, exps)
    gw = oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt[ke], pe[ke], pw[ke], want=("dwg", "dwu", "dwd"))
    for n in ("dwg", "dwu", "dwd"):
        errs[n] = rel_err(res[n][exps], gw[n][exps])
    bad = {n: v for n, v in errs.items() if not v <= tol}
    return errs, bad
