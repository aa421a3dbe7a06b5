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


GUARD_BYTES = 512   # guard band before and after every buffer the path reads or writes
GUARD_BYTE = 0xA5


class Guards:
    """Buffers with guard bands: each tensor sits inside a larger byte buffer whose first and
    last GUARD_BYTES bytes hold a fixed pattern; check() fails if a call wrote into any band.
    The views stay 16-byte aligned (the bands are multiples of 256 bytes)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.bufs = []

    def alloc(self, name, shape, dtype):
        import torch
        shape = tuple(shape) if isinstance(shape, (tuple, list)) else (int(shape),)
        n = int(np.prod(shape)) if shape else 1
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        full = torch.full((2 * GUARD_BYTES + nbytes,), GUARD_BYTE, dtype=torch.uint8, device=self.device)
        view = full[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)
        self.bufs.append((name, full, nbytes))
        return view

    def upload(self, name, arr, dtype=None):
        """A guarded device copy of host array `arr` (bf16 bit patterns given as uint16)."""
        import torch
        if arr.dtype == np.uint16:
            t = self.alloc(name, arr.shape, torch.bfloat16)
            t.view(torch.int16).copy_(torch.from_numpy(arr.view(np.int16)))
        else:
            t = self.alloc(name, arr.shape, dtype or getattr(torch, str(arr.dtype)))
            t.copy_(torch.from_numpy(np.ascontiguousarray(arr)))
        return t

    def check(self, after: str):
        import torch
        torch.cuda.synchronize()
        for name, full, nbytes in self.bufs:
            lo = full[:GUARD_BYTES]
            hi = full[GUARD_BYTES + nbytes:]
            if not (bool((lo == GUARD_BYTE).all()) and bool((hi == GUARD_BYTE).all())):
                raise AssertionError(f"guard band of {name} overwritten after {after}")


def upload(T: W.Tensors, guards: Guards | None = None):
    guards = guards or Guards()
    out = {}
    if T.wl.dtype == "bf16":
        for n in ("x", "wg", "wu", "wd", "dout"):
            out[n] = guards.upload(n, T.bits[n])
    else:
        for n in ("x", "wg", "wu", "wd", "dout"):
            out[n] = guards.upload(n, getattr(T, n))
    out["logits"] = guards.upload("logits", T.logits)
    out["bias"] = None if T.bias is None else guards.upload("bias", T.bias)
    out["guards"] = guards
    return out


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def run_gpu(T: W.Tensors, D=None):
    """The whole hot path through the C ABI, every buffer (inputs, outputs, plan arrays and
    workspaces) guarded and the guard bands checked after each call; returns host copies of
    every output."""
    import torch
    import grouped_gemm_top_amd as G
    wl = T.wl
    D = D or upload(T)
    g = D["guards"]
    N, H, I, E, k = wl.N, wl.H, wl.I, wl.E, wl.k
    dt = G.MOE_BF16 if wl.dtype == "bf16" else G.MOE_F32
    edt = D["x"].dtype
    f32, i32 = torch.float32, torch.int32
    idx = g.alloc("topk_idx", (N, k), i32)
    w = g.alloc("topk_w", (N, k), f32)
    probs = g.alloc("probs", (N, E), f32)
    ws_bytes = lambda op, mc=0: G.workspace_bytes(op, dt, N, E, k, H, I, mc)  # noqa: E731
    alloc = lambda name, n, dtype: g.alloc("plan." + name, (n,), dtype)  # noqa: E731
    if wl.routing in ("tr", "cap"):
        kind = G.PLAN_TR if wl.routing == "tr" else G.PLAN_CAP
        plan = G.Plan(N, E, k, kind=kind, mtile=wl.mtile, alloc=alloc)
        ws = g.alloc("ws_route", (ws_bytes(G.OP_ROUTE_TR),), torch.uint8)
        if wl.routing == "tr":
            G.route_token_rounding(D["logits"], k, wl.mtile, bias=D["bias"], plan=plan, ws=ws, idx=idx, w=w,
                                   probs=probs)
        else:
            G.route_capacity(D["logits"], k, wl.mtile, wl.cap_policy, bias=D["bias"], plan=plan, ws=ws, idx=idx,
                             w=w, probs=probs)
        g.check("routing")
    else:
        G.route_topk(D["logits"], k, bias=D["bias"], idx=idx, w=w, probs=probs)
        g.check("route_topk")
        plan = G.Plan(N, E, k, alloc=alloc)
        ws = g.alloc("ws_permute", (ws_bytes(G.OP_PERMUTE),), torch.uint8)
        G.permute(idx, w, E, plan=plan, ws=ws)
        g.check("permute")
    mc = max(plan.M_cap, 1)
    hcache = g.alloc("hcache", (mc, 2 * I), edt)
    y = g.alloc("y", (mc, H), edt)
    ws = g.alloc("ws_fwd", (ws_bytes(G.OP_GEMM_FWD, plan.M_cap),), torch.uint8)
    G.grouped_gemm_fwd(D["x"], D["wg"], D["wu"], D["wd"], plan, hcache=hcache, y=y, ws=ws)
    g.check("grouped_gemm_fwd")
    out = g.alloc("out", (N, H), edt)
    G.unpermute_combine(y, plan, out=out)
    g.check("unpermute_combine")
    dx = g.alloc("dx", (N, H), edt)
    dwg = g.alloc("dw_gate", (E, I, H), edt)
    dwu = g.alloc("dw_up", (E, I, H), edt)
    dwd = g.alloc("dw_down", (E, H, I), edt)
    ds = g.alloc("ds", (N, k) if plan.kind == G.PLAN_TOPK else (mc,), f32)
    ws = g.alloc("ws_bwd", (ws_bytes(G.OP_LAYER_BWD, plan.M_cap),), torch.uint8)
    G.layer_bwd(D["dout"], D["x"], D["wg"], D["wu"], D["wd"], plan, hcache, dx=dx, dw_gate=dwg, dw_up=dwu,
                dw_down=dwd, ds=ds, ws=ws)
    g.check("layer_bwd")
    res = dict(idx=idx.cpu().numpy(), w=w.cpu().numpy(), probs=probs.cpu().numpy(), plan=plan.host(),
               out=to_np(out), dx=to_np(dx), dwg=to_np(dwg), dwu=to_np(dwu), dwd=to_np(dwd), ds=ds.cpu().numpy())
    m = int(res["plan"]["offsets"][-1])
    res["hcache"] = to_np(hcache[:m]) if m > 0 else np.zeros((0, 2 * wl.I))
    res["y"] = to_np(y[:m]) if m > 0 else np.zeros((0, wl.H))
    # release the guarded outputs of this run (the inputs stay for a second run)
    g.bufs = [b for b in g.bufs if b[0] in ("x", "wg", "wu", "wd", "dout", "logits", "bias")]
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


def oracle_plan(T: W.Tensors):
    """The oracle's own top-k plan from the logits (route_topk then permute); nothing in it
    comes from the GPU."""
    wl = T.wl
    idx, w, _ = oracle.route_topk(T.logits, T.bias, wl.k)
    return oracle.permute(idx, w, wl.E)


def check_layer(T: W.Tensors, res: dict, toks=None, exps=None, plan=None):
    """Forward/backward against the fp64 oracle.  The pairs (token, expert, weight) come from
    `plan`; by default that is, for top-k routing, the oracle's own plan from the logits
    (oracle_plan: an end-to-end comparison in which nothing on the oracle side comes from the
    GPU) and, for token rounding and capacity plans, the GPU plan (verified bit-exact given the
    GPU's own probabilities beforehand, as those plans are defined).  toks/exps select a sample
    (None = everything)."""
    wl = T.wl
    tol = TOL[wl.dtype]
    if plan is None:
        plan = oracle_plan(T) if wl.routing == "topk" else res["plan"]
    pt, pe, pw = oracle.pairs_from_plan(plan, wl.E)
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
        gds = res["ds"].reshape(-1)[np.asarray(plan["row_pair"])[tr]]
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
