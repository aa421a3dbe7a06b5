"""GPU parity of the MX-FP8 path (moe_quantize_mxfp8, moe_grouped_gemm_fwd_mxfp8) against the
oracle's MX-FP8 functions, through the C ABI, every buffer guarded:

* quantization: codes and scale codes bit-exact (integer results of exact arithmetic: a
  bf16 value scaled by a power of two and rounded to nearest e4m3), for activations and
  weights of the headline layer, K tails (K = 2880, K = 96), zero and tiny blocks, fp32 input;
* forward: [G | U] (hcache) and the combined output within 1e-2 of the oracle's fp64 result
  (max |diff| / max |ref|); the quantized activation A, a decision the kernel takes on its own
  fp32 value of A: at least 99 % of its codes equal the oracle's, and every code is a
  round-to-nearest e4m3 code (at the kernel's block scale) of a value within 1e-4 of the
  oracle's fp64 A, with block scales one step apart at most and only at a power-of-two
  threshold of the block maximum; two runs bitwise identical."""
import numpy as np
import pytest

import oracle
from grouped_gemm_top_amd import workloads as W
from harness import Guards, check_routing, log, oracle_plan, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import grouped_gemm_top_amd as G
    G.lib()


def _quant_gpu(g, name, arr, dtype="bf16"):
    import torch
    import grouped_gemm_top_amd as G
    from grouped_gemm_top_amd.workloads import bf16_round
    src = g.upload(name, bf16_round(arr) if dtype == "bf16" else np.ascontiguousarray(arr, np.float32))
    K = arr.shape[-1]
    q = g.alloc(name + "_q", arr.shape, torch.uint8)
    s = g.alloc(name + "_s", arr.shape[:-1] + (G.mx_scale_cols(K),), torch.uint8)
    G.quantize_mxfp8(src, q=q, scales=s)
    g.check(f"quantize_mxfp8({name})")
    return q, s


def _assert_quant_equal(gq, gs, arr):
    oq, os_ = oracle.quantize_mxfp8(arr)
    np.testing.assert_array_equal(gs.cpu().numpy(), os_)
    np.testing.assert_array_equal(gq.cpu().numpy(), oq)


def test_quantize_bit_exact_headline_tensors():
    wl = W.WORKLOADS[2]
    T = W.generate(wl)
    g = Guards()
    for name, arr in (("x", T.x), ("wg", T.wg), ("wd", T.wd)):
        log(f"[quantize] {name} {arr.shape}")
        q, s = _quant_gpu(g, name, arr)
        _assert_quant_equal(q, s, arr)
        g.bufs.clear()


@pytest.mark.parametrize("K", [96, 2880])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact_edge_blocks(K, dtype):
    """Ragged K (scale padding), all-zero blocks, tiny and huge magnitudes, exact 448 * 2^j
    boundaries and values just past them."""
    from grouped_gemm_top_amd.workloads import bf16_round, bf16_to_f32
    rng = np.random.default_rng(K)
    a = (rng.standard_normal((37, K)) * np.exp2(rng.integers(-30, 30, (37, 1)))).astype(np.float32)
    a[3] = 0.0
    a[5, :32] = 0.0
    a[7] *= np.float32(2.0 ** -100)
    a[8, :32] = np.float32(448.0 * 2.0 ** -3)
    a[9, 1] = np.float32(448.0 * 2.0 ** 5)
    a[9, 2] = np.nextafter(np.float32(448.0 * 2.0 ** 5), np.float32(1e30))
    if dtype == "bf16":
        a = bf16_to_f32(bf16_round(a))
    g = Guards()
    q, s = _quant_gpu(g, "a", a, dtype)
    _assert_quant_equal(q, s, a)


def _run_fp8(T):
    """Route + permute (bf16 path) on the GPU, quantize x and the weights, the MX-FP8 forward and
    the combine; returns host copies and the GPU plan."""
    import torch
    import grouped_gemm_top_amd as G
    wl = T.wl
    N, H, I, E, k = wl.N, wl.H, wl.I, wl.E, wl.k
    g = Guards()
    logits = g.upload("logits", T.logits)
    bias = None if T.bias is None else g.upload("bias", T.bias)
    idx = g.alloc("idx", (N, k), torch.int32)
    w = g.alloc("w", (N, k), torch.float32)
    G.route_topk(logits, k, bias=bias, idx=idx, w=w)
    plan = G.Plan(N, E, k, alloc=lambda name, n, dt: g.alloc("plan." + name, (n,), dt))
    ws = g.alloc("ws_perm", (G.workspace_bytes(G.OP_PERMUTE, G.MOE_BF16, N, E, k),), torch.uint8)
    G.permute(idx, w, E, plan=plan, ws=ws)
    g.check("route/permute")
    x = _quant_gpu(g, "x", T.x)
    wg = _quant_gpu(g, "wg", T.wg)
    wu = _quant_gpu(g, "wu", T.wu)
    wd = _quant_gpu(g, "wd", T.wd)
    mc = plan.M_cap
    hc = g.alloc("hcache", (mc, 2 * I), torch.bfloat16)
    y = g.alloc("y", (mc, H), torch.bfloat16)
    nb = G.workspace_bytes(G.OP_GEMM_FWD_MXFP8, G.MOE_BF16, N, E, k, H, I, mc)
    ws = g.alloc("ws_fwd8", (nb,), torch.uint8)
    G.grouped_gemm_fwd_mxfp8(x, wg, wu, wd, plan, hcache=hc, y=y, ws=ws)
    g.check("grouped_gemm_fwd_mxfp8")
    out = g.alloc("out", (N, H), torch.bfloat16)
    G.unpermute_combine(y, plan, out=out)
    g.check("unpermute_combine")
    torch.cuda.synchronize()
    m = int(plan.offsets[-1].item())
    aoff = (mc * I + 255) // 256 * 256
    ksi = G.mx_scale_cols(I)
    wsh = ws.cpu().numpy()
    res = dict(idx=idx.cpu().numpy(), w=w.cpu().numpy(), probs=None, plan=plan.host(),
               hcache=hc[:m].float().cpu().numpy(), out=out.float().cpu().numpy(),
               aq=wsh[: m * I].reshape(m, I), as_=wsh[aoff: aoff + m * ksi].reshape(m, ksi),
               xq=x[0].cpu().numpy(), xs=x[1].cpu().numpy())
    return res


def _check_fp8(T, res, toks=None):
    wl = T.wl
    op = oracle_plan(T)
    for n in ("counts", "offsets", "row_token", "row_pair"):
        np.testing.assert_array_equal(res["plan"][n], op[n], err_msg=n)
    Q = [oracle.quantize_mxfp8(a) for a in (T.x, T.wg, T.wu, T.wd)]
    np.testing.assert_array_equal(res["xq"], Q[0][0])
    np.testing.assert_array_equal(res["xs"], Q[0][1])
    pt, pe, pw = oracle.pairs_from_plan(op, wl.E)
    rows = np.arange(len(pt))
    if toks is not None:
        keep = np.isin(pt, toks)
        rows, pt, pe, pw = rows[keep], pt[keep], pe[keep], pw[keep]
    else:
        toks = np.arange(wl.N)
    out, st = oracle.layer_fwd_mxfp8(*Q, pt, pe, pw, want_stages=True)
    errs = {"out": rel_err(res["out"][toks], out[toks]), "hcache": rel_err(res["hcache"][rows], st["gu"])}
    I = wl.I
    ga, oa = res["aq"][rows], st["aq"]
    gsc, osc = res["as_"][rows][:, : I // 32].astype(np.int64), st["as"][:, : I // 32].astype(np.int64)
    errs["a_codes_equal"] = float(np.mean(ga == oa))
    errs["a_scales_equal"] = float(np.mean(gsc == osc))
    # The kernel quantizes its own fp32 A, the product of the fp8 matrix instruction, whose
    # accumulation differs from the oracle's fp64 sums (most where a dot product cancels, by up
    # to ~1e-5 of the block's largest |A|).  So each GPU value (code times the GPU's block scale
    # X) must lie within half an e4m3 step of the oracle's a, plus 1e-4 of the block's largest
    # |a| for the accumulation difference; a wrong scale or a wrong code is far outside that.
    # A block scale may differ only by one step where the block's largest |a| sits within 1e-3
    # of a power-of-two threshold.
    g, u = st["gu"][:, :I], st["gu"][:, I:]
    a = g / (1.0 + np.exp(-g)) * u
    amax = np.abs(a).reshape(len(a), I // 32, 32).max(axis=2)
    sd = gsc != osc
    assert np.all(np.abs(gsc - osc)[sd] == 1), "scale codes more than one step apart"
    thr = 448.0 * 2.0 ** (np.minimum(gsc, osc)[sd] - 127)
    assert np.all(np.abs(amax[sd] - thr) <= 1e-3 * thr), "a scale differs away from a threshold"
    X = np.repeat(2.0 ** (gsc - 127.0), 32, axis=1)
    t = np.abs(a) / X
    half = np.where(t < 2.0 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -126))) - 4))
    dev = np.abs(torch_e4m3(ga) * X - a)
    bad = dev > half * X * (1 + 1e-6) + 1e-4 * np.repeat(amax, 32, axis=1)
    log(f"[fp8 {wl.name}] {errs}; A codes differing from the oracle's {int((ga != oa).sum())} of {ga.size}, "
        f"outside the bound {int(bad.sum())}, largest deviation / block max "
        f"{float((np.maximum(dev - half * X, 0) / np.repeat(amax, 32, axis=1)).max()):.2e}")
    assert errs["out"] <= 1e-2 and errs["hcache"] <= 1e-2, errs
    assert not bad.any(), (errs, np.argwhere(bad)[:5])
    assert errs["a_codes_equal"] >= 0.99, errs
    return errs


def torch_e4m3(q):
    import torch
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("shape", [
    dict(N=300, H=256, I=96, E=6, k=2),        # I not a multiple of 64: half-used column groups
    dict(N=48, H=2880, I=2880, E=4, k=2),      # K tails of both GEMMs (2880 = 22.5 * 128)
    dict(N=200, H=512, I=384, E=9, k=3),       # several N-tiles, ragged groups
])
def test_fwd_mxfp8_against_oracle(shape):
    wl = W.custom("fp8", dtype="bf16", bias="normal", bias_std=0.5, seed=41, **shape)
    T = W.generate(wl)
    res = _run_fp8(T)
    res2 = _run_fp8(T)
    for n in ("hcache", "out", "aq", "as_"):
        assert np.array_equal(res[n].view(np.uint8), res2[n].view(np.uint8)), n
    _check_fp8(T, res)


def test_fwd_mxfp8_headline_sampled():
    """The headline layer (E=128, H=2048, I=512, k=8, N=4096), compared on the rows of 256
    sampled tokens (rows are independent given the weights)."""
    T = W.generate(W.WORKLOADS[2])
    res = _run_fp8(T)
    toks = np.sort(np.random.default_rng(2).choice(T.wl.N, 256, replace=False))
    _check_fp8(T, res, toks)


def _run_bwd8(T):
    """Route, permute and bf16 forward, then the backward twice on the same plan: layer_bwd
    (bf16 dX product) and layer_bwd_mxfp8 (MX-FP8 dX product, weights from
    quantize_dx_weights_mxfp8); every buffer guarded.  Returns host copies, including the fp8
    backward's dH (bf16), its codes and scale codes, read from the workspace."""
    import torch
    import grouped_gemm_top_amd as G
    from harness import upload
    wl = T.wl
    N, H, I, E, k = wl.N, wl.H, wl.I, wl.E, wl.k
    D = upload(T)
    g = D["guards"]
    f32, i32, u8, bf = torch.float32, torch.int32, torch.uint8, torch.bfloat16
    idx, w = g.alloc("idx", (N, k), i32), g.alloc("w", (N, k), f32)
    probs = g.alloc("probs", (N, E), f32)
    alloc = lambda name, n, dtype: g.alloc("plan." + name, (n,), dtype)  # noqa: E731
    if wl.routing == "tr":
        plan = G.Plan(N, E, k, kind=G.PLAN_TR, mtile=wl.mtile, alloc=alloc)
        G.route_token_rounding(D["logits"], k, wl.mtile, bias=D["bias"], plan=plan, idx=idx, w=w, probs=probs,
                               ws=g.alloc("ws_tr", (G.workspace_bytes(G.OP_ROUTE_TR, G.MOE_BF16, N, E, k),), u8))
    else:
        G.route_topk(D["logits"], k, bias=D["bias"], idx=idx, w=w, probs=probs)
        plan = G.Plan(N, E, k, alloc=alloc)
        G.permute(idx, w, E, plan=plan,
                  ws=g.alloc("ws_perm", (G.workspace_bytes(G.OP_PERMUTE, G.MOE_BF16, N, E, k),), u8))
    mc = plan.M_cap
    hc, y = g.alloc("hcache", (mc, 2 * I), bf), g.alloc("y", (mc, H), bf)
    G.grouped_gemm_fwd(D["x"], D["wg"], D["wu"], D["wd"], plan, hcache=hc, y=y,
                       ws=g.alloc("ws_fwd", (G.workspace_bytes(G.OP_GEMM_FWD, G.MOE_BF16, N, E, k, H, I, mc),), u8))
    wt = (g.alloc("wt_q", (E, H, 2 * I), u8), g.alloc("wt_s", (E, H, G.mx_scale_cols(2 * I)), u8))
    G.quantize_dx_weights_mxfp8(D["wg"], D["wu"], q=wt[0], scales=wt[1])
    g.check("quantize_dx_weights_mxfp8")
    outs = {}
    for tag in ("bf16", "fp8"):
        o = dict(dx=g.alloc(f"dx_{tag}", (N, H), bf), dw_gate=g.alloc(f"dwg_{tag}", (E, I, H), bf),
                 dw_up=g.alloc(f"dwu_{tag}", (E, I, H), bf), dw_down=g.alloc(f"dwd_{tag}", (E, H, I), bf),
                 ds=g.alloc(f"ds_{tag}", (N, k) if wl.routing != "tr" else (mc,), f32))
        if tag == "bf16":
            nb = G.workspace_bytes(G.OP_LAYER_BWD, G.MOE_BF16, N, E, k, H, I, mc)
            ws = g.alloc("ws_bwd", (nb,), u8)
            G.layer_bwd(D["dout"], D["x"], D["wg"], D["wu"], D["wd"], plan, hc, ws=ws, **o)
        else:
            nb = G.workspace_bytes(G.OP_LAYER_BWD_MXFP8, G.MOE_BF16, N, E, k, H, I, mc)
            ws = g.alloc("ws_bwd8", (nb,), u8)
            G.layer_bwd_mxfp8(D["dout"], D["x"], D["wg"], D["wu"], D["wd"], wt, plan, hc, ws=ws, **o)
        g.check(f"layer_bwd ({tag})")
        outs[tag] = {n: t.cpu().numpy() if t.dtype != bf else t.view(torch.int16).cpu().numpy() for n, t in o.items()}
    torch.cuda.synchronize()
    a256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    m = int(plan.offsets[-1].item())
    wsh = ws.cpu().numpy()
    o_ap = a256(mc * 2 * I * 2)                       # dH [M_cap, 2I] bf16 at 0, then A' (dH codes)
    o_sc = o_ap + a256(mc * I * 2) + a256(mc * H * 2) + a256(mc * 2 * ((I + 255) // 256) * 4)
    ks = G.mx_scale_cols(2 * I)
    res = dict(plan=plan.host(), outs=outs, wtq=wt[0].cpu().numpy(), wts=wt[1].cpu().numpy(),
               idx=idx.cpu().numpy(), probs=probs.cpu().numpy(),
               dh_bits=wsh[: m * 2 * I * 2].view(np.uint16).reshape(m, 2 * I),
               dhq=wsh[o_ap: o_ap + m * 2 * I].reshape(m, 2 * I), dhs=wsh[o_sc: o_sc + m * ks].reshape(m, ks))
    return res


def _check_bwd8(T, res, toks=None):
    wl = T.wl
    N, E = wl.N, wl.E
    if wl.routing == "tr":
        # the token-rounding plan, bit-exact given the GPU's own probabilities and indices; the
        # oracle side then runs on it
        op = oracle.token_round(res["probs"], res["idx"], wl.mtile)
    else:
        op = oracle_plan(T)
    for n in ("counts", "offsets", "row_token", "row_pair"):
        np.testing.assert_array_equal(res["plan"][n], op[n], err_msg=n)
    # the weight operand: bit-exact
    oq, os_ = oracle.dx_weights_mxfp8(T.wg, T.wu)
    np.testing.assert_array_equal(res["wts"], os_)
    np.testing.assert_array_equal(res["wtq"], oq)
    # weight gradients and dS: the same kernels as the bf16 backward, bit for bit
    b, f = res["outs"]["bf16"], res["outs"]["fp8"]
    for n in ("dw_gate", "dw_up", "dw_down", "ds"):
        assert np.array_equal(b[n], f[n]), n
    # the quantization of the GPU's own dH (bf16 values from the workspace): bit-exact
    dh_gpu = W.bf16_to_f32(res["dh_bits"])
    q, s = oracle.quantize_mxfp8(dh_gpu)
    np.testing.assert_array_equal(res["dhs"], s)
    np.testing.assert_array_equal(res["dhq"], q)
    # dH and dx against the oracle: dh of the oracle's own pairs, stored in bf16 (the layer's
    # storage type), quantized and multiplied by the oracle's weight operand
    pt, pe, pw = oracle.pairs_from_plan(op, E)
    rows = np.arange(len(pt))
    if toks is not None:
        keep = np.isin(pt, toks)
        rows, pt, pe, pw = rows[keep], pt[keep], pe[keep], pw[keep]
    else:
        toks = np.arange(N)
    dh = oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt, pe, pw, want=("dh",))["dh"]
    dhb = W.bf16_to_f32(W.bf16_round(dh.astype(np.float32)))
    dx_gpu = W.bf16_to_f32(f["dx"].view(np.uint16))
    # The quantization of dH is a decision taken on the bf16 values each side holds, and the
    # GPU's dH differs from the oracle's by bf16 rounding steps (fp32 against fp64 sums), which
    # moves a few codes by one e4m3 step.  So, as for plans that depend on the GPU's
    # probabilities: the GPU's codes are checked bit-exact given its dH (above), its dH against
    # the oracle's, and the product against the oracle run on the GPU's dH; the end-to-end
    # result from the oracle's own dH is held to the bound of those code steps.  (The GPU's
    # dSwiGLU reads G and U from the bf16 hcache while the oracle recomputes them in fp64, so
    # nearly every dH value differs by bf16 steps and a few % of the codes by one e4m3 step.)
    dx_cond = oracle.dx_mxfp8(dh_gpu[rows], (oq, os_), pt, pe, N)
    dx_e2e, oq2, os2 = oracle.dx_mxfp8(dhb, (oq, os_), pt, pe, N, want_codes=True)
    errs = {"dh": rel_err(dh_gpu[rows], dh), "dx": rel_err(dx_gpu[toks], dx_cond[toks]),
            "dx_end_to_end": rel_err(dx_gpu[toks], dx_e2e[toks]),
            "dh_codes_equal": float(np.mean(res["dhq"][rows] == oq2)),
            "dx_vs_bf16_path": rel_err(dx_gpu[toks], W.bf16_to_f32(b["dx"].view(np.uint16))[toks])}
    log(f"[bwd fp8 {wl.name}] {errs}")
    assert errs["dh"] <= 1e-2 and errs["dx"] <= 1e-2, errs
    assert errs["dh_codes_equal"] >= 0.95 and errs["dx_end_to_end"] <= 5e-2, errs
    return errs


@pytest.mark.parametrize("shape", [
    dict(N=300, H=256, I=96, E=6, k=2),        # 2I = 192: a K tail in the 128-wide fp8 k-steps
    dict(N=200, H=512, I=384, E=9, k=3),       # several N-tiles, ragged groups
])
def test_bwd_dx_mxfp8_against_oracle(shape):
    wl = W.custom("bwd8", dtype="bf16", bias="normal", bias_std=0.5, seed=43, **shape)
    T = W.generate(wl)
    res = _run_bwd8(T)
    res2 = _run_bwd8(T)
    assert np.array_equal(res["outs"]["fp8"]["dx"], res2["outs"]["fp8"]["dx"])
    _check_bwd8(T, res)


def test_bwd_dx_mxfp8_token_rounding():
    """A token-rounding plan (row capacity above the rows used, dS in row order): dW and dS
    bitwise as in the bf16 backward, dH's codes bit-exact, dx within 1e-2 on the GPU's codes."""
    wl = W.custom("bwd8-tr", N=320, H=256, I=128, E=8, k=2, dtype="bf16", bias="normal", bias_std=0.4,
                  routing="tr", mtile=32, seed=47)
    T = W.generate(wl)
    res = _run_bwd8(T)
    assert int(res["plan"]["offsets"][-1]) > 0
    _check_bwd8(T, res)


def test_bwd_dx_mxfp8_headline_sampled():
    """The headline layer, dx compared on 64 sampled tokens (rows are independent given the
    weights); the weight codes, dH's codes, dW and dS in full."""
    T = W.generate(W.WORKLOADS[2])
    res = _run_bwd8(T)
    toks = np.sort(np.random.default_rng(3).choice(T.wl.N, 64, replace=False))
    _check_bwd8(T, res, toks)
