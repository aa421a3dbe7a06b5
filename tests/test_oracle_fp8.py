"""Pins of the oracle's MX-FP8 functions (oracle_quantize_mxfp8, oracle_layer_fwd_mxfp8), each
tied to something other than the oracle: torch's float8_e4m3fn cast (round to nearest even),
the quantization rule written as a literal search, exact round trips, numpy matrix products
on operands decoded by torch, exact scale equivariance, and the error bound of quantizing the
activation against the unquantized fp64 oracle.  CPU only."""
import numpy as np
import pytest
import torch

import oracle

E4M3_MAX = 448.0


def torch_e4m3_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(q, s):
    """Dequantize (codes, scale codes) with torch's e4m3 decoding and 2^(code - 127)."""
    vals = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    K = q.shape[-1]
    sc = 2.0 ** (s[..., : K // 32].astype(np.float64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def literal_scale_code(amax):
    """The rule as stated: the smallest s in [-127, 127] with amax <= 448 * 2^s."""
    for s in range(-127, 128):
        if amax <= E4M3_MAX * 2.0 ** s:
            return s + 127
    return 254


def e4m3_grid():
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def test_element_rounding_matches_torch_cast():
    """Blocks holding 448 have scale 1, so each other value is stored as its e4m3 rounding:
    every code, every midpoint and its fp32 neighbours, subnormals, signed zeros and random
    values agree with torch's float8_e4m3fn cast."""
    rng = np.random.default_rng(1)
    g = e4m3_grid()
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    vals = np.concatenate([g, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           rng.uniform(-448, 448, 4000), rng.uniform(-0.03, 0.03, 4000), [0.0, -0.0, 2.0 ** -10]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    n = -(-len(vals) // 31) * 31
    vals = np.concatenate([vals, np.zeros(n - len(vals), np.float32)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((len(vals), 1), 448.0, np.float32), vals], axis=1)  # [rows, 32]
    q, s = oracle.quantize_mxfp8(blocks)
    assert np.all(s[:, 0] == 127) and np.all(s[:, 1:] == 0)
    np.testing.assert_array_equal(q[:, 1:], torch_e4m3_codes(vals))
    assert np.all(q[:, 0] == 0x7E)


def test_scale_rule_against_literal_search():
    rng = np.random.default_rng(2)
    amax = [0.0, 448.0, 448.0 * 2.0 ** -20, 1.0, 2.0 ** -140, 2.0 ** -126, 3.0e38]
    for j in range(-40, 40, 3):
        b = 448.0 * 2.0 ** j
        amax += [b, float(np.nextafter(np.float32(b), np.float32(0))), float(np.nextafter(np.float32(b), np.float32(1e38)))]
    amax += list(np.ldexp(rng.uniform(0.5, 1.0, 300), rng.integers(-135, 120, 300)))
    amax = np.array(amax, np.float32)
    blocks = np.zeros((len(amax), 32), np.float32)
    blocks[:, 5] = -amax
    blocks[:, 9] = amax * np.float32(0.25)
    q, s = oracle.quantize_mxfp8(blocks)
    want = np.array([literal_scale_code(float(a)) for a in amax])
    np.testing.assert_array_equal(s[:, 0], want)
    # no value clips: |v| / X <= 448 everywhere
    X = 2.0 ** (s[:, 0].astype(np.float64) - 127)
    assert np.all(np.abs(blocks.astype(np.float64)) / X[:, None] <= E4M3_MAX)


def test_round_trip_of_representable_blocks():
    """Values that are e4m3 numbers times 2^j, in blocks whose largest is 448 * 2^j, come back
    exactly; all-zero blocks get scale code 0; scale entries past K / 32 are 0."""
    rng = np.random.default_rng(3)
    g = e4m3_grid()
    rows, K = 50, 96                           # K / 32 = 3 blocks, 4 scale bytes per row
    v = rng.choice(g, size=(rows, K)) * rng.choice([-1.0, 1.0], size=(rows, K))
    j = rng.integers(-20, 10, size=(rows, 3))
    v[:, ::32] = 448.0
    v = v * np.repeat(2.0 ** j, 32, axis=1)
    v[7, 32:64] = 0.0
    q, s = oracle.quantize_mxfp8(v.astype(np.float32))
    np.testing.assert_array_equal(torch_decode(q, s), v)
    assert s.shape == (rows, 4) and np.all(s[:, 3] == 0)
    assert s[7, 1] == 0 and np.all(q[7, 32:64] == 0)
    want = j + 127
    want[7, 1] = 0
    np.testing.assert_array_equal(s[:, :3], want)


def _small_layer(seed=4, N=40, H=64, I=96, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H)).astype(np.float32)
    wg = (0.05 * rng.standard_normal((E, I, H))).astype(np.float32)
    wu = (0.05 * rng.standard_normal((E, I, H))).astype(np.float32)
    wd = (0.05 * rng.standard_normal((E, H, I))).astype(np.float32)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    idx, w, _ = oracle.route_topk(lg, None, k)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    Q = [oracle.quantize_mxfp8(a) for a in (x, wg, wu, wd)]
    return Q, (pt, pe, pw), (N, H, I, E)


def test_layer_fwd_mxfp8_stages_against_numpy():
    """The forward's stages against numpy products on torch-decoded operands: [g | u] per pair,
    the quantized activation (torch's rounding of a / X with X from the literal rule), and the
    output sum over pairs."""
    Q, (pt, pe, pw), (N, H, I, E) = _small_layer()
    out, st = oracle.layer_fwd_mxfp8(*Q, pt, pe, pw, want_stages=True)
    xd, gd, ud, dd = (torch_decode(q, s) for q, s in Q)
    g = np.einsum("pih,ph->pi", gd[pe], xd[pt])
    u = np.einsum("pih,ph->pi", ud[pe], xd[pt])
    np.testing.assert_allclose(st["gu"], np.concatenate([g, u], axis=1), rtol=1e-12, atol=1e-12)
    a32 = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    for p in range(0, len(pt), 7):
        for b in range(I // 32):
            blk = a32[p, 32 * b:32 * b + 32]
            c = literal_scale_code(float(np.abs(blk).max()))
            assert st["as"][p, b] == c
            np.testing.assert_array_equal(st["aq"][p, 32 * b:32 * b + 32],
                                          torch_e4m3_codes(blk.astype(np.float64) / 2.0 ** (c - 127)))
    ad = torch_decode(st["aq"], st["as"])
    y = np.einsum("phi,pi->ph", dd[pe], ad)
    ref = np.zeros((N, H))
    np.add.at(ref, pt, pw[:, None].astype(np.float64) * y)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_layer_fwd_mxfp8_scale_equivariance():
    """Raising every scale code of W_down by one doubles the output exactly."""
    Q, (pt, pe, pw), _ = _small_layer(seed=5)
    out = oracle.layer_fwd_mxfp8(*Q, pt, pe, pw)
    dq, ds = Q[3]
    ds2 = ds.copy()
    K = dq.shape[-1]
    ds2[..., : K // 32] += 1
    out2 = oracle.layer_fwd_mxfp8(Q[0], Q[1], Q[2], (dq, ds2), pt, pe, pw)
    np.testing.assert_array_equal(out2, 2 * out)


def test_layer_fwd_mxfp8_within_activation_quantization_bound():
    """Against the fp64 oracle on the dequantized operands (no quantization of the activation):
    the difference is bounded by what quantizing a can change, |da_i| <= max(|a_i| 2^-4,
    2^-10 X_b) (half an e4m3 step) plus a's fp32 rounding, summed through |W_down| and w."""
    Q, (pt, pe, pw), (N, H, I, E) = _small_layer(seed=6, N=64, H=96, I=128, E=5)
    out = oracle.layer_fwd_mxfp8(*Q, pt, pe, pw)
    xd, gd, ud, dd = (torch_decode(q, s).astype(np.float32) for q, s in Q)  # exact in fp32
    plain = oracle.layer_fwd(xd, gd, ud, dd, pt, pe, pw)
    _, st = oracle.layer_fwd_mxfp8(*Q, pt, pe, pw, want_stages=True)
    g, u = st["gu"][:, :I], st["gu"][:, I:]
    a = g / (1 + np.exp(-g)) * u
    X = np.repeat(2.0 ** (st["as"][:, : I // 32].astype(np.float64) - 127), 32, axis=1)
    da = np.maximum(np.abs(a) * 2.0 ** -4, 2.0 ** -10 * X) + np.abs(a) * 2.0 ** -23
    bound = np.zeros((N, H))
    np.add.at(bound, pt, np.abs(pw)[:, None] * np.einsum("phi,pi->ph", np.abs(dd[pe]).astype(np.float64), da))
    diff = np.abs(out - plain)
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-12), float((diff / np.maximum(bound, 1e-30)).max())
    # and quantizing a does change the result (the test is not vacuous)
    assert diff.max() > 0


@pytest.mark.parametrize("K", [32, 64, 160, 2880])
def test_quantize_shapes_and_ragged_k(K):
    rng = np.random.default_rng(K)
    v = rng.standard_normal((9, K)).astype(np.float32) * 0.02
    q, s = oracle.quantize_mxfp8(v)
    assert q.shape == (9, K) and s.shape == (9, 4 * ((K + 127) // 128))
    assert np.all(s[:, K // 32:] == 0)
    d = torch_decode(q, s)
    # each value within half an e4m3 step (relative 2^-4, or 2^-10 X below the normal range)
    X = np.repeat(2.0 ** (s[:, : K // 32].astype(np.float64) - 127), 32, axis=1)
    assert np.all(np.abs(d - v) <= np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * X) * (1 + 1e-12))


def _small_bwd(seed=6, N=40, H=64, I=96, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H)).astype(np.float32)
    wg = (0.05 * rng.standard_normal((E, I, H))).astype(np.float32)
    wu = (0.05 * rng.standard_normal((E, I, H))).astype(np.float32)
    wd = (0.05 * rng.standard_normal((E, H, I))).astype(np.float32)
    dout = rng.standard_normal((N, H)).astype(np.float32)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    idx, w, _ = oracle.route_topk(lg, None, k)
    pt, pe, pw = oracle.pairs_from_topk(idx, w)
    return x, wg, wu, wd, dout, (pt, pe, pw), (N, H, I, E)


def test_layer_bwd_dh_output_reproduces_dx():
    """The backward's per-pair [dg | du] output, pushed through the weights by numpy
    (dx[t] = sum over t's pairs of W_gate[e]^T dg + W_up[e]^T du), gives the backward's own dx."""
    x, wg, wu, wd, dout, (pt, pe, pw), (N, H, I, E) = _small_bwd()
    r = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw, want=("dx", "dh"))
    dh = r["dh"]
    w64 = np.concatenate([wg.astype(np.float64), wu.astype(np.float64)], axis=1)  # [E, 2I, H]
    contrib = np.einsum("pkh,pk->ph", w64[pe], dh)
    ref = np.zeros((N, H))
    np.add.at(ref, pt, contrib)
    np.testing.assert_allclose(r["dx"], ref, rtol=1e-10, atol=1e-12)


def test_dx_weights_layout_and_codes():
    """The dX product's weight operand: row h of expert e is W_gate[e][:, h] then W_up[e][:, h],
    each 32-block quantized by the pinned row quantization (torch's e4m3 rounding of v / X,
    X from the literal scale rule)."""
    x, wg, wu, wd, dout, _, (N, H, I, E) = _small_bwd()
    q, s = oracle.dx_weights_mxfp8(wg, wu)
    assert q.shape == (E, H, 2 * I) and s.shape == (E, H, oracle.mx_scale_cols(2 * I))
    for e, h in ((0, 0), (1, 17), (E - 1, H - 1)):
        row = np.concatenate([wg[e, :, h], wu[e, :, h]]).astype(np.float64)
        for b in range(2 * I // 32):
            blk = row[32 * b:32 * b + 32]
            c = literal_scale_code(float(np.abs(blk).max()))
            assert s[e, h, b] == c
            np.testing.assert_array_equal(q[e, h, 32 * b:32 * b + 32], torch_e4m3_codes(blk / 2.0 ** (c - 127)))


def test_dx_mxfp8_against_numpy():
    """The dX product on MX-FP8 operands against a numpy product of torch-decoded operands:
    each pair's dh row quantized by the literal rule, times its expert's decoded weight rows,
    summed per token."""
    x, wg, wu, wd, dout, (pt, pe, pw), (N, H, I, E) = _small_bwd()
    dh = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw, want=("dh",))["dh"].astype(np.float32)
    wt = oracle.dx_weights_mxfp8(wg, wu)
    dx, dq, dsc = oracle.dx_mxfp8(dh, wt, pt, pe, N, want_codes=True)
    for p in range(0, len(pt), 5):
        for b in range(2 * I // 32):
            blk = dh[p, 32 * b:32 * b + 32].astype(np.float64)
            c = literal_scale_code(float(np.abs(blk).max()))
            assert dsc[p, b] == c
            np.testing.assert_array_equal(dq[p, 32 * b:32 * b + 32], torch_e4m3_codes(blk / 2.0 ** (c - 127)))
    wdec = torch_decode(*wt)  # [E, H, 2I]
    contrib = np.einsum("phk,pk->ph", wdec[pe], torch_decode(dq, dsc))
    ref = np.zeros((N, H))
    np.add.at(ref, pt, contrib)
    np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-12)


def test_dx_mxfp8_within_quantization_bound():
    """Against the unquantized fp64 dx: the error stays within what quantizing both operands
    allows (each e4m3 value within 2^-4 relative, so a product within about 2^-3 of its
    magnitude): |dx_q - dx| <= 0.13 sum |dh| |W| per element."""
    x, wg, wu, wd, dout, (pt, pe, pw), (N, H, I, E) = _small_bwd()
    r = oracle.layer_bwd(dout, x, wg, wu, wd, pt, pe, pw, want=("dx", "dh"))
    dxq = oracle.dx_mxfp8(r["dh"].astype(np.float32), oracle.dx_weights_mxfp8(wg, wu), pt, pe, N)
    w64 = np.abs(np.concatenate([wg.astype(np.float64), wu.astype(np.float64)], axis=1))
    bound = np.zeros((N, H))
    np.add.at(bound, pt, np.einsum("pkh,pk->ph", w64[pe], np.abs(r["dh"])))
    assert np.all(np.abs(dxq - r["dx"]) <= 0.13 * bound + 1e-12)
    assert np.abs(dxq - r["dx"]).max() > 0  # the quantization is not the identity here
