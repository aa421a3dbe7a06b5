"""ctypes wrapper over the plain C oracle in ``moe_oracle.c``.

Test infrastructure: importable only by tests, the smoke check and the benchmark's
CPU-baseline leg.  Arrays go in and out as numpy arrays on the host.  The C file is built
with gcc into ``liboracle_f64.so`` (fp64 arithmetic, used for parity) and
``liboracle_f32.so`` (fp32 arithmetic, used only as a timing baseline).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIBS: dict = {}

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def lib_path(real: str = "f64") -> str:
    """The oracle library; ORACLE_LIB_DIR (set only by the sanitizer tests) names a directory
    holding another build of the same source, e.g. with AddressSanitizer."""
    return os.path.join(os.environ.get("ORACLE_LIB_DIR") or _HERE, f"liboracle_{real}.so")


def build(verbose: bool = False) -> None:
    """Compile both oracle variants with gcc (always recompiles)."""
    for real, ctype in (("f64", "double"), ("f32", "float")):
        out = lib_path(real)
        tmp = out + ".tmp"
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", f"-DORACLE_REAL={ctype}",
               "-fvisibility=hidden", _SRC, "-o", tmp, "-lm"]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    _LIBS.clear()


def _lib(real: str = "f64"):
    if real in _LIBS:
        return _LIBS[real]
    path = lib_path(real)
    if os.environ.get("ORACLE_LIB_DIR"):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing")
    elif not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(path)
    lib.oracle_route_topk.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _i32p, _f32p, _f32p]
    lib.oracle_permute.argtypes = [_i32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   _i32p, _i32p, _i32p, _f32p, _i32p, _i32p, _i32p]
    lib.oracle_token_round.argtypes = [_f32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, _i32p, _i32p, _i32p, _f32p,
                                       _i32p, _i32p, _i32p]
    lib.oracle_layer_fwd.argtypes = [_f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _f32p,
                                     _f64p]
    lib.oracle_layer_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _i32p, _i32p, _f32p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_capacity_plan.argtypes = [_f32p, _i32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _i32p, _f32p,
                                         _i32p, _i32p, _i32p]
    lib.oracle_router_logits.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _f32p]
    lib.oracle_router_bwd.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p,
                                      ctypes.c_int, _i32p, _i32p, _f32p, _f32p, _f32p, ctypes.c_int,
                                      _f64p, _f64p, _f64p, _f64p]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    _u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_quantize_mxfp8.argtypes = [_f32p, ctypes.c_long, ctypes.c_int, _u8p, _u8p]
    lib.oracle_layer_fwd_mxfp8.argtypes = [_u8p, _u8p, _u8p, _u8p, _u8p, _u8p, _u8p, _u8p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p,
                                           _f32p, _f64p, _f64p, _u8p, _u8p]
    lib.oracle_dx_mxfp8.argtypes = [_f32p, _u8p, _u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, _i32p, _i32p, _f64p, _u8p, _u8p]
    for fn in ("oracle_quantize_mxfp8", "oracle_layer_fwd_mxfp8", "oracle_dx_mxfp8", "oracle_set_threads", "oracle_route_topk", "oracle_permute", "oracle_token_round", "oracle_layer_fwd",
               "oracle_layer_bwd", "oracle_router_logits", "oracle_router_bwd", "oracle_capacity_plan",
               "oracle_real_bytes",
               "oracle_threads"):
        getattr(lib, fn).restype = ctypes.c_int
    _LIBS[real] = lib
    return lib


def threads(real: str = "f64") -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_lib(real).oracle_threads())


def set_threads(n: int, real: str = "f64") -> int:
    """Use n OpenMP threads in later calls (from this thread); returns the resulting count."""
    return int(_lib(real).oracle_set_threads(int(n)))


def _p(a, t):
    if a is None:
        return None
    return a.ctypes.data_as(t)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc < 0:
        raise RuntimeError(f"{what} failed with code {rc}")
    return rc


def route_topk(logits, bias, k, real="f64", want_probs=False):
    """Returns (idx [N,k] int32, w [N,k] float32, probs [N,E] float32 or None)."""
    logits = _f32(logits)
    N, E = logits.shape
    bias = None if bias is None else _f32(bias)
    idx = np.empty((N, k), np.int32)
    w = np.empty((N, k), np.float32)
    probs = np.empty((N, E), np.float32) if want_probs else None
    _check(_lib(real).oracle_route_topk(_p(logits, _f32p), _p(bias, _f32p), N, E, k,
                                        _p(idx, _i32p), _p(w, _f32p), _p(probs, _f32p)),
           "oracle_route_topk")
    return idx, w, probs


def _plan_arrays(N, E, mcap):
    return dict(counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
                row_token=np.empty(mcap, np.int32), row_w=np.empty(mcap, np.float32),
                row_pair=np.empty(mcap, np.int32), tok_ptr=np.empty(N + 1, np.int32),
                tok_rows=np.empty(mcap, np.int32))


def permute(idx, w, E):
    """Top-k routing plan: dict of counts, offsets, row_token, row_w, row_pair, tok_ptr,
    tok_rows (numpy, exactly M = N*k rows)."""
    idx = _i32(idx)
    w = _f32(w)
    N, k = idx.shape
    pl = _plan_arrays(N, E, N * k)
    _check(_lib().oracle_permute(_p(idx, _i32p), _p(w, _f32p), N, E, k,
                                 *[_p(pl[n], _i32p if pl[n].dtype == np.int32 else _f32p)
                                   for n in ("counts", "offsets", "row_token", "row_w",
                                             "row_pair", "tok_ptr", "tok_rows")]),
           "oracle_permute")
    return pl


def token_round(probs, idx, mtile, mcap=None):
    """Token-rounding plan given fp32 probs [N,E] and the top-k idx [N,k].  Arrays are
    trimmed to the actual row count M."""
    probs = _f32(probs)
    idx = _i32(idx)
    N, E = probs.shape
    k = idx.shape[1]
    if mcap is None:
        mcap = N * k + E * (mtile // 2)
    pl = _plan_arrays(N, E, max(mcap, 1))
    m = _check(_lib().oracle_token_round(_p(probs, _f32p), _p(idx, _i32p), N, E, k, mtile, mcap,
                                         *[_p(pl[n], _i32p if pl[n].dtype == np.int32 else _f32p)
                                           for n in ("counts", "offsets", "row_token", "row_w",
                                                     "row_pair", "tok_ptr", "tok_rows")]),
               "oracle_token_round")
    for n in ("row_token", "row_w", "row_pair", "tok_rows"):
        pl[n] = pl[n][:m].copy()
    return pl


def capacity_plan(idx, w, E, C, policy, probs=None):
    """Capacity plan: each expert keeps at most C of its assigned tokens, lined up by token
    index (policy 0, "position") or by P[t,e] descending then token (policy 1, "probs").
    Arrays are trimmed to the actual row count M."""
    idx = _i32(idx)
    w = _f32(w)
    N, k = idx.shape
    mcap = max(N * k, 1)
    pl = _plan_arrays(N, E, mcap)
    pp = None if probs is None else _f32(probs)
    m = _check(_lib().oracle_capacity_plan(_p(pp, _f32p), _p(idx, _i32p), _p(w, _f32p), N, E, k, C, policy, mcap,
                                           *[_p(pl[n], _i32p if pl[n].dtype == np.int32 else _f32p)
                                             for n in ("counts", "offsets", "row_token", "row_w",
                                                       "row_pair", "tok_ptr", "tok_rows")]),
               "oracle_capacity_plan")
    for n in ("row_token", "row_w", "row_pair", "tok_rows"):
        pl[n] = pl[n][:m].copy()
    return pl


def pairs_from_topk(idx, w):
    """Flat (token, expert, weight) pair lists in (t, j) order."""
    idx = _i32(idx)
    N, k = idx.shape
    t = np.repeat(np.arange(N, dtype=np.int32), k)
    return t, idx.reshape(-1).copy(), _f32(w).reshape(-1).copy()


def pairs_from_plan(plan, E):
    """Flat pair lists in row order from a plan (row r -> token row_token[r], the expert
    whose slice holds r, weight row_w[r])."""
    counts = np.asarray(plan["counts"])
    e = np.repeat(np.arange(E, dtype=np.int32), counts)
    m = int(counts.sum())
    return _i32(plan["row_token"][:m]), e, _f32(plan["row_w"][:m])


def layer_fwd(x, wg, wu, wd, pair_t, pair_e, pair_w, real="f64"):
    """out [N,H] float64 = sum over pairs of w * expert_e(x_t)."""
    x, wg, wu, wd = _f32(x), _f32(wg), _f32(wu), _f32(wd)
    N, H = x.shape
    E, I, _ = wg.shape
    pair_t, pair_e, pair_w = _i32(pair_t), _i32(pair_e), _f32(pair_w)
    out = np.empty((N, H), np.float64)
    _check(_lib(real).oracle_layer_fwd(_p(x, _f32p), _p(wg, _f32p), _p(wu, _f32p), _p(wd, _f32p),
                                       N, H, I, E, len(pair_t), _p(pair_t, _i32p),
                                       _p(pair_e, _i32p), _p(pair_w, _f32p), _p(out, _f64p)),
           "oracle_layer_fwd")
    return out


def layer_bwd(dout, x, wg, wu, wd, pair_t, pair_e, pair_w, want=("dx", "dwg", "dwu", "dwd", "ds"),
              real="f64"):
    """Returns a dict with the requested float64 gradients: dx [N,H], dwg/dwu [E,I,H],
    dwd [E,H,I], ds [P] (per pair), dh [P,2I] (each pair's [dg | du], only when asked for)."""
    dout, x, wg, wu, wd = _f32(dout), _f32(x), _f32(wg), _f32(wu), _f32(wd)
    N, H = x.shape
    E, I, _ = wg.shape
    pair_t, pair_e, pair_w = _i32(pair_t), _i32(pair_e), _f32(pair_w)
    P = len(pair_t)
    res = {}
    res["dx"] = np.empty((N, H), np.float64) if "dx" in want else None
    res["dwg"] = np.empty((E, I, H), np.float64) if "dwg" in want else None
    res["dwu"] = np.empty((E, I, H), np.float64) if "dwu" in want else None
    res["dwd"] = np.empty((E, H, I), np.float64) if "dwd" in want else None
    res["ds"] = np.empty((P,), np.float64) if "ds" in want else None
    res["dh"] = np.empty((P, 2 * I), np.float64) if "dh" in want else None
    _check(_lib(real).oracle_layer_bwd(_p(dout, _f32p), _p(x, _f32p), _p(wg, _f32p), _p(wu, _f32p),
                                       _p(wd, _f32p), N, H, I, E, P, _p(pair_t, _i32p),
                                       _p(pair_e, _i32p), _p(pair_w, _f32p),
                                       *[_p(res[n], _f64p) for n in ("dx", "dwg", "dwu", "dwd", "ds", "dh")]),
           "oracle_layer_bwd")
    return {n: v for n, v in res.items() if v is not None}


def router_logits(x, wr, bias=None, real="f64"):
    """logits [N,E] float32 = x @ W_r (+ bias), accumulated in `real`, rounded once."""
    x, wr = _f32(x), _f32(wr)
    N, H = x.shape
    E = wr.shape[1]
    bias = None if bias is None else _f32(bias)
    out = np.empty((N, E), np.float32)
    _check(_lib(real).oracle_router_logits(_p(x, _f32p), _p(wr, _f32p), _p(bias, _f32p), N, H, E,
                                           _p(out, _f32p)),
           "oracle_router_logits")
    return out


def router_bwd(logits, bias, idx, pair_t, pair_e, pair_ds, x=None, wr=None,
               want=("dz", "dwr", "dx", "dbias"), real="f64"):
    """Router backward from the per-pair gradients dS (one entry per final pair).
    Returns float64 dz [N,E] and, as requested, dwr [H,E], dx [N,H] (router share only),
    dbias [E]."""
    logits = _f32(logits)
    N, E = logits.shape
    idx = _i32(idx)
    k = idx.shape[1]
    bias = None if bias is None else _f32(bias)
    pair_t, pair_e, pair_ds = _i32(pair_t), _i32(pair_e), _f32(pair_ds)
    H = 1
    if x is not None:
        x, wr = _f32(x), _f32(wr)
        H = x.shape[1]
    res = {"dz": np.empty((N, E), np.float64)}
    res["dwr"] = np.empty((H, E), np.float64) if ("dwr" in want and x is not None) else None
    res["dx"] = np.empty((N, H), np.float64) if ("dx" in want and x is not None) else None
    res["dbias"] = np.empty((E,), np.float64) if "dbias" in want else None
    _check(_lib(real).oracle_router_bwd(_p(logits, _f32p), _p(bias, _f32p), N, E, k, _p(idx, _i32p),
                                        len(pair_t), _p(pair_t, _i32p), _p(pair_e, _i32p),
                                        _p(pair_ds, _f32p), _p(x, _f32p), _p(wr, _f32p), H,
                                        *[_p(res[n], _f64p) for n in ("dz", "dwr", "dx", "dbias")]),
           "oracle_router_bwd")
    return {n: v for n, v in res.items() if v is not None}


_u8p = ctypes.POINTER(ctypes.c_uint8)


def mx_scale_cols(K: int) -> int:
    """Scale bytes per row of an MX-FP8 matrix with K columns: 4 * ceil(K / 128)."""
    return 4 * ((K + 127) // 128)


def quantize_mxfp8(src):
    """MX-FP8 quantization of src [..., K] (values as float32, K a multiple of 32) along its
    last dimension: returns (codes uint8 [..., K], scale codes uint8 [..., 4 ceil(K/128)])."""
    src = _f32(src)
    K = src.shape[-1]
    rows = int(np.prod(src.shape[:-1])) if src.ndim > 1 else 1
    q = np.empty(src.shape, np.uint8)
    s = np.empty(src.shape[:-1] + (mx_scale_cols(K),), np.uint8)
    _check(_lib().oracle_quantize_mxfp8(_p(src, _f32p), rows, K, _p(q, _u8p), _p(s, _u8p)), "oracle_quantize_mxfp8")
    return q, s


def layer_fwd_mxfp8(x, wg, wu, wd, pair_t, pair_e, pair_w, want_stages=False, real="f64"):
    """Layer forward on MX-FP8 operands: x, wg, wu, wd are (codes, scale codes) pairs as from
    quantize_mxfp8 of x [N,H], W_gate / W_up [E,I,H] and W_down [E,H,I].  Returns out [N,H]
    (float64) and, with want_stages, a dict with gu [P,2I] (float64), aq [P,I] and as [P,KS(I)]
    (the quantized activation of every pair)."""
    (xq, xs), (gq, gs), (uq, us), (dq, ds) = x, wg, wu, wd
    N, H = xq.shape
    E, I, _ = gq.shape
    pair_t, pair_e, pair_w = _i32(pair_t), _i32(pair_e), _f32(pair_w)
    P = len(pair_t)
    c = lambda a: np.ascontiguousarray(a, np.uint8)  # noqa: E731
    xq, xs, gq, gs, uq, us, dq, ds = map(c, (xq, xs, gq, gs, uq, us, dq, ds))
    out = np.empty((N, H), np.float64)
    st = None
    if want_stages:
        st = {"gu": np.empty((P, 2 * I), np.float64), "aq": np.empty((P, I), np.uint8),
              "as": np.empty((P, mx_scale_cols(I)), np.uint8)}
    _check(_lib(real).oracle_layer_fwd_mxfp8(
        _p(xq, _u8p), _p(xs, _u8p), _p(gq, _u8p), _p(gs, _u8p), _p(uq, _u8p), _p(us, _u8p), _p(dq, _u8p),
        _p(ds, _u8p), N, H, I, E, P, _p(pair_t, _i32p), _p(pair_e, _i32p), _p(pair_w, _f32p), _p(out, _f64p),
        None if st is None else _p(st["gu"], _f64p), None if st is None else _p(st["aq"], _u8p),
        None if st is None else _p(st["as"], _u8p)), "oracle_layer_fwd_mxfp8")
    return (out, st) if want_stages else out



def dx_weights_mxfp8(wg, wu):
    """The dX product's weight operand: for each expert e, [W_gate[e]^T | W_up[e]^T] ([H, 2I]:
    row h holds W_gate[e][i][h] for i < I, then W_up[e][i][h]) quantized along its rows ->
    (codes uint8 [E, H, 2I], scale codes uint8 [E, H, 4 ceil(2I/128)])."""
    wt = np.concatenate([np.swapaxes(_f32(wg), 1, 2), np.swapaxes(_f32(wu), 1, 2)], axis=2)
    return quantize_mxfp8(np.ascontiguousarray(wt))


def dx_mxfp8(dh, wt, pair_t, pair_e, N, want_codes=False, real="f64"):
    """dx [N,H] (float64) of the dX product on MX-FP8 operands: each pair's dh row [2I] (fp32
    values) quantized, times its expert's quantized [W_gate^T | W_up^T] rows (wt = (codes,
    scale codes) from dx_weights_mxfp8), summed per token.  With want_codes also the
    quantized dh rows (codes [P, 2I], scale codes [P, KS(2I)])."""
    wq, ws = (np.ascontiguousarray(a, np.uint8) for a in wt)
    E, H, K = wq.shape
    I = K // 2
    dh = _f32(dh)
    pair_t, pair_e = _i32(pair_t), _i32(pair_e)
    P = len(pair_t)
    dx = np.empty((N, H), np.float64)
    q = np.empty((P, K), np.uint8) if want_codes else None
    s = np.empty((P, mx_scale_cols(K)), np.uint8) if want_codes else None
    _check(_lib(real).oracle_dx_mxfp8(_p(dh, _f32p), _p(wq, _u8p), _p(ws, _u8p), N, H, I, E, P, _p(pair_t, _i32p),
                                      _p(pair_e, _i32p), _p(dx, _f64p), None if q is None else _p(q, _u8p),
                                      None if s is None else _p(s, _u8p)), "oracle_dx_mxfp8")
    return (dx, q, s) if want_codes else dx
