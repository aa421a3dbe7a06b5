"""MI355X-native dropless MoE expert-MLP layer: thin Python binding over libmoe.so.

Every function here only marshals arguments (torch device tensors -> raw pointers and
sizes) into the C ABI declared in ``include/moe.h``; all computation runs in the HIP
kernels of ``libmoe.so``.  There is no fallback: if the library is missing or a call fails,
an exception is raised.  PyTorch supplies device memory and the current stream only.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MoEError", "lib", "lib_path", "load_library", "Plan", "route_topk", "permute", "permute_noalloc",
    "route_token_rounding", "quantize_mxfp8", "grouped_gemm_fwd_mxfp8", "mx_scale_cols", "OP_GEMM_FWD_MXFP8",
    "quantize_dx_weights_mxfp8", "layer_bwd_mxfp8", "OP_LAYER_BWD_MXFP8",
    "route_capacity", "grouped_gemm_fwd", "unpermute_combine", "layer_bwd", "router_logits", "router_bwd",
    "workspace_bytes", "plan_rows_cap", "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE",
    "MOE_EHIP", "OP_PERMUTE", "OP_ROUTE_TR", "OP_GEMM_FWD", "OP_LAYER_BWD", "OP_ROUTER_BWD",
    "OP_ROUTER_LOGITS", "PLAN_TOPK", "PLAN_TR", "PLAN_CAP", "CAP_POSITION", "CAP_PROBS",
    "EXPORTED_SYMBOLS", "KERNEL_IDS", "set_kernel_events",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16 = 0, 1
PLAN_TOPK, PLAN_TR, PLAN_CAP = 0, 1, 2
CAP_POSITION, CAP_PROBS = 0, 1
OP_PERMUTE, OP_ROUTE_TR, OP_GEMM_FWD, OP_LAYER_BWD, OP_ROUTER_BWD, OP_ROUTER_LOGITS = 0, 1, 2, 3, 4, 5
OP_GEMM_FWD_MXFP8 = 6
OP_LAYER_BWD_MXFP8 = 7

EXPORTED_SYMBOLS = (
    "moe_plan_rows_cap", "moe_workspace_bytes", "moe_last_error", "moe_route_topk", "moe_permute",
    "moe_permute_noalloc",
    "moe_route_token_rounding", "moe_route_capacity", "moe_grouped_gemm_fwd", "moe_unpermute_combine",
    "moe_layer_bwd",
    "moe_router_logits", "moe_router_bwd", "moe_set_kernel_events", "moe_quantize_mxfp8",
    "moe_grouped_gemm_fwd_mxfp8", "moe_quantize_dx_weights_mxfp8", "moe_layer_bwd_mxfp8",
)

# kernel ids of the measurement hook (moe_kernel_id in include/moe.h)
KERNEL_IDS = {"gateup": 0, "down": 1, "dh": 2, "dx": 3, "dwd": 4, "dw1": 5, "combine": 6, "dx_combine": 7,
              "route": 8, "permute": 9, "route_tr_plan": 10, "dswiglu": 11, "router_logits": 12,
              "router_dz": 13, "router_dx": 14, "router_dw": 15, "gateup_fp8": 16, "down_fp8": 17, "quant": 18,
              "dx_fp8": 19}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    """The in-tree libmoe.so (built by ``grouped_gemm_top_amd.build``)."""
    return os.path.join(_HERE, "libmoe.so")


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


class CPlan(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("N", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("M_cap", ctypes.c_int32), ("mtile", ctypes.c_int32),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("row_token", ctypes.c_void_p), ("row_w", ctypes.c_void_p),
                ("row_pair", ctypes.c_void_p), ("tok_ptr", ctypes.c_void_p),
                ("tok_rows", ctypes.c_void_p)]


def lib():
    """Load libmoe.so (built by ``grouped_gemm_top_amd.build``); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m grouped_gemm_top_amd.build` "
                           "(there is no fallback path)")
    _LIB = load_library(path)
    return _LIB


def load_library(path: str):
    """ctypes handle of a build of libmoe.so at `path` with every entry point's signature set
    (lib() uses it for the in-tree library; the host-sanitizer tests for their own build)."""
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pp = ctypes.POINTER(CPlan)
    L.moe_plan_rows_cap.argtypes = [i32, i32, i32, i32, i32]
    L.moe_plan_rows_cap.restype = ctypes.c_int64
    L.moe_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, i32, i32, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_route_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.moe_permute.argtypes = [vp, vp, i32, i32, i32, pp, vp, sz, vp]
    L.moe_permute_noalloc.argtypes = [vp, vp, i32, i32, i32, pp, vp]
    L.moe_route_token_rounding.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, pp, vp, sz, vp]
    L.moe_route_capacity.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, pp, vp, sz, vp]
    L.moe_grouped_gemm_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, i32, i32, pp, vp, vp, vp, sz, vp]
    L.moe_unpermute_combine.argtypes = [ctypes.c_int, vp, i32, pp, vp, vp, vp]
    L.moe_layer_bwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, pp, vp, vp, vp, vp, vp, vp,
                                vp, sz, vp]
    L.moe_router_logits.argtypes = [ctypes.c_int, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    L.moe_router_bwd.argtypes = [ctypes.c_int, vp, vp, vp, pp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_set_kernel_events.argtypes = [i32, vp, vp]
    L.moe_quantize_mxfp8.argtypes = [ctypes.c_int, vp, ctypes.c_int64, i32, vp, vp, vp]
    L.moe_grouped_gemm_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, pp, vp, vp, vp, sz, vp]
    L.moe_quantize_dx_weights_mxfp8.argtypes = [ctypes.c_int, vp, vp, i32, i32, i32, vp, vp, vp]
    L.moe_layer_bwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, pp, vp, vp, vp, vp, vp, vp, vp, sz,
                                      vp]
    for fn in ("moe_route_topk", "moe_permute", "moe_permute_noalloc", "moe_route_token_rounding",
               "moe_route_capacity",
               "moe_grouped_gemm_fwd",
               "moe_unpermute_combine", "moe_layer_bwd", "moe_router_logits", "moe_router_bwd",
               "moe_set_kernel_events", "moe_quantize_mxfp8", "moe_grouped_gemm_fwd_mxfp8",
               "moe_quantize_dx_weights_mxfp8", "moe_layer_bwd_mxfp8"):
        getattr(L, fn).restype = ctypes.c_int
    return L


def _check(st: int):
    if st != MOE_OK:
        raise MoEError(st, lib().moe_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def set_kernel_events(name: str, start=None, stop=None):
    """Register torch.cuda.Event objects (enable_timing=True) to be recorded around every
    later launch of the named kernel on its launch stream; None switches it off."""
    h = (lambda ev: None if ev is None else ctypes.c_void_p(ev.cuda_event))
    _check(lib().moe_set_kernel_events(KERNEL_IDS[name], h(start), h(stop)))


def plan_rows_cap(kind: int, N: int, E: int, k: int, mtile: int = 0) -> int:
    v = lib().moe_plan_rows_cap(kind, N, E, k, mtile)
    if v < 0:
        raise MoEError(MOE_EINVAL, "invalid plan dimensions")
    return int(v)


def workspace_bytes(op: int, dtype_code: int, N: int, E: int, k: int, H: int = 8, I: int = 8,
                    M_cap: int = 0) -> int:
    v = lib().moe_workspace_bytes(op, dtype_code, N, E, k, H, I, M_cap)
    if v == 0:
        raise MoEError(MOE_EINVAL, "invalid workspace query")
    return int(v)


class Plan:
    """Device arrays of a routing plan (see moe_plan in include/moe.h), allocated with torch."""

    def __init__(self, N: int, E: int, k: int, kind: int = PLAN_TOPK, mtile: int = 0, device="cuda",
                 alloc=None):
        """alloc(name, numel, dtype) -> 1-D device tensor, if given, supplies the arrays
        (default: torch.empty on `device`)."""
        import torch
        self.N, self.E, self.k, self.kind = N, E, k, kind
        self.mtile = mtile if kind in (PLAN_TR, PLAN_CAP) else 0  # capacity plans: the capacity
        self.M_cap = plan_rows_cap(kind, N, E, k, self.mtile)
        if alloc is None:
            alloc = lambda name, n, dt: torch.empty(n, dtype=dt, device=device)  # noqa: E731
        i32 = torch.int32
        mc = max(self.M_cap, 1)
        self.counts = alloc("counts", E, i32)
        self.offsets = alloc("offsets", E + 1, i32)
        self.row_token = alloc("row_token", mc, i32)
        self.row_w = alloc("row_w", mc, torch.float32)
        self.row_pair = alloc("row_pair", mc, i32)
        self.tok_ptr = alloc("tok_ptr", N + 1, i32)
        self.tok_rows = alloc("tok_rows", mc, i32)
        self._c = CPlan(kind, N, E, k, self.M_cap, self.mtile, *(t.data_ptr() for t in (
            self.counts, self.offsets, self.row_token, self.row_w, self.row_pair, self.tok_ptr,
            self.tok_rows)))

    @property
    def c(self):
        return ctypes.byref(self._c)

    def host(self) -> dict:
        """Copy the plan to host numpy arrays, trimmed to the rows in use."""
        off = self.offsets.cpu().numpy()
        m = int(off[-1])
        return dict(counts=self.counts.cpu().numpy(), offsets=off,
                    row_token=self.row_token[:m].cpu().numpy(), row_w=self.row_w[:m].cpu().numpy(),
                    row_pair=self.row_pair[:m].cpu().numpy(), tok_ptr=self.tok_ptr.cpu().numpy(),
                    tok_rows=self.tok_rows[:m].cpu().numpy())


def _ws(nbytes: int, device, ws=None):
    import torch
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise MoEError(MOE_EWORKSPACE, f"workspace holds {ws.numel() * ws.element_size()} < {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def route_topk(logits, k: int, bias=None, want_probs: bool = False, idx=None, w=None, probs=None,
               stream=None):
    """-> (topk_idx int32 [N,k], topk_w fp32 [N,k], probs fp32 [N,E] or None)."""
    import torch
    N, E = logits.shape
    idx = idx if idx is not None else torch.empty((N, k), dtype=torch.int32, device=logits.device)
    w = w if w is not None else torch.empty((N, k), dtype=torch.float32, device=logits.device)
    if probs is None and want_probs:
        probs = torch.empty((N, E), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_ptr(logits), _ptr(bias), N, E, k, _ptr(idx), _ptr(w), _ptr(probs),
                                _stream(stream)))
    return idx, w, probs


def permute(topk_idx, topk_w, E: int, plan: Plan | None = None, ws=None, stream=None) -> Plan:
    N, k = topk_idx.shape
    plan = plan or Plan(N, E, k, device=topk_idx.device)
    nb = workspace_bytes(OP_PERMUTE, MOE_BF16, N, E, k)
    ws = _ws(nb, topk_idx.device, ws)
    _check(lib().moe_permute(_ptr(topk_idx), _ptr(topk_w), N, E, k, plan.c, _ptr(ws), nb, _stream(stream)))
    return plan


def permute_noalloc(topk_idx, topk_w, E: int, plan: Plan, stream=None) -> Plan:
    """moe_permute_noalloc: the permute with the library's fixed scratch instead of a
    workspace; `plan` (caller-allocated) is required, so this call allocates nothing."""
    N, k = topk_idx.shape
    _check(lib().moe_permute_noalloc(_ptr(topk_idx), _ptr(topk_w), N, E, k, plan.c, _stream(stream)))
    return plan


def route_token_rounding(logits, k: int, mtile: int, bias=None, plan: Plan | None = None, ws=None,
                         idx=None, w=None, probs=None, stream=None):
    """-> (plan, topk_idx, topk_w, probs)."""
    import torch
    N, E = logits.shape
    dev = logits.device
    plan = plan or Plan(N, E, k, kind=PLAN_TR, mtile=mtile, device=dev)
    idx = idx if idx is not None else torch.empty((N, k), dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty((N, k), dtype=torch.float32, device=dev)
    probs = probs if probs is not None else torch.empty((N, E), dtype=torch.float32, device=dev)
    nb = workspace_bytes(OP_ROUTE_TR, MOE_BF16, N, E, k)
    ws = _ws(nb, dev, ws)
    _check(lib().moe_route_token_rounding(_ptr(logits), _ptr(bias), N, E, k, mtile, _ptr(idx), _ptr(w),
                                          _ptr(probs), plan.c, _ptr(ws), nb, _stream(stream)))
    return plan, idx, w, probs


def route_capacity(logits, k: int, capacity: int, policy: int = CAP_POSITION, bias=None, plan: Plan | None = None,
                   ws=None, idx=None, w=None, probs=None, stream=None):
    """-> (plan, topk_idx, topk_w, probs): top-k routing, then each expert keeps at most
    `capacity` of its tokens (policy CAP_POSITION: token order; CAP_PROBS: largest P first)."""
    import torch
    N, E = logits.shape
    dev = logits.device
    plan = plan or Plan(N, E, k, kind=PLAN_CAP, mtile=capacity, device=dev)
    idx = idx if idx is not None else torch.empty((N, k), dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty((N, k), dtype=torch.float32, device=dev)
    probs = probs if probs is not None else torch.empty((N, E), dtype=torch.float32, device=dev)
    nb = workspace_bytes(OP_ROUTE_TR, MOE_BF16, N, E, k)
    ws = _ws(nb, dev, ws)
    _check(lib().moe_route_capacity(_ptr(logits), _ptr(bias), N, E, k, capacity, policy, _ptr(idx), _ptr(w),
                                    _ptr(probs), plan.c, _ptr(ws), nb, _stream(stream)))
    return plan, idx, w, probs


def grouped_gemm_fwd(x, w_gate, w_up, w_down, plan: Plan, hcache=None, y=None, ws=None, stream=None):
    """-> (hcache [M_cap, 2I], y [M_cap, H])."""
    import torch
    N, H = x.shape
    E, I, _ = w_gate.shape
    dt = _dtype_code(x)
    mc = max(plan.M_cap, 1)
    hcache = hcache if hcache is not None else torch.empty((mc, 2 * I), dtype=x.dtype, device=x.device)
    y = y if y is not None else torch.empty((mc, H), dtype=x.dtype, device=x.device)
    nb = workspace_bytes(OP_GEMM_FWD, dt, plan.N, plan.E, plan.k, H, I, plan.M_cap)
    ws = _ws(nb, x.device, ws)
    _check(lib().moe_grouped_gemm_fwd(dt, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), H, I, plan.c,
                                      _ptr(hcache), _ptr(y), _ptr(ws), nb, _stream(stream)))
    return hcache, y


def mx_scale_cols(K: int) -> int:
    """Scale codes per row of an MX-FP8 matrix with K columns: 4 * ceil(K / 128)."""
    return 4 * ((K + 127) // 128)


def quantize_mxfp8(src, q=None, scales=None, stream=None):
    """MX-FP8 quantization of src [..., K] (bf16 or fp32, K a multiple of 32) along its last
    dimension -> (codes uint8 [..., K], scale codes uint8 [..., 4 ceil(K/128)])."""
    import torch
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    q = q if q is not None else torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    scales = scales if scales is not None else torch.empty(src.shape[:-1] + (mx_scale_cols(K),), dtype=torch.uint8,
                                                           device=src.device)
    _check(lib().moe_quantize_mxfp8(_dtype_code(src), _ptr(src), rows, K, _ptr(q), _ptr(scales), _stream(stream)))
    return q, scales


def grouped_gemm_fwd_mxfp8(x, w_gate, w_up, w_down, plan: Plan, hcache=None, y=None, ws=None, stream=None):
    """Forward on MX-FP8 operands; x, w_gate, w_up, w_down are (codes, scale codes) pairs from
    quantize_mxfp8 of x [N,H], W_gate / W_up [E,I,H] and W_down [E,H,I].  -> (hcache [M_cap, 2I],
    y [M_cap, H]), both bf16."""
    import torch
    (xq, xs), (gq, gs), (uq, us), (dq, dsc) = x, w_gate, w_up, w_down
    N, H = xq.shape
    E, I, _ = gq.shape
    mc = max(plan.M_cap, 1)
    hcache = hcache if hcache is not None else torch.empty((mc, 2 * I), dtype=torch.bfloat16, device=xq.device)
    y = y if y is not None else torch.empty((mc, H), dtype=torch.bfloat16, device=xq.device)
    nb = workspace_bytes(OP_GEMM_FWD_MXFP8, MOE_BF16, plan.N, plan.E, plan.k, H, I, plan.M_cap)
    ws = _ws(nb, xq.device, ws)
    _check(lib().moe_grouped_gemm_fwd_mxfp8(_ptr(xq), _ptr(xs), _ptr(gq), _ptr(gs), _ptr(uq), _ptr(us), _ptr(dq),
                                            _ptr(dsc), H, I, plan.c, _ptr(hcache), _ptr(y), _ptr(ws), nb,
                                            _stream(stream)))
    return hcache, y


def unpermute_combine(y, plan: Plan, row_w="plan", out=None, stream=None):  # noqa: D401
    """out [N,H] = per-token sum of row_w[r] * y[r] (row_w: 'plan' for the plan's weights,
    None for weights 1, or an fp32 tensor [M_cap])."""
    import torch
    H = y.shape[1]
    dt = _dtype_code(y)
    out = out if out is not None else torch.empty((plan.N, H), dtype=y.dtype, device=y.device)
    rw = plan.row_w if isinstance(row_w, str) else row_w
    _check(lib().moe_unpermute_combine(dt, _ptr(y), H, plan.c, _ptr(rw), _ptr(out), _stream(stream)))
    return out


def layer_bwd(dout, x, w_gate, w_up, w_down, plan: Plan, hcache, dx=None, dw_gate=None, dw_up=None,
              dw_down=None, ds=None, ws=None, stream=None):
    """-> dict(dx, dw_gate, dw_up, dw_down, ds).  ds is [N,k] for top-k plans, [M_cap] for
    token-rounding plans."""
    import torch
    N, H = x.shape
    E, I, _ = w_gate.shape
    dt = _dtype_code(x)
    dev = x.device
    dx = dx if dx is not None else torch.empty_like(x)
    dw_gate = dw_gate if dw_gate is not None else torch.empty_like(w_gate)
    dw_up = dw_up if dw_up is not None else torch.empty_like(w_up)
    dw_down = dw_down if dw_down is not None else torch.empty_like(w_down)
    if ds is None:
        shape = (N, plan.k) if plan.kind == PLAN_TOPK else (max(plan.M_cap, 1),)
        ds = torch.empty(shape, dtype=torch.float32, device=dev)
    nb = workspace_bytes(OP_LAYER_BWD, dt, plan.N, plan.E, plan.k, H, I, plan.M_cap)
    ws = _ws(nb, dev, ws)
    _check(lib().moe_layer_bwd(dt, _ptr(dout), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), H, I, plan.c,
                               _ptr(hcache), _ptr(dx), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(ds),
                               _ptr(ws), nb, _stream(stream)))
    return dict(dx=dx, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down, ds=ds)


def quantize_dx_weights_mxfp8(w_gate, w_up, q=None, scales=None, stream=None):
    """The dX product's MX-FP8 weight operand: each expert's [W_gate^T | W_up^T] ([H, 2I])
    quantized along 2I -> (codes uint8 [E, H, 2I], scale codes uint8 [E, H, 4 ceil(2I/128)])."""
    import torch
    E, I, H = w_gate.shape
    q = q if q is not None else torch.empty((E, H, 2 * I), dtype=torch.uint8, device=w_gate.device)
    scales = scales if scales is not None else torch.empty((E, H, mx_scale_cols(2 * I)), dtype=torch.uint8,
                                                           device=w_gate.device)
    _check(lib().moe_quantize_dx_weights_mxfp8(_dtype_code(w_gate), _ptr(w_gate), _ptr(w_up), E, H, I, _ptr(q),
                                               _ptr(scales), _stream(stream)))
    return q, scales


def layer_bwd_mxfp8(dout, x, w_gate, w_up, w_down, wt, plan: Plan, hcache, dx=None, dw_gate=None, dw_up=None,
                    dw_down=None, ds=None, ws=None, stream=None):
    """layer_bwd for bf16 layers with the dX product on MX-FP8 operands; wt = (codes, scale
    codes) from quantize_dx_weights_mxfp8.  -> dict(dx, dw_gate, dw_up, dw_down, ds)."""
    import torch
    N, H = x.shape
    E, I, _ = w_gate.shape
    wq, wsc = wt
    dev = x.device
    dx = dx if dx is not None else torch.empty_like(x)
    dw_gate = dw_gate if dw_gate is not None else torch.empty_like(w_gate)
    dw_up = dw_up if dw_up is not None else torch.empty_like(w_up)
    dw_down = dw_down if dw_down is not None else torch.empty_like(w_down)
    if ds is None:
        shape = (N, plan.k) if plan.kind == PLAN_TOPK else (max(plan.M_cap, 1),)
        ds = torch.empty(shape, dtype=torch.float32, device=dev)
    nb = workspace_bytes(OP_LAYER_BWD_MXFP8, MOE_BF16, plan.N, plan.E, plan.k, H, I, plan.M_cap)
    ws = _ws(nb, dev, ws)
    _check(lib().moe_layer_bwd_mxfp8(_ptr(dout), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wq),
                                     _ptr(wsc), H, I, plan.c, _ptr(hcache), _ptr(dx), _ptr(dw_gate), _ptr(dw_up),
                                     _ptr(dw_down), _ptr(ds), _ptr(ws), nb, _stream(stream)))
    return dict(dx=dx, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down, ds=ds)


def router_logits(x, w_r, bias=None, logits=None, ws=None, stream=None):
    """logits [N,E] fp32 = x @ w_r (+ bias); x [N,H] (bf16 or fp32), w_r fp32 [H,E]."""
    import torch
    N, H = x.shape
    E = w_r.shape[1]
    dt = _dtype_code(x)
    logits = logits if logits is not None else torch.empty((N, E), dtype=torch.float32, device=x.device)
    nb = workspace_bytes(OP_ROUTER_LOGITS, dt, N, E, 1, H, 8, 0)
    ws = _ws(nb, x.device, ws)
    _check(lib().moe_router_logits(dt, _ptr(x), _ptr(w_r), _ptr(bias), N, H, E, _ptr(logits), _ptr(ws), nb,
                                   _stream(stream)))
    return logits


def router_bwd(logits, topk_idx, plan: Plan, ds, x, w_r, bias=None, dx_in=None, dx_out=None, dlogits=None,
               dw_r=None, dbias=None, want_dx=True, want_dw=True, want_dbias=True, ws=None, stream=None):
    """Router backward from dS (moe_layer_bwd's ds) -> dict(dlogits, dx, dw_r, dbias).
    dx = dx_in + the router's share (dx_in defaults to zeros; dx_out may be dx_in)."""
    import torch
    N, H = x.shape
    E = logits.shape[1]
    dt = _dtype_code(x)
    dev = x.device
    dlogits = dlogits if dlogits is not None else torch.empty((N, E), dtype=torch.float32, device=dev)
    if want_dx:
        dx_in = dx_in if dx_in is not None else torch.zeros_like(x)
        dx_out = dx_out if dx_out is not None else torch.empty_like(x)
    else:
        dx_in = dx_out = None
    if want_dw:
        dw_r = dw_r if dw_r is not None else torch.empty((H, E), dtype=torch.float32, device=dev)
    else:
        dw_r = None
    if want_dbias:
        dbias = dbias if dbias is not None else torch.empty((E,), dtype=torch.float32, device=dev)
    else:
        dbias = None
    nb = workspace_bytes(OP_ROUTER_BWD, dt, plan.N, plan.E, plan.k, H, 8, 0) if (want_dx or want_dw or want_dbias) \
        else 0
    ws = _ws(nb, dev, ws) if nb else None
    _check(lib().moe_router_bwd(dt, _ptr(logits), _ptr(bias), _ptr(topk_idx), plan.c, _ptr(ds), _ptr(x), _ptr(w_r),
                                H, _ptr(dx_in), _ptr(dx_out), _ptr(dlogits), _ptr(dw_r), _ptr(dbias), _ptr(ws), nb,
                                _stream(stream)))
    return dict(dlogits=dlogits, dx=dx_out, dw_r=dw_r, dbias=dbias)
