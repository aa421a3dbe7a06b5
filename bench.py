#!/usr/bin/env python3
"""Benchmark of the MoE expert-MLP layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, through the C ABI:
router top-k -> permute (counts, offsets, row lists) -> grouped GEMM forward (gate/up +
SwiGLU, down) -> weighted combine -> layer backward (dH/dS/A', dW_down, dX + combine,
dW_gate/dW_up).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  `value` is the layer throughput in TFLOPS (18*M*H*I algorithmic
FLOPs per fwd+bwd step over the wall time of the timed steps, which run without any
measurement hook).  Per-kernel durations come from a second run of the same number of steps,
with HIP events recorded by the library around each launch on its launch stream.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd ms & TFLOPS (% bf16 MFMA peak), E=128 H=2048 I=512 k=8 N=4096"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2      # dense fp8 MFMA: twice the bf16 rate
GEMMS = ("gateup", "down", "dh", "dx", "dwd", "dw1")
ALL_KERNELS = ("route", "permute", "route_tr_plan", "gateup", "down", "combine", "dh", "dwd", "dx",
               "dx_combine", "dw1")


def kernel_work(name, wl, M, e_act, es):
    """Algorithmic (flops, bytes) of one launch: each tensor touched once, gathered rows
    counted once (served from cache), weights of the active experts read once, dW written
    for every expert."""
    N, H, I, E = wl.N, wl.H, wl.I, wl.E
    if name == "gateup":
        return 4.0 * M * H * I, es * (2.0 * e_act * I * H + N * H + 3.0 * M * I)
    if name == "down":
        return 2.0 * M * H * I, es * (1.0 * e_act * H * I + M * I + M * H)
    # dS partials per row of the dH kernel's dSwiGLU epilogue
    n_part = 2 * ((I + 255) // 256) if es == 2 else (I + 127) // 128
    if name == "dh":  # reads W_down, dOut rows, G, U, w; writes dG, dU, A' and the dS partials
        return 2.0 * M * H * I, es * (1.0 * e_act * H * I + N * H + 5.0 * M * I) + 4.0 * M * (n_part + 1)
    if name == "dx":
        return 4.0 * M * H * I, es * (2.0 * e_act * I * H + 2.0 * M * I + M * H)
    if name == "dwd":
        return 2.0 * M * H * I, es * (1.0 * E * H * I + N * H + M * I)
    if name == "dw1":
        return 4.0 * M * H * I, es * (2.0 * E * I * H + N * H + 2.0 * M * I)
    if name == "combine":
        return 2.0 * M * H, es * (1.0 * M * H + N * H) + 8.0 * M
    if name == "dx_combine":  # also the ordered sum of the dS partials
        return 2.0 * M * H, es * (1.0 * M * H + N * H) + 8.0 * M + 4.0 * M * n_part + 8.0 * M
    return 0.0, 0.0


def layer_bytes(wl, M, e_act, es):
    """Algorithmic HBM bytes of one forward + backward step: weights of the active experts read
    in the forward and the backward, dW written for every expert, x, out, dOut and dX once,
    hcache, A, dH and A' traffic (14 M I) and Y and dXe each written and read (4 M H)."""
    N, H, I, E = wl.N, wl.H, wl.I, wl.E
    return float(es) * ((6.0 * e_act + 3.0 * E) * H * I + 4.0 * N * H + 14.0 * M * I + 4.0 * M * H)


def load_traffic(name, workload):
    """HBM bytes per launch of kernel `name`, from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    summarised in profiles/traffic_<workload>.txt.  Returned only while the kernel's source files
    (comma-separated, hashed in order) still hash to the value recorded beside the counters;
    otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in kv.get(f"{name}.source", "gemm.hip").split(","):
        src = os.path.join(ROOT, "grouped_gemm_top_amd", "csrc", f.strip())
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if kv.get(f"{name}.source_sha") != h.hexdigest()[:16]:
        return None
    try:
        return float(kv[f"{name}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_facts():
    """The host the CPU baseline ran on: CPU model, logical CPUs, CPUs this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_available": len(os.sched_getaffinity(0))}


def cpu_baseline(T, pt, pe, pw, what, single_tokens):
    """The fp32 oracle as it stands (plain C loops, -O3, OpenMP over the host's threads), the
    layer forward then backward (out, dx, dW_gate, dW_up, dW_down, dS) on the given pairs;
    then the same on one thread for the pairs of the first `single_tokens` tokens."""
    import oracle
    wl = T.wl
    thr = oracle.threads("f32")
    t0 = time.perf_counter()
    oracle.layer_fwd(T.x, T.wg, T.wu, T.wd, pt, pe, pw, real="f32")
    t1 = time.perf_counter()
    oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt, pe, pw, real="f32")
    t2 = time.perf_counter()
    flops = 18.0 * len(pt) * wl.H * wl.I
    keep = pt < single_tokens
    oracle.set_threads(1, "f32")
    try:
        s0 = time.perf_counter()
        oracle.layer_fwd(T.x, T.wg, T.wu, T.wd, pt[keep], pe[keep], pw[keep], real="f32")
        oracle.layer_bwd(T.dout, T.x, T.wg, T.wu, T.wd, pt[keep], pe[keep], pw[keep], real="f32")
        s1 = time.perf_counter()
    finally:
        oracle.set_threads(thr, "f32")
    sflops = 18.0 * int(keep.sum()) * wl.H * wl.I
    res = {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOPS", "cores": thr, "kind": "oracle",
           "sample": f"fp32 oracle forward + backward on {what} ({len(pt)} (token, expert) pairs); "
                     f"{t2 - t0:.1f} s on {thr} threads; TFLOPS = 18*pairs*H*I / time",
           "fwd_s": round(t1 - t0, 3), "bwd_s": round(t2 - t1, 3), "layer_ms": round((t2 - t0) * 1e3, 1),
           "single_thread": {"pairs": int(keep.sum()), "tokens": single_tokens, "seconds": round(s1 - s0, 3),
                             "tflops": sflops / (s1 - s0) / 1e12 if s1 > s0 else None}}
    res.update(host_facts())
    return res


def padded_fractions(counts, M):
    """MFMA rows computed beyond the real rows, as a fraction of M, for the kernels' own
    granules: varlen-M tiles skip 16-row blocks that start past a group's rows (so a group of
    c rows costs 16*ceil(c/16)); varlen-K tiles run k-steps of 32 rows (32*ceil(c/32))."""
    c = np.asarray(counts, np.int64)
    m = max(int(M), 1)
    return {"varlen_m_16row_blocks": round(float((16 * ((c + 15) // 16)).sum()) / m - 1.0, 5),
            "varlen_k_32row_steps": round(float((32 * ((c + 31) // 32)).sum()) / m - 1.0, 5),
            "fixed_128row_tiles": round(float((128 * ((c + 127) // 128)).sum()) / m - 1.0, 5)}


def fp8_forward(args, wl, x, wg, wu, wd, plan, M, e_act, kern_ms):
    """The MX-FP8 forward on the same plan: the weights quantized once (timed on their own, a
    cost the caller pays once per weight update), then per step x quantized and the gate/up and
    down GEMMs on fp8 operands, each kernel timed with HIP events on its launch stream."""
    import torch
    import grouped_gemm_top_amd as G
    N, H, I, E = wl.N, wl.H, wl.I, wl.E
    qw = [G.quantize_mxfp8(t) for t in (wg, wu, wd)]
    xq = G.quantize_mxfp8(x)
    mc = max(plan.M_cap, 1)
    hc8 = torch.empty((mc, 2 * I), dtype=torch.bfloat16, device="cuda")
    y8 = torch.empty((mc, H), dtype=torch.bfloat16, device="cuda")
    ws8 = torch.empty(G.workspace_bytes(G.OP_GEMM_FWD_MXFP8, G.MOE_BF16, N, E, wl.k, H, I, plan.M_cap),
                      dtype=torch.uint8, device="cuda")
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_.record()
    for t, q in zip((wg, wu, wd), qw):
        G.quantize_mxfp8(t, q=q[0], scales=q[1])
    b_.record()
    torch.cuda.synchronize()
    wq_ms = a_.elapsed_time(b_)

    def step8():
        G.quantize_mxfp8(x, q=xq[0], scales=xq[1])
        G.grouped_gemm_fwd_mxfp8(xq, qw[0], qw[1], qw[2], plan, hcache=hc8, y=y8, ws=ws8)

    for _ in range(args.warmup):
        step8()
    names = ("quant", "gateup_fp8", "down_fp8")
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for n in names}
    for pairs in evs.values():
        for e0, e1 in pairs:
            e0.record()
            e1.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        for n in names:
            G.set_kernel_events(n, *evs[n][i])
        step8()
    torch.cuda.synchronize()
    for n in names:
        G.set_kernel_events(n, None, None)
    us = {n: 1e3 * float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[n]])) for n in names}
    f_gu, f_dn = 4.0 * M * H * I, 2.0 * M * H * I
    sc = 1.0 + 1.0 / 32  # codes plus one scale byte per 32
    b_gu = 2.0 * e_act * I * H * sc + N * H * sc + 2.0 * M * 2 * I + M * I * sc
    b_dn = e_act * H * I * sc + M * I * sc + 2.0 * M * H
    gemm_us = us["gateup_fp8"] + us["down_fp8"]
    bf16_us = 1e3 * (kern_ms["gateup"] + kern_ms["down"])
    out = {"note": "MX-FP8 forward (e4m3, one power-of-two scale per 32 values along K) on the bf16 run's plan; "
                   "weights quantized once, x every step",
           "kernels_us": {n: round(v, 2) for n, v in us.items()},
           "weights_quant_ms": round(wq_ms, 3),
           "fwd_gemms_us": round(gemm_us, 2), "bf16_fwd_gemms_us": round(bf16_us, 2),
           "speedup_vs_bf16_gemms": round(bf16_us / gemm_us, 3),
           "fwd_gemm_tflops": round((f_gu + f_dn) / (gemm_us * 1e-6) / 1e12, 1),
           "pct_fp8_peak": round(100.0 * (f_gu + f_dn) / (gemm_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 2)}
    dom = "gateup_fp8" if us["gateup_fp8"] >= us["down_fp8"] else "down_fp8"
    f, b = (f_gu, b_gu) if dom == "gateup_fp8" else (f_dn, b_dn)
    t_s = us[dom] * 1e-6
    if b / (PEAK_HBM_GBS * 1e9) >= f / (PEAK_FP8_TFLOPS * 1e12):
        out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": round(b / t_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(b / t_s / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
                           "algorithmic_bytes": b, "us": round(us[dom], 2)}
    else:
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(f / t_s / 1e12, 1),
                           "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(f / t_s / 1e12 / PEAK_FP8_TFLOPS, 4),
                           "traffic": None, "algorithmic_flops": f, "us": round(us[dom], 2)}
    return out


def fp8_backward_dx(args, wl, x, wg, wu, wd, dout, plan, hcache, M, e_act, kern_ms):
    """The backward with its dX product on MX-FP8 operands (moe_layer_bwd_mxfp8) on the bf16
    run's plan and forward: each expert's [W_gate^T | W_up^T] quantized once (timed on its own,
    a cost paid once per weight update), then per step the whole backward, with the quantization
    of dH and the fp8 dX GEMM timed by HIP events beside the bf16 run's dX GEMM."""
    import torch
    import grouped_gemm_top_amd as G
    N, H, I, E = wl.N, wl.H, wl.I, wl.E
    wt = G.quantize_dx_weights_mxfp8(wg, wu)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_.record()
    G.quantize_dx_weights_mxfp8(wg, wu, q=wt[0], scales=wt[1])
    b_.record()
    torch.cuda.synchronize()
    wq_ms = a_.elapsed_time(b_)
    o = dict(dx=torch.empty_like(x), dw_gate=torch.empty_like(wg), dw_up=torch.empty_like(wu),
             dw_down=torch.empty_like(wd), ds=torch.empty((N, wl.k), dtype=torch.float32, device="cuda"))
    ws8 = torch.empty(G.workspace_bytes(G.OP_LAYER_BWD_MXFP8, G.MOE_BF16, N, E, wl.k, H, I, plan.M_cap),
                      dtype=torch.uint8, device="cuda")

    def stepb():
        G.layer_bwd_mxfp8(dout, x, wg, wu, wd, wt, plan, hcache, ws=ws8, **o)

    for _ in range(args.warmup):
        stepb()
    names = ("quant", "dx_fp8")
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for n in names}
    for pairs in evs.values():
        for e0, e1 in pairs:
            e0.record()
            e1.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        for n in names:
            G.set_kernel_events(n, *evs[n][i])
        stepb()
    torch.cuda.synchronize()
    for n in names:
        G.set_kernel_events(n, None, None)
    us = {n: 1e3 * float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[n]])) for n in names}
    sc = 1.0 + 1.0 / 32  # codes plus one scale byte per 32
    f = 4.0 * M * H * I
    b = M * 2 * I * sc + 2.0 * e_act * I * H * sc + 2.0 * M * H  # dH codes, weight codes, dXe (bf16)
    bf16_us = 1e3 * kern_ms["dx"]
    t_s = us["dx_fp8"] * 1e-6
    out = {"note": "backward with the dX product on MX-FP8 operands (moe_layer_bwd_mxfp8) on the bf16 run's plan; "
                   "[W_gate^T | W_up^T] quantized once, dH every step; dW and dS as in the bf16 backward",
           "kernels_us": {"quant_dh": round(us["quant"], 2), "dx_fp8": round(us["dx_fp8"], 2)},
           "weights_quant_ms": round(wq_ms, 3),
           "bf16_dx_us": round(bf16_us, 2),
           "speedup_vs_bf16_dx": round(bf16_us / (us["quant"] + us["dx_fp8"]), 3),
           "gemm_speedup_vs_bf16_dx": round(bf16_us / us["dx_fp8"], 3),
           "dx_fp8_tflops": round(f / t_s / 1e12, 1)}
    if b / (PEAK_HBM_GBS * 1e9) >= f / (PEAK_FP8_TFLOPS * 1e12):
        out["roofline"] = {"kernel": "dx_fp8", "bound": "hbm", "achieved": round(b / t_s / 1e9, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(b / t_s / 1e9 / PEAK_HBM_GBS, 4),
                           "traffic": None, "algorithmic_bytes": b, "us": round(us["dx_fp8"], 2)}
    else:
        out["roofline"] = {"kernel": "dx_fp8", "bound": "mfma", "achieved": round(f / t_s / 1e12, 1),
                           "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(f / t_s / 1e12 / PEAK_FP8_TFLOPS, 4), "traffic": None,
                           "algorithmic_flops": f, "us": round(us["dx_fp8"], 2)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first (the clock and caches settle over the first few dozen)")
    ap.add_argument("--config", type=int, default=2, help="workload number (1-5); 2 is the headline")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens in the CPU-oracle baseline sample (0 disables it)")
    ap.add_argument("--cpu-single-tokens", type=int, default=256,
                    help="tokens of the single-thread CPU-oracle run")
    ap.add_argument("--kernel-events", type=int, default=1, help="record per-kernel HIP events (1/0)")
    ap.add_argument("--routing", choices=("workload", "capacity"), default="workload",
                    help="capacity: route with a capacity plan (each expert keeps at most "
                         "C = ceil(factor * N * k / E) tokens) instead of the workload's routing")
    ap.add_argument("--capacity-factor", type=float, default=1.0)
    ap.add_argument("--cap-policy", type=int, choices=(0, 1), default=0,
                    help="capacity drop policy: 0 keeps the first C tokens, 1 the C most probable")
    ap.add_argument("--mode", choices=("layer", "copy", "peak"), default="layer",
                    help="copy: time a plain 1 GiB device-to-device copy (the calibration run for the "
                         "FETCH_SIZE / WRITE_SIZE counters); peak: only the measured device peaks "
                         "(dense bf16 MFMA and HBM streaming probes)")
    ap.add_argument("--peaks", type=int, default=1, help="measure the device peaks after the layer (1/0)")
    ap.add_argument("--fp8", type=int, default=1,
                    help="also time the MX-FP8 forward (quantize x, gate/up + down on fp8 operands) beside the "
                         "bf16 forward GEMMs, and the backward's dX product on fp8 operands beside the bf16 one "
                         "(1/0; bf16 top-k workloads)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this layer has no multi-GPU path to time", file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_gemm_top_amd as G
    from grouped_gemm_top_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "copy":
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": args.steps,
                          "ms": round(dt * 1e3, 4), "gbs": round(2 * nbytes / dt / 1e9, 1)}), flush=True)
        return
    if args.mode == "peak":
        from grouped_gemm_top_amd import probe
        pk = probe.measure_peaks()
        pk.update({"mode": "peak", "published_mfma_bf16_tflops": PEAK_BF16_TFLOPS,
                   "published_hbm_gbs": PEAK_HBM_GBS})
        print(json.dumps(pk), flush=True)
        return
    G.lib()
    wl = W.WORKLOADS[args.config]
    print(f"# generating {wl.name}", file=sys.stderr, flush=True)
    T = W.generate(wl)
    dev = "cuda"
    if wl.dtype == "bf16":
        up = lambda n: torch.from_numpy(T.bits[n].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        up = lambda n: torch.from_numpy(getattr(T, n)).to(dev)
    x, wg, wu, wd, dout = (up(n) for n in ("x", "wg", "wu", "wd", "dout"))
    logits = torch.from_numpy(T.logits).to(dev)
    bias = None if T.bias is None else torch.from_numpy(T.bias).to(dev)
    N, H, I, E, k = wl.N, wl.H, wl.I, wl.E, wl.k
    tr = wl.routing == "tr"
    cap = args.routing == "capacity"
    if cap:
        import math
        if tr:
            print("--routing capacity replaces top-k routing; this workload uses token rounding", file=sys.stderr)
            sys.exit(2)
        C = int(math.ceil(args.capacity_factor * N * k / E))
    dt_code = G.MOE_BF16 if wl.dtype == "bf16" else G.MOE_F32
    es = 2 if wl.dtype == "bf16" else 4

    # every buffer allocated once, outside the timed region
    if cap:
        plan = G.Plan(N, E, k, kind=G.PLAN_CAP, mtile=C)
    else:
        plan = G.Plan(N, E, k, kind=G.PLAN_TR if tr else G.PLAN_TOPK, mtile=wl.mtile if tr else 0)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    wts = torch.empty((N, k), dtype=torch.float32, device=dev)
    probs = torch.empty((N, E), dtype=torch.float32, device=dev) if (tr or cap) else None
    mc = max(plan.M_cap, 1)
    hcache = torch.empty((mc, 2 * I), dtype=x.dtype, device=dev)
    y = torch.empty((mc, H), dtype=x.dtype, device=dev)
    out = torch.empty((N, H), dtype=x.dtype, device=dev)
    dx = torch.empty_like(x)
    dwg, dwu, dwd = torch.empty_like(wg), torch.empty_like(wu), torch.empty_like(wd)
    ds = torch.empty((mc,) if (tr or cap) else (N, k), dtype=torch.float32, device=dev)
    ws_route = torch.empty(G.workspace_bytes(G.OP_ROUTE_TR if (tr or cap) else G.OP_PERMUTE, dt_code, N, E, k),
                           dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(G.workspace_bytes(G.OP_GEMM_FWD, dt_code, N, E, k, H, I, plan.M_cap), dtype=torch.uint8,
                         device=dev)
    ws_bwd = torch.empty(G.workspace_bytes(G.OP_LAYER_BWD, dt_code, N, E, k, H, I, plan.M_cap),
                         dtype=torch.uint8, device=dev)

    def step():
        if tr:
            G.route_token_rounding(logits, k, wl.mtile, bias=bias, plan=plan, ws=ws_route, idx=idx, w=wts,
                                   probs=probs)
        elif cap:
            G.route_capacity(logits, k, C, args.cap_policy, bias=bias, plan=plan, ws=ws_route, idx=idx, w=wts,
                             probs=probs)
        else:
            G.route_topk(logits, k, bias=bias, idx=idx, w=wts)
            G.permute(idx, wts, E, plan=plan, ws=ws_route)
        G.grouped_gemm_fwd(x, wg, wu, wd, plan, hcache=hcache, y=y, ws=ws_fwd)
        G.unpermute_combine(y, plan, out=out)
        G.layer_bwd(dout, x, wg, wu, wd, plan, hcache, dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd, ds=ds,
                    ws=ws_bwd)

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps run without the per-kernel event hook: every event recorded between two
    # kernels holds the queue for several microseconds, which would count against the step.
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # Per-step durations: the same number of steps again, a HIP event on the current stream
    # between consecutive steps (one event per step; no per-kernel hook).
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e_ in sev:
        e_.record()
    torch.cuda.synchronize()
    sev[0].record()
    for i in range(args.steps):
        step()
        sev[i + 1].record()
    torch.cuda.synchronize()
    step_ms = [sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)]

    # Per-kernel durations: the same steps again, each kernel bracketed by HIP events on its
    # launch stream (the library's hook).
    rt = tr or cap  # routing through the rounding / capacity plan kernels
    names = [n for n in ALL_KERNELS if not (rt and n == "permute") and not (not rt and n == "route_tr_plan")]
    evs = {}
    if args.kernel_events:
        evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)] for n in names}
        for pairs in evs.values():  # torch creates the HIP event lazily, at its first record
            for a, b in pairs:
                a.record()
                b.record()
        print(f"# per-kernel events over {args.steps} more steps", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        for i in range(args.steps):
            for n in evs:
                G.set_kernel_events(n, *evs[n][i])
            step()
        torch.cuda.synchronize()
        for n in evs:
            G.set_kernel_events(n, None, None)

    kern_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in evs[n]])) for n in evs}
    counts = plan.counts.cpu().numpy()
    M = int(plan.offsets[-1].item())
    e_act = int((counts > 0).sum())
    flops = 18.0 * M * H * I
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS

    res = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded gaussian inputs, see workloads.py)",
        "config": {"workload": wl.name, "N": N, "H": H, "I": I, "E": E, "k": k,
                   "routing": "capacity" if cap else wl.routing,
                   "rows": M, "active_experts": e_act, "parallelism": "single GPU"},
        "pct_peak": round(100.0 * tflops / peak, 2),
        "layer_ms": {"mean": round(ms, 4), "median": round(float(np.median(step_ms)), 4),
                     "min": round(float(np.min(step_ms)), 4), "max": round(float(np.max(step_ms)), 4),
                     "note": "mean: the timed steps; median/min/max: per-step HIP events over as many more steps"},
    }
    if kern_ms:
        gemm_ms = sum(kern_ms[n] for n in GEMMS)
        res["gemm_ms"] = round(gemm_ms, 4)
        res["gemm_tflops"] = round(flops / (gemm_ms * 1e-3) / 1e12, 2)
        res["gemm_pct_peak"] = round(100.0 * res["gemm_tflops"] / peak, 2)
        res["fwd_ms"] = round(sum(kern_ms.get(n, 0.0) for n in ("route", "permute", "route_tr_plan", "gateup",
                                                                  "down", "combine")), 4)
        res["bwd_ms"] = round(sum(kern_ms.get(n, 0.0) for n in ("dh", "dwd", "dx", "dx_combine",
                                                                  "dw1")), 4)
        kinfo = {}
        for n in names:
            f, b = kernel_work(n, wl, M, e_act, es)
            kinfo[n] = {"us": round(kern_ms[n] * 1e3, 2)}
            if f:
                kinfo[n]["tflops"] = round(f / (kern_ms[n] * 1e-3) / 1e12, 2)
                kinfo[n]["gbs"] = round(b / (kern_ms[n] * 1e-3) / 1e9, 1)
        res["kernels"] = kinfo
        dom = max(GEMMS, key=lambda n: kern_ms[n])
        f, b = kernel_work(dom, wl, M, e_act, es)
        t_s = kern_ms[dom] * 1e-3
        hbm_bound = b / (PEAK_HBM_GBS * 1e9) >= f / (peak * 1e12)
        traffic = load_traffic(dom, wl.name)
        if hbm_bound:
            ach = b / t_s / 1e9
            res["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                               "algorithmic_bytes": b, "us": round(kern_ms[dom] * 1e3, 2)}
        else:
            ach = f / t_s / 1e12
            res["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                               "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                               "algorithmic_flops": f, "us": round(kern_ms[dom] * 1e3, 2)}
    # The router's own product and backward (logits = x W_r + bias; dS -> dlogits, dW_r, dbias
    # and the router's share of dx), timed on their own after the layer: the layer's metric
    # starts from the logits, as the workload defines it.
    if args.kernel_events:
        wr = torch.from_numpy(T.wr).to(dev)
        lg_r = torch.empty((N, E), dtype=torch.float32, device=dev)
        dlg = torch.empty((N, E), dtype=torch.float32, device=dev)
        dwr = torch.empty((H, E), dtype=torch.float32, device=dev)
        dbias = torch.empty((E,), dtype=torch.float32, device=dev)
        dx_r = torch.empty_like(dx)
        ws_r = torch.empty(G.workspace_bytes(G.OP_ROUTER_BWD, dt_code, N, E, k, H, 8, 0), dtype=torch.uint8,
                           device=dev)
        ws_l = torch.empty(G.workspace_bytes(G.OP_ROUTER_LOGITS, dt_code, N, E, 1, H, 8, 0), dtype=torch.uint8,
                           device=dev)

        def router_step():
            G.router_logits(x, wr, bias, logits=lg_r, ws=ws_l)
            G.router_bwd(logits, idx, plan, ds, x, wr, bias=bias, dx_in=dx, dx_out=dx_r, dlogits=dlg, dw_r=dwr,
                         dbias=dbias, ws=ws_r)

        for _ in range(args.warmup):
            router_step()
        rnames = ("router_logits", "router_dz", "router_dx", "router_dw")
        rev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)] for n in rnames}
        for pairs in rev.values():
            for a_, b_ in pairs:
                a_.record()
                b_.record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            for n in rnames:
                G.set_kernel_events(n, *rev[n][i])
            router_step()
        torch.cuda.synchronize()
        for n in rnames:
            G.set_kernel_events(n, None, None)
        r_us = {n: round(float(np.mean([a_.elapsed_time(b_) for a_, b_ in rev[n]])) * 1e3, 2) for n in rnames}
        fl = 2.0 * N * H * E
        res["router"] = {
            "note": "router logits product and router backward, timed separately (not in ms_per_step)",
            "kernels_us": r_us,
            "logits_tflops": round(fl / (r_us["router_logits"] * 1e-6) / 1e12, 2),
            "bwd_us": round(r_us["router_dz"] + r_us["router_dx"] + r_us["router_dw"], 2),
        }
    if args.fp8 and wl.dtype == "bf16" and not rt and args.kernel_events:
        res["fp8"] = fp8_forward(args, wl, x, wg, wu, wd, plan, M, e_act, kern_ms)
        if wl.H % 32 == 0 and wl.I % 32 == 0:
            res["fp8"]["backward_dx"] = fp8_backward_dx(args, wl, x, wg, wu, wd, dout, plan, hcache, M, e_act,
                                                        kern_ms)
    # The bound the whole step can reach: the larger of its FLOPs at the MFMA peak and its
    # algorithmic bytes (every tensor touched once per pass) at the HBM peak.
    lb = layer_bytes(wl, M, e_act, es)
    t_bound = max(flops / (peak * 1e12), lb / (PEAK_HBM_GBS * 1e9))
    res["attainable"] = {"algorithmic_bytes": lb, "t_bound_ms": round(t_bound * 1e3, 4),
                         "bound": "hbm" if lb / (PEAK_HBM_GBS * 1e9) >= flops / (peak * 1e12) else "mfma",
                         "frac_of_bound": round(t_bound / (ms * 1e-3), 4),
                         "max_pct_of_mfma_peak": round(100.0 * flops / (peak * 1e12) / t_bound, 2)}
    if args.peaks:
        from grouped_gemm_top_amd import probe
        pk = probe.measure_peaks()
        pk["note"] = ("measured with the probes of libmoe_probe.so (inline-asm MFMA loop on registers; "
                      "16-byte streaming copy and read of 1 GiB); roofline.peak stays the published figure")
        res["measured_peaks"] = pk
        res["pct_of_measured_mfma_peak"] = round(100.0 * tflops / max(pk["mfma_bf16_16x16x32_tflops"],
                                                                      pk["mfma_bf16_32x32x16_tflops"]), 2)
    res["padded_row_fraction"] = padded_fractions(counts, M)
    if cap:
        res["config"].update({"capacity_factor": args.capacity_factor, "capacity": C,
                              "cap_policy": "probs" if args.cap_policy else "position"})
        res["capacity"] = {"dropped_pairs": N * k - M, "dropped_fraction": round((N * k - M) / (N * k), 4),
                           "dense_layout_rows": E * C, "dense_padding_rows": E * C - M,
                           "dense_padding_fraction": round((E * C - M) / max(E * C, 1), 4)}

    if args.cpu_tokens > 0:
        import oracle
        nt = min(args.cpu_tokens, N)
        print(f"# cpu baseline (fp32 oracle) on the rows of {nt} tokens", file=sys.stderr, flush=True)
        pt, pe, pw = oracle.pairs_from_plan(plan.host(), E)
        keep = pt < nt
        what = (f"the whole workload" if nt == N else f"the rows of the first {nt} of {N} tokens") + \
            (" (the GPU's routing plan)" if (tr or cap) else "")
        res["cpu_baseline"] = cpu_baseline(T, pt[keep], pe[keep], pw[keep], what, min(args.cpu_single_tokens, nt))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
