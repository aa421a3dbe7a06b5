"""Seeded synthetic workloads for the MoE expert-MLP layer.

This module only draws random inputs; it holds none of the layer's arithmetic.  Both the
HIP path (through tests and the benchmark) and the CPU oracle consume exactly the arrays it
returns, so the two sides always see identical inputs.

Recipe (fixed, so every run of a workload sees the same numbers):
  * numpy PCG64 streams from ``SeedSequence(seed)``, seed = 1000 + workload number (or
    an explicit seed).  The sequence is spawned into one child per draw slot, in the order
    x [N,H], W_r [H,E], bias [E], W_gate [E,I,H], W_up [E,I,H], W_down [E,H,I], dOut [N,H],
    expert permutation; each tensor is cut into chunks of 2^22 elements and chunk c is drawn
    from the c-th child of its slot, so the values do not depend on the thread count;
  * every draw is an fp32 standard normal times the stated standard deviation;
  * for bf16 workloads x, the three weight tensors and dOut are rounded to bf16
    (round-to-nearest-even); the fp32 copies handed out hold exactly those values;
  * router logits = (x as fp64) @ (W_r as fp64) + bias, rounded once to fp32.  The logits are
    an input of the routed layer, shared by both sides;
  * Zipf bias: pi = a random permutation of the E experts, p_r proportional to r^-s
    (r = 1..E), bias_e = ln p_{pi(e)+1}.  It makes a few experts receive most tokens and
    many receive none, the skew that the expert-parallel page ("EP: Expert를 나누고 토큰
    보내기", section "Expert가 같은 개수여도 처리할 토큰 수는 다르다") warns about.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    I: int
    E: int
    k: int
    dtype: str            # "f32" or "bf16" storage; accumulation is always fp32 or wider
    bias: str = "none"    # "none" | "normal" | "zipf"
    bias_std: float = 0.0
    zipf_s: float = 0.0
    routing: str = "topk"  # "topk" | "tr" (token rounding) | "cap" (capacity: mtile = C)
    mtile: int = 128
    cap_policy: int = 0    # capacity plans: 0 keeps the first C tokens, 1 the C most probable
    seed: int = 0
    w_std: float = 0.02
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def flops(self) -> float:
        """Algorithmic fwd+bwd FLOPs for M = N*k rows (18*M*H*I: gate+up 4MHI, down 2MHI,
        backward twice the forward)."""
        return 18.0 * self.N * self.k * self.H * self.I


# The five workloads.  Shapes follow the pages: the microbenchmark of "DeepSeek 계열 MoE 학습
# 가속" (Experiments: E=128, H=2048, moe_intermediate=512, top_k=8, N=4096), the
# DeepSeek-V3 expert shape of the same page (E=256, H=2048, I=512), the E=128 / k=4 model of
# "Deep EP" (GPT-OSS structure), and the high-sparsity token-rounding regime of "SonicMoE".
WORKLOADS = {
    1: Workload("tiny-fp32", N=64, H=64, I=32, E=8, k=2, dtype="f32", seed=1001),
    2: Workload("microbench-E128-H2048-I512-k8-N4096", N=4096, H=2048, I=512, E=128, k=8,
                dtype="bf16", seed=1002),
    3: Workload("coarse-E128-H2880-I2880-k4-N8192", N=8192, H=2880, I=2880, E=128, k=4,
                dtype="bf16", bias="normal", bias_std=0.5, seed=1003),
    4: Workload("zipf-E256-H2048-I512-k8-N8192", N=8192, H=2048, I=512, E=256, k=8,
                dtype="bf16", bias="zipf", zipf_s=1.2, seed=1004),
    5: Workload("tokenround-E256-H4096-I256-k8-N16384", N=16384, H=4096, I=256, E=256, k=8,
                dtype="bf16", routing="tr", mtile=128, seed=1005),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round-to-nearest-even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.left_shift(bits, 16, dtype=np.uint32).view(np.float32)


@dataclass
class Tensors:
    """Host copies.  ``x, wg, wu, wd, dout`` hold the exact values as fp32 (bf16 values
    widened for bf16 workloads); ``bits`` maps the same names to the bf16 bit patterns
    (empty for fp32 workloads)."""
    wl: Workload
    x: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    dout: np.ndarray
    logits: np.ndarray
    bias: np.ndarray | None
    wr: np.ndarray
    bits: dict


_CHUNK = 1 << 22
_SLOTS = ("x", "wr", "bias", "wg", "wu", "wd", "dout", "perm")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal(seq: np.random.SeedSequence, shape, std, bf16: bool, pool):
    """fp32 normals * std, drawn chunk by chunk from children of ``seq``.  With ``bf16`` the
    values are rounded and (bits, widened fp32) is returned, else (None, values)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    bits = np.empty(n, np.uint16) if bf16 else None
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seq.spawn(nch)

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        seg = out[lo:hi]
        np.random.Generator(np.random.PCG64(kids[c])).standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= np.float32(std)
        if bf16:
            b = bf16_round(seg)
            bits[lo:hi] = b
            seg[:] = bf16_to_f32(b)

    list(pool.map(work, range(nch)))
    return (None if bits is None else bits.reshape(shape)), out.reshape(shape)


def generate(wl: Workload, seed: int | None = None, weights: bool = True) -> Tensors:
    """Draw the workload.  ``weights=False`` draws only what routing needs (x, W_r, bias,
    logits); the expert weights and dOut are then None.  The values drawn do not change."""
    ss = np.random.SeedSequence(wl.seed if seed is None else seed)
    slot = dict(zip(_SLOTS, ss.spawn(len(_SLOTS))))
    N, H, I, E = wl.N, wl.H, wl.I, wl.E
    if wl.dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {wl.dtype}")
    b16 = wl.dtype == "bf16"
    bits = {}
    with ThreadPoolExecutor(_threads()) as pool:
        bx, x = _normal(slot["x"], (N, H), 1.0, b16, pool)
        _, wr = _normal(slot["wr"], (H, E), wl.w_std, False, pool)
        bias = None
        if wl.bias == "normal":
            _, bias = _normal(slot["bias"], (E,), wl.bias_std, False, pool)
        bg = wg = bu = wu = bd = wd = bo = dout = None
        if weights:
            bg, wg = _normal(slot["wg"], (E, I, H), wl.w_std, b16, pool)
            bu, wu = _normal(slot["wu"], (E, I, H), wl.w_std, b16, pool)
            bd, wd = _normal(slot["wd"], (E, H, I), wl.w_std, b16, pool)
            bo, dout = _normal(slot["dout"], (N, H), 1.0, b16, pool)
    if wl.bias == "zipf":
        perm = np.random.Generator(np.random.PCG64(slot["perm"])).permutation(E)
        r = np.arange(1, E + 1, dtype=np.float64)
        p = r ** (-wl.zipf_s)
        p /= p.sum()
        bias = np.log(p[perm]).astype(np.float32)
    if b16:
        bits = {n: b for n, b in (("x", bx), ("wg", bg), ("wu", bu), ("wd", bd), ("dout", bo))
                if b is not None}
    lg = x.astype(np.float64) @ wr.astype(np.float64)
    if bias is not None:
        lg += bias.astype(np.float64)
    logits = lg.astype(np.float32)
    return Tensors(wl, x, wg, wu, wd, dout, logits, bias, wr, bits)


def custom(name="custom", N=256, H=128, I=96, E=8, k=2, dtype="bf16", bias="none", bias_std=0.0,
           zipf_s=0.0, routing="topk", mtile=128, seed=7, cap_policy=0) -> Workload:
    return Workload(name, N=N, H=H, I=I, E=E, k=k, dtype=dtype, bias=bias, bias_std=bias_std,
                    zipf_s=zipf_s, routing=routing, mtile=mtile, seed=seed, cap_policy=cap_policy)
