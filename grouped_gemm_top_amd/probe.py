"""Binding of libmoe_probe.so: the measurement probes for the device peaks (dense bf16 MFMA
throughput, HBM streaming bandwidth) that bench.py reports beside the published peaks.
Argument marshalling only; the probes are HIP kernels declared in ``include/moe_probe.h``."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

PROBE_SYMBOLS = ("moe_probe_mfma_bf16", "moe_probe_copy", "moe_probe_read", "moe_probe_mfma_fp8_layout",
                 "moe_probe_cvt_fp8", "moe_probe_reread")
FLOP_PER_ITER_WAVE = 131072  # eight 16x16x32 (or four 32x32x16) bf16 MFMAs


def lib_path() -> str:
    return os.path.join(_HERE, "libmoe_probe.so")


def lib():
    """Load libmoe_probe.so; raise if it is missing (build it with grouped_gemm_top_amd.build)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m grouped_gemm_top_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_probe_mfma_bf16.argtypes = [i32, i32, i32, vp, vp]
        L.moe_probe_copy.argtypes = [vp, vp, sz, i32, vp]
        L.moe_probe_read.argtypes = [vp, sz, i32, vp, vp]
        L.moe_probe_mfma_fp8_layout.argtypes = [vp, vp, vp, vp, i32, vp, vp]
        L.moe_probe_cvt_fp8.argtypes = [vp, i32, vp, vp]
        L.moe_probe_reread.argtypes = [vp, sz, i32, i32, i32, vp, vp]
        for n in PROBE_SYMBOLS:
            getattr(L, n).restype = i32
        _LIB = L
    return _LIB


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with status {rc}")


def mfma_bf16(shape: int, blocks: int, iters: int, sink, stream=None) -> float:
    """Queue the MFMA probe; returns the FLOPs it performs.  sink: float32 cuda tensor of at
    least blocks * 256 elements."""
    assert sink.numel() >= blocks * 256 and sink.is_cuda
    _check(lib().moe_probe_mfma_bf16(shape, blocks, iters, ctypes.c_void_p(sink.data_ptr()), _stream(stream)),
           "moe_probe_mfma_bf16")
    return float(blocks) * 4 * iters * FLOP_PER_ITER_WAVE


def copy(src, dst, blocks: int, stream=None) -> int:
    """Queue the copy probe over src's bytes; returns the bytes moved (read + written)."""
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nb and src.is_cuda and dst.is_cuda
    _check(lib().moe_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nb, blocks,
                                _stream(stream)), "moe_probe_copy")
    return 2 * nb


def read(src, blocks: int, sink, stream=None) -> int:
    """Queue the read probe over src's bytes; sink: int32/uint32 cuda tensor of at least
    blocks * 256 elements.  Returns the bytes read."""
    nb = src.numel() * src.element_size()
    assert sink.numel() >= blocks * 256 and sink.element_size() == 4 and src.is_cuda and sink.is_cuda
    _check(lib().moe_probe_read(ctypes.c_void_p(src.data_ptr()), nb, blocks, ctypes.c_void_p(sink.data_ptr()),
                                _stream(stream)), "moe_probe_read")
    return nb


def measure_peaks(reps: int = 5) -> dict:
    """Time each probe `reps` times with HIP events on the current stream (after one untimed
    launch) and return the best rates."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"compute_units": cus}

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            work = fn()
            b.record()
            b.synchronize()
            ts.append((a.elapsed_time(b) * 1e-3, work))
        t, work = min(ts)
        return work / t

    blocks = 4 * cus  # four workgroups of four wavefronts per CU: four wavefronts per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for shape, name in ((0, "mfma_bf16_16x16x32_tflops"), (1, "mfma_bf16_32x32x16_tflops")):
        out[name] = round(best(lambda: mfma_bf16(shape, blocks, 40000, sink)) / 1e12, 1)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sblocks = 16 * cus
    isink = torch.empty(sblocks * 256, dtype=torch.int32, device="cuda")
    out["copy_gbs"] = round(best(lambda: copy(src, dst, sblocks)) / 1e9, 1)
    out["read_gbs"] = round(best(lambda: read(src, sblocks, isink)) / 1e9, 1)
    del src, dst
    # kilobyte loads into LDS (the GEMMs' load form) of a 2 MiB buffer, 512 passes: each XCD
    # reads its eighth of it, which stays in its L2
    small = torch.ones(1 << 19, dtype=torch.float32, device="cuda")
    rblocks = 2 * cus
    rsink = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
    out["l2_lds_load_gbs"] = round(best(lambda: reread(small, 512, 1, rblocks, rsink)) / 1e9, 1)
    return out


def mfma_fp8_layout(a, b, sa, sb, d, stream=None):
    """Queue the scaled-fp8 MFMA lane-layout probe.  a, b: uint8 cuda [cases, 64, 32]; sa, sb:
    int32 cuda [cases, 64]; d: float32 cuda [cases, 64, 4] (written)."""
    cases = a.shape[0]
    assert a.shape == (cases, 64, 32) and b.shape == a.shape and sa.shape == (cases, 64) and sb.shape == sa.shape
    assert d.shape == (cases, 64, 4)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(lib().moe_probe_mfma_fp8_layout(p(a), p(b), p(sa), p(sb), cases, p(d), _stream(stream)),
           "moe_probe_mfma_fp8_layout")


def cvt_fp8(src, dst, stream=None):
    """Queue the fp32 -> fp8 e4m3 conversion probe: dst (uint8 cuda) = codes of src (float32
    cuda, even length)."""
    assert src.numel() == dst.numel() and src.numel() % 2 == 0
    _check(lib().moe_probe_cvt_fp8(ctypes.c_void_p(src.data_ptr()), src.numel(), ctypes.c_void_p(dst.data_ptr()),
                                   _stream(stream)), "moe_probe_cvt_fp8")


def reread(src, passes: int, mode: int, blocks: int, sink, stream=None) -> int:
    """Queue the re-read probe over src (cuda, contiguous, a multiple of 1 KiB); mode 0 loads
    into registers, mode 1 into LDS.  Returns the bytes read."""
    nb = src.numel() * src.element_size()
    _check(lib().moe_probe_reread(ctypes.c_void_p(src.data_ptr()), nb, passes, mode, blocks,
                                  ctypes.c_void_p(sink.data_ptr()), _stream(stream)), "moe_probe_reread")
    return nb * passes
