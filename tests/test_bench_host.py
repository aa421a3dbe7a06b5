"""bench.py's host side, on the CPU (no GPU is touched): the per-kernel work model behind the
`roofline` object, the source-hash guard on the committed HBM-traffic figures, and the refusal of
more than one GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from grouped_gemm_top_amd import workloads as W  # noqa: E402

HEADLINE = "microbench-E128-H2048-I512-k8-N4096"


def _headline():
    wl = W.WORKLOADS[2]
    assert wl.name == HEADLINE
    return wl, wl.N * wl.k  # every pair makes a row under top-k routing


def test_gemm_flops_add_up_to_the_layer_metric():
    """The six GEMMs' FLOPs are the 18 M H I that the layer's TFLOPS figure divides by."""
    for n in (1, 2, 3, 4, 5):
        wl = W.WORKLOADS[n]
        M = wl.N * wl.k
        total = sum(bench.kernel_work(k, wl, M, wl.E, 2)[0] for k in bench.GEMMS)
        assert total == pytest.approx(wl.flops)
        assert wl.flops == 18.0 * M * wl.H * wl.I


def test_headline_byte_counts():
    """Algorithmic bytes at the headline shape, counted tensor by tensor (bf16, 128 experts all
    active, 32768 rows): the dominant kernel's figure is the one the roofline divides by."""
    wl, M = _headline()
    MiB = 1 << 20
    w_gu = 2 * 128 * 512 * 2048 * 2      # W_gate and W_up of every expert: 512 MiB
    w_d = 128 * 2048 * 512 * 2           # W_down: 256 MiB
    x = 4096 * 2048 * 2                  # x, out, dOut, dX: 16 MiB each
    rows_i = M * 512 * 2                 # one [M, I] bf16 row tensor: 32 MiB
    rows_h = M * 2048 * 2                # one [M, H] bf16 row tensor: 128 MiB
    assert w_gu == 512 * MiB and w_d == 256 * MiB and x == 16 * MiB
    # gate/up: both weights, x once, [G | U] and A written
    assert bench.kernel_work("gateup", wl, M, 128, 2)[1] == w_gu + x + 3 * rows_i
    # down: W_down, A read, Y written
    assert bench.kernel_work("down", wl, M, 128, 2)[1] == w_d + rows_i + rows_h
    # dW_g/u: both weight gradients written, x and [dG | dU] read
    assert bench.kernel_work("dw1", wl, M, 128, 2)[1] == w_gu + x + 2 * rows_i == 620756992
    # dW_d: its gradient written, dOut and A' read
    assert bench.kernel_work("dwd", wl, M, 128, 2)[1] == w_d + x + rows_i
    # dX: both weights, [dG | dU] read, dXe written
    assert bench.kernel_work("dx", wl, M, 128, 2)[1] == w_gu + 2 * rows_i + rows_h
    # combine: Y read, out written, row weights and row lists
    assert bench.kernel_work("combine", wl, M, 128, 2)[1] == rows_h + x + 8 * M


def _tree(tmp_path):
    """A copy of the profiles and kernel sources that load_traffic reads."""
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    shutil.copytree(os.path.join(ROOT, "grouped_gemm_top_amd", "csrc"), tmp_path / "grouped_gemm_top_amd" / "csrc")
    return tmp_path


def test_traffic_guard_follows_the_sources(tmp_path, monkeypatch):
    if not os.path.exists(os.path.join(ROOT, "profiles", f"traffic_{HEADLINE}.txt")):
        pytest.skip("no committed traffic summary")
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    v = bench.load_traffic("dw1", HEADLINE)
    if v is None:
        pytest.skip("the committed traffic summary predates the current GEMM source")
    assert v > bench.kernel_work("dw1", *_headline(), 128, 2)[1] * 0.5
    # one changed byte in a source the figure depends on: the figure is withdrawn
    src = root / "grouped_gemm_top_amd" / "csrc" / "gemm_lds.h"
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.load_traffic("dw1", HEADLINE) is None
    assert bench.load_traffic("no_such_kernel", HEADLINE) is None
    assert bench.load_traffic("dw1", "no-such-workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
