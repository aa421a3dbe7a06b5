"""Build libmoe.so (all HIP sources under csrc/) and libmoe_probe.so (the measurement probes
under csrc/probe/) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe.so")
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile_link(srcs, lib, tag, verbose, jobs):
    def compile_one(src):
        obj = os.path.join(BUILD, tag + os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, flush=True)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source (always) and link libmoe.so and libmoe_probe.so.  Returns the
    path of libmoe.so."""
    os.makedirs(BUILD, exist_ok=True)
    _compile_link(sources(), LIB, "", verbose, jobs)
    _compile_link(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB, "probe_", verbose, jobs)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
