"""Host-code sanitizer runs, on the CPU (no GPU is touched):

* the C oracle built with gcc -fsanitize=address,undefined, running the oracle's pins
  (tests/test_oracle.py, tests/test_oracle_fp8.py) on that build;
* libmoe.so with AddressSanitizer on its host pass only (argument validation, workspace and
  plan sizing, launch sequencing up to the first HIP call), running the C-ABI checks
  (tests/test_abi.py) on that build.

Python itself is not instrumented, so each run is a child process with the sanitizer runtime
preloaded; any report makes the child fail.  The builds go to a temporary directory."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow


def _child(env_extra, test_files, extra_args=()):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    test_files = [test_files] if isinstance(test_files, str) else list(test_files)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu and not slow",
           *[os.path.join(ROOT, "tests", f) for f in test_files], *extra_args]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized run of {test_files} failed (rc {r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return r


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"{name} not found")
    return p


def test_oracle_pins_under_asan_ubsan(tmp_path):
    src = os.path.join(ROOT, "oracle", "moe_oracle.c")
    for real, ctype in (("f64", "double"), ("f32", "float")):
        out = tmp_path / f"liboracle_{real}.so"
        subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared",
                        f"-DORACLE_REAL={ctype}", "-fvisibility=hidden", src, "-o", str(out), "-lm"], check=True)
    preload = _gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so")
    r = _child({"ORACLE_LIB_DIR": str(tmp_path), "LD_PRELOAD": preload}, ["test_oracle.py", "test_oracle_fp8.py"])
    assert " passed" in r.stdout


def test_abi_checks_under_host_asan(tmp_path):
    from grouped_gemm_top_amd import build as B
    rt = None
    for base in ("/opt/rocm/llvm/lib/clang", "/opt/rocm/lib/llvm/lib/clang"):
        if os.path.isdir(base):
            for v in sorted(os.listdir(base)):
                cand = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(cand):
                    rt = cand
    if rt is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    # the sanitizer applies to the host pass only; the device code is built as usual
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    objs = []
    for src in B.sources():
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([B.HIPCC, *B.FLAGS, *host_asan, "-c", src, "-o", str(obj)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(str(obj))
    lib = tmp_path / "libmoe_asan.so"
    # the sanitizer's symbols come from the preloaded runtime
    subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", str(lib)], check=True,
                   capture_output=True)
    r = _child({"MOE_ABI_TEST_LIB": str(lib), "LD_PRELOAD": rt}, "test_abi.py", ("-k", "not probe"))
    assert " passed" in r.stdout
