"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`build()` links libw12_hostcheck.so: the library with its host-side C ABI
(argument checks, workspace sizes, plans, dispatch) compiled with both
sanitizers. A small C driver (tests/host/abi_host_check.c), itself built with
them, calls every entry point along paths that return before any HIP call:
plans over a grid of shapes, M, ops, flags and test hooks, and the argument
errors of each call. Any sanitizer report aborts the driver."""
import os
import shutil
import subprocess

import pytest

from lossless_compressed_weight_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(b.HOSTCHECK_LIB):
        pytest.skip("libw12_hostcheck.so is not built (run the package build)")
    cc = CLANG if os.path.exists(CLANG) else shutil.which("clang")
    if cc is None:
        pytest.skip("no clang for the sanitized driver")
    exe = str(tmp_path / "abi_host_check")
    libdir = os.path.dirname(b.HOSTCHECK_LIB)
    cmd = [cc, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1",
           f"-I{b.INCLUDE}", os.path.join(HERE, "host", "abi_host_check.c"), b.HOSTCHECK_LIB,
           f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"driver build failed:\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"host checks failed (exit {r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
