"""Build libw12.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m lossless_compressed_weight_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libw12.so")
# The same library with AddressSanitizer and UndefinedBehaviorSanitizer in the
# host code of the C ABI (argument checks, sizes, plans, dispatch); its device
# code is the normal build. Loaded only by the host-side check in tests/host.
HOSTCHECK_LIB = os.path.join(PKG, "libw12_hostcheck.so")
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer -Xarch_host -g".split()
HOSTCHECK_SOURCE = "w12_api.hip"
SOURCES = ["w12_gemm.hip", "w12_gemm_mx.hip", "w12_api.hip", "w12_encode.hip", "w12_certify.hip", "w12_fixup.hip", "w12_argmax.hip", "w12_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the W12 library needs ROCm's hipcc to build")


def _jobs() -> int:
    try:
        return max(1, min(16, int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    except ValueError:
        return max(1, min(16, os.cpu_count() or 1))


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 (in parallel) and link libw12.so next to this file."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="w12build") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
            return obj

        def compile_hostcheck():
            obj = os.path.join(tmp, "hostcheck_" + HOSTCHECK_SOURCE.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, *HOST_SANITIZE, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                   os.path.join(CSRC, HOSTCHECK_SOURCE), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc (host sanitizers) failed on {HOSTCHECK_SOURCE}:\n{r.stdout}\n{r.stderr}")
            return obj

        with ThreadPoolExecutor(_jobs()) as ex:
            check_obj = ex.submit(compile_hostcheck)
            objs = list(ex.map(compile_one, SOURCES))
            check_obj = check_obj.result()

        def link(objects, out):
            tmp_lib = out + ".tmp"
            cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp_lib]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
            os.replace(tmp_lib, out)
        link(objs, LIB)
        link([check_obj if os.path.basename(o) == HOSTCHECK_SOURCE.replace(".hip", ".o") else o for o in objs],
             HOSTCHECK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
