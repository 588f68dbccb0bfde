"""Build libmnb.so (HIP, gfx950) in-tree with hipcc.

    python blockwise_bit_quantized_amd/build.py

(run by path: importing the package loads the library this script builds)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmnb.so")
# measurement helper for the benchmark (a streaming-read ceiling kernel), not the ABI
CEILING_LIB = os.path.join(PKG, "libmnb_ceiling.so")
CEILING_SOURCE = "ceiling.hip"
OBJ = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "gemv.hip", "gemv_mfma.hip", "gemv_acc4.hip", "tproj.hip", "gemm.hip", "pack.hip"]
ARCH = os.environ.get("MNB_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # code object v5 loads under both the system ROCm runtime and the one torch bundles
    "-mcode-object-version=5",
    # packed FP32 ops are disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
        if err.strip() and verbose:
            print(err, flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-mcode-object-version=5", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    _check_undefined(tmp)
    os.replace(tmp, LIB)
    _build_ceiling(hipcc, verbose)
    return LIB


def _build_ceiling(hipcc: str, verbose: bool) -> None:
    tmp = CEILING_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", os.path.join(CSRC, CEILING_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (CEILING_SOURCE, r.stderr))
    os.replace(tmp, CEILING_LIB)


def _check_undefined(path: str) -> None:
    """A kernel whose host-side launch stub was not emitted links fine but cannot be
    loaded; refuse such a library here instead of at import time."""
    r = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True)
    if r.returncode != 0:
        return                                   # nm unavailable: the loader still checks
    bad = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN3mnb" in l]
    if bad:
        os.remove(path)
        raise RuntimeError("libmnb links against undefined symbols of its own: " + ", ".join(bad[:4]))


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
