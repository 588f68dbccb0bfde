"""CPU sanitizer runs (no GPU is used).

 - The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
   ``oracle.build.build(sanitize=True)``) runs the whole pin suite, every finding fatal.
 - libmnb's host code (validation, the dispatcher, workspace layout, the GEMM planner,
   route descriptions) is compiled from the library's sources with both sanitizers on the
   host side only (``-Xarch_host``; the GPU code is compiled as usual and never runs), and
   linked into ``tests/host_harness.cpp``, which sweeps every host-only call over shapes up
   to the int limits and every validation path of the matmul and pack calls.

Commands (what the tests run; from the repository root):

    python -c "from oracle import build; build.build(sanitize=True)"
    MNB_ORACLE_LIB=oracle/liboracle_san.so LD_PRELOAD=$(gcc -print-file-name=libasan.so) \\
        ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_oracle_pins.py -x -q
    python -m pytest tests/test_sanitizers.py -k host     # builds and runs the host harness
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from _util import ROOT

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan():
    from oracle import build as obuild
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = obuild.build(sanitize=True)
    env = dict(os.environ, MNB_ORACLE_LIB=lib, LD_PRELOAD=asan, **SAN_ENV)
    check = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.load()._name)"], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=300)
    assert check.returncode == 0 and check.stdout.strip() == lib, check.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout


def _library_build():
    spec = importlib.util.spec_from_file_location(
        "_mnb_build", os.path.join(ROOT, "blockwise_bit_quantized_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def test_host_logic_under_asan_and_ubsan():
    b = _library_build()
    hipcc = b._hipcc()
    if not os.path.exists(hipcc) and os.path.sep in hipcc:
        pytest.skip("hipcc not found")
    out = os.path.join(b.OBJ, "sanitize")
    os.makedirs(out, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src).rsplit(".", 1)[0] + ".o")
        if os.path.exists(obj) and os.path.getmtime(obj) > max(
                os.path.getmtime(p) for p in (src, os.path.join(b.CSRC, "common.h"),
                                              os.path.join(ROOT, "include", "mnb.h"))):
            return obj
        lang = ["-x", "c++"] if src.endswith(".cpp") else []
        cmd = [hipcc, *b.HIPCC_FLAGS, *san, *lang, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stderr[-3000:])
        return obj

    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES] + [os.path.join(ROOT, "tests", "host_harness.cpp")]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(out, "host_harness")
    r = subprocess.run([hipcc, "--offload-arch=" + b.ARCH, *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], env=dict(os.environ, **SAN_ENV), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "0 failures" in r.stdout, r.stdout
