"""Build the CPU oracle library (test infrastructure only).

    python -m oracle.build            # oracle/liboracle.so
    build(mutation=n, out=path)       # a copy with one planted mistake, for the pin tests
    build(sanitize=True)              # oracle/liboracle_san.so: AddressSanitizer + UBSan build
                                      # (load it with MNB_ORACLE_LIB and libasan preloaded)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mnb_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
# host-only sanitizers (gcc; the oracle has no GPU code): every finding aborts the process
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(mutation: int = 0, out: str | None = None, verbose: bool = False, sanitize: bool = False) -> str:
    out = out or (SAN_LIB if sanitize else LIB)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter", *(SAN_FLAGS if sanitize else []),
           "-DMNBO_MUTATION=%d" % mutation, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
