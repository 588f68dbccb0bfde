"""Build the CPU oracle library (test infrastructure only).

    python -m oracle.build            # oracle/liboracle.so
    build(mutation=n, out=path)       # a copy with one planted mistake, for the pin tests
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mnb_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(mutation: int = 0, out: str | None = None, verbose: bool = False) -> str:
    out = out or LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-DMNBO_MUTATION=%d" % mutation, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
