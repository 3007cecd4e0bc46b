"""Build the CPU oracle shared library (plain C, gcc).

Test infrastructure: the library built here is loaded only by the test suite, the smoke
check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmm_oracle.c")
LIB = os.path.join(HERE, "libqmm_oracle.so")

# -ffp-contract=off and no fast-math: every float operation is one IEEE operation.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
