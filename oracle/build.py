"""Compile the oracle's C library (test infrastructure only).

    python oracle/build.py      # writes oracle/libtsoracle.so

Plain gcc, -O2, no fast-math (the ascending-k fp64 summation must be kept).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_gemm.c")
LIB = os.path.join(HERE, "libtsoracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
