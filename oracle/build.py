"""Build the fp64 CPU oracle (test infrastructure) with gcc.

    python oracle/build.py

Produces oracle/libfdoracle.so.  No -ffast-math: the oracle relies on IEEE
exp/log and on NaN comparisons behaving as specified.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fd_oracle.c")
OUT = os.path.join(HERE, "libfdoracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-shared", "-fPIC",
           SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
