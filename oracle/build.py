"""Compile the CPU oracle (test infrastructure) into oracle/libswe_oracle.so.

Plain gcc, -O2, no fast-math and no floating-point contraction, OpenMP over
cells (results do not depend on the thread count: every cell's update is
computed on its own and the time-step minimum is exact).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "swe_oracle.c")
LIB = os.path.join(HERE, "libswe_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile src (default: the oracle) into the shared library lib."""
    tmp = lib + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
