"""Compile the fp64 CPU oracle (oracle.c) into liboracle.so with gcc.

TEST INFRASTRUCTURE ONLY: the library built here serves the test suite, the
smoke check and the benchmark's CPU-baseline leg.  Nothing on the product
path loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle.c -> liboracle.so (always recompiles); returns the path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    # -ffp-contract=off: no fused multiply-add, so each product and sum is
    # rounded once in double, in the order the source writes.
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
