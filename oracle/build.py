"""Build the oracle's C core (plain gcc, OpenMP, strict IEEE fp64).

Test infrastructure only; see ``oracle/__init__.py``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tp_oracle.c")
LIB = os.path.join(HERE, "libtporacle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off and no -ffast-math: every sum is the plain in-order
    # fp64 sum the source spells out. No -march: the library also runs on
    # other hosts.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
