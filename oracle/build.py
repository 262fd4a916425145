"""Build the CPU oracle (test infrastructure) with gcc.

Flags: -O2, no FMA contraction, OpenMP over output elements.  x86-64 uses SSE scalar
arithmetic, so every float/double operation in qv_oracle.c is one IEEE operation rounded
to nearest-even.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qv_oracle.c")
OUT = os.path.join(HERE, "libqv_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
