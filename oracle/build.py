"""Builds the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is compiled with -O2 -ffp-contract=off and no
fast-math so that every fp32 operation is a single IEEE-rounded operation in
the order the source states, and nearbyintf rounds half to even.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
