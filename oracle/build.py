"""Build the CPU oracle (``liboracle_ep.so``) with gcc.

Test infrastructure: the tests, the smoke check and the benchmark's CPU-baseline leg load the
result; the GPU library never does. Flags keep every fp32 operation a single IEEE operation:
no -ffast-math and no FMA contraction (the oracle calls ``fmaf`` where it means a fused
multiply-add).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "liboracle_ep.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


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
