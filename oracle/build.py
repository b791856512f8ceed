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

# The sanitizer build (a test runs the oracle's tests against it): gcc's AddressSanitizer and
# UndefinedBehaviorSanitizer, any finding fatal. CPU code only.
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    out = out or LIB
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
