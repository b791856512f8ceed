"""Build libep_mi355x.so: the gfx950 HIP kernels and their C ABI (include/ep.h).

``python -m combine_ep_layout_06_amd.build`` (or ``build()``) compiles every source under
``csrc/`` with hipcc for gfx950 into ``combine_ep_layout_06_amd/libep_mi355x.so``. Extra
``-D`` definitions (launch-shape overrides) can be passed with ``defines``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libep_mi355x.so"
LIB = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-command-line-argument",
    # no packed-fp32 instructions (v_pk_*_f32) in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out: str = LIB, defines: dict | None = None, verbose: bool = False) -> str:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}"]
    cmd += [f"-D{k}={v}" for k, v in (defines or {}).items()]
    cmd += [*sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {out}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
