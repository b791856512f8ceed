"""Build ep_c_client.so: the plain C client of libep_mi355x.so (gcc, HIP runtime, include/ep.h).

``python tests/c_abi/build.py`` (or ``build()``, which ``__graft_entry__.build()`` calls) links
against the built library, so build that first.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "combine_ep_layout_06_amd")
OUT = os.path.join(HERE, "ep_c_client.so")


def build(out: str = OUT, verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(rocm, 'include')}", os.path.join(HERE, "ep_c_client.c"),
           f"-L{PKG}", "-lep_mi355x", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../combine_ep_layout_06_amd",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"gcc failed ({res.returncode}) building {out}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
