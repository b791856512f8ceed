"""Build libep_mi355x.so: the gfx950 HIP kernels and their C ABI (include/ep.h).

``python -m combine_ep_layout_06_amd.build`` (or ``build()``) compiles every source under
``csrc/`` with hipcc for gfx950, one process per source in parallel, and links them into
``combine_ep_layout_06_amd/libep_mi355x.so``. Extra ``-D`` definitions (launch-shape overrides)
can be passed with ``defines`` (command line: ``-D EP_NAME=VALUE``, and ``--out`` for a variant
library elsewhere, which the binding loads when ``EP_MI355X_LIB`` names it).

The same compilation writes ``kernel_resources.json`` beside the library: per kernel (mangled
symbol), the compiler's own resource report (scalar and vector registers, spills, LDS, the
wavefronts per SIMD it allows), for recording beside measurements.

``build(out, sanitize=True)`` builds a library for checking the host code on the CPU: the host
side under AddressSanitizer and UndefinedBehaviorSanitizer (clang's runtime, which the process
that loads it must preload), the device side unoptimised to keep the build short. It is for the
host argument checks only and never launches a kernel that matters.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libep_mi355x.so"
LIB = os.path.join(PKG, LIB_NAME)
RESOURCES = os.path.join(PKG, "kernel_resources.json")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-command-line-argument",
    # no packed-fp32 instructions (v_pk_*_f32) in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# host code under ASan and UBSan, each flag for the host compilation only; device code at -O0
SANITIZE_FLAGS = [
    "-O1", "-Xarch_device", "-O0",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
]
SANITIZE_LINK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-shared-libasan"]

# the compiler's per-kernel resource remarks
_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]"
                     r"|Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill"
                     r"|LDS Size \[bytes/block\]):\s*(\S+)")
_KEYS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
         "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "waves_per_simd",
         "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
         "LDS Size [bytes/block]": "static_lds_bytes"}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def parse_resources(text: str) -> dict:
    """Kernel -> resource figures from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, obj: str, defines: dict | None, verbose: bool, sanitize: bool = False):
    cmd = [hipcc(), *HIPCC_FLAGS]
    cmd += SANITIZE_FLAGS if sanitize else ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [f"-I{INCLUDE}", f"-I{CSRC}"]
    cmd += [f"-D{k}={v}" for k, v in (defines or {}).items()]
    cmd += ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return src, res


def build(out: str = LIB, defines: dict | None = None, verbose: bool = False,
          sanitize: bool = False) -> str:
    if sanitize and os.path.abspath(out) == LIB:
        raise ValueError("a sanitized build goes elsewhere than the package's library")
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(os.path.dirname(out), "_build", os.path.basename(out) + ".obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in sources]
    jobs = max(1, min(len(sources), os.cpu_count() or 1, 16))
    resources = {}
    with cf.ThreadPoolExecutor(jobs) as pool:
        for src, res in pool.map(lambda a: _compile(*a, defines, verbose, sanitize),
                                 zip(sources, objs)):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed ({res.returncode}) on {src}")
            resources.update(parse_resources(res.stderr))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *(SANITIZE_LINK_FLAGS if sanitize else []), *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) linking {out}")
    os.replace(tmp, out)
    if out == LIB and not sanitize:
        with open(RESOURCES + ".tmp", "w") as f:
            json.dump({"arch": ARCH, "kernels": resources}, f, indent=1, sort_keys=True)
        os.replace(RESOURCES + ".tmp", RESOURCES)
    return out


def main(argv=None) -> int:
    import argparse
    ap = argparse.ArgumentParser(description="build the gfx950 library")
    ap.add_argument("--out", default=LIB, help="library path (default: the package's own)")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME=VALUE",
                    help="a launch-shape override, e.g. -D EP_FUSED_TT=16 (repeatable)")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    defines = {}
    for d in a.defines:
        name, sep, value = d.partition("=")
        if not re.fullmatch(r"EP_[A-Z0-9_]+", name) or not sep or not value:
            ap.error(f"-D {d}: expected EP_NAME=VALUE")
        defines[name] = value
    print(build(os.path.abspath(a.out), defines or None, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
