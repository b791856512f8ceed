"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is built a second time with its host side instrumented (build.py, sanitize=True:
clang's -fsanitize=address,undefined on the host compilation only, no recovery), and the C-ABI
tests (tests/test_abi.py: every entry point's argument checks, which run on the host and return
before any launch) run against that build in a child process, with clang's ASan runtime first in
its preload list and leak detection off for the interpreter. An out-of-bounds access, a use
after free or undefined behaviour in the checks aborts the child; the test requires a clean exit.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clang_asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "*",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "*",
                                         "libclang_rt.asan.so")))
    return hits[-1] if hits else None


def test_abi_checks_pass_under_sanitizers(tmp_path):
    runtime = _clang_asan_runtime()
    if runtime is None or shutil.which("hipcc") is None and not os.path.exists(
            os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")):
        pytest.skip("needs hipcc and clang's ASan runtime")
    sys.path.insert(0, ROOT)
    from combine_ep_layout_06_amd import build as Bld
    lib = Bld.build(str(tmp_path / "libep_mi355x_sanitized.so"), sanitize=True)
    env = dict(os.environ)
    env.update(EP_MI355X_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
