"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

ep_oracle.c is built with gcc's -fsanitize=address,undefined (oracle/build.py, sanitize=True)
and the oracle's own test files run against that build in a child process (EP_ORACLE_LIB selects
it; gcc's ASan runtime goes first in the child's preload list, leak detection off for the
interpreter). Any out-of-bounds access, use after free or undefined behaviour aborts the child
and leaves a sanitizer log; the test requires a clean exit and no log.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["test_oracle_layout.py", "test_oracle_dispatch_combine.py",
                "test_oracle_two_stage.py", "test_oracle_packed.py", "test_oracle_formats.py"]


def _asan_runtime():
    if not shutil.which("gcc"):
        return None
    res = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_tests_pass_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_ep_san.so"))
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    env["EP_ORACLE_LIB"] = lib
    # the binade sweeps call the same two encoders as the random-pattern tests, over tens of
    # millions of values: left out here to keep the instrumented run short
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           "-k", "not exhaustive_binades",
           *[os.path.join(ROOT, "tests", f) for f in ORACLE_TESTS]]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = ""
    for f in glob.glob(log + "*"):
        with open(f) as fh:
            reports += fh.read()[:4000]
    assert res.returncode == 0 and not reports, (
        f"exit {res.returncode}\n{res.stdout[-3000:]}\n{res.stderr[-2000:]}\n{reports}")
    assert " passed" in res.stdout
