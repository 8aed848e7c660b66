"""The host code of libpkv (planner, cost model, argument validation) under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/build_sanitized.py compiles planner.cpp, cost_model.cpp and
api.cpp with g++ -fsanitize=address,undefined (stub kernel launchers, no
device code).  This test runs the rest of the CPU suite in a child process
that loads that build through PKV_LIBRARY with the ASan runtime preloaded;
any sanitizer report aborts the child and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "sanitize"))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_cpu_suite_under_asan_and_ubsan():
    import build_sanitized

    lib = build_sanitized.build()
    asan = build_sanitized.asan_runtime()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("g++ has no ASan runtime")
    env = dict(os.environ, PKV_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run(
        # -s: a sanitizer report ends the child inside a test, so output
        # capture must not hold it back.
        [sys.executable, "-m", "pytest", "tests", "-q", "-s", "-m", "not gpu",
         "-p", "no:cacheprovider",
         "--ignore", os.path.join("tests", os.path.basename(__file__))],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
