"""The C-ABI checks of test_abi.py, run against a host-sanitizer build.

The library's host code (argument validation, plan arithmetic, workspace
layout, status strings) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (structured_attention_video_amd/build.py,
build_hostsan) and test_abi.py runs in a child process that preloads the
clang ASan runtime and loads that build. Any out-of-bounds access, use after
free or undefined behaviour on those paths aborts the child with a report.
No GPU is used: every case stops before a launch.
"""
import os
import subprocess
import sys

import pytest

from structured_attention_video_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(os.environ.get("MONARCH_HOSTSAN") == "1", reason="inside the sanitized run itself")
def test_abi_checks_under_host_sanitizers():
    build.build_hostsan(jobs=min(8, os.cpu_count() or 1), verbose=False)
    env = dict(os.environ,
               LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               MONARCH_HOSTSAN="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "hostsan library mapped: True" in out, out[-2000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
