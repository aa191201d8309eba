"""The host side of the library (argument validation, workspace planning,
the entry points' error paths) under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with host instrumentation
and tests/test_abi.py runs against it in a child process with the ASan
runtime preloaded. No GPU is needed; any sanitizer report aborts the child."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

from sparse_top_kl_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_abi_suite_under_asan_and_ubsan():
    lib = build.build(sanitize=True)
    env = dict(os.environ,
               FKL_LIBRARY=lib,
               LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in res.stdout
