"""The oracle's CPU pins under AddressSanitizer and UndefinedBehaviorSanitizer: kda_oracle.c is
built a second time with -fsanitize=address,undefined (oracle/build.py build_sanitized) and
tests/test_oracle_pins.py runs against that build in a child process (libasan preloaded, any
report fails the run)."""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime()
    if asan is None:
        pytest.skip("gcc's libasan runtime not found")
    lib = oracle_build.build_sanitized()
    env = dict(os.environ, KDA_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_backward.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in res.stdout, tail
