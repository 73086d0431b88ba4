"""The oracle's pins re-run against an AddressSanitizer + UndefinedBehavior
Sanitizer build of the oracle's C code (CPU only): every out-of-bounds
access, signed overflow, invalid shift or misaligned load in the oracle
aborts the child process and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_asan_ubsan():
    from oracle import build
    build.build(sanitize=True)
    rt = build.asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ, LD_PRELOAD=rt, TQ2_ORACLE_SANITIZED="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
