"""The oracle's pins, run again against a build of the oracle under
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts the run),
in a child process with the ASan runtime preloaded (CPU only)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_ubsan():
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for g++")
    import oracle
    san = oracle.build(sanitize=True)
    env = dict(os.environ)
    env.update(ORACLE_LIB=san, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
