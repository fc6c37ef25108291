"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every parity claim rests on the oracle, whose quantizer, dequantizer and
decoders index raw buffers in C.  This test builds an instrumented copy of
``oracle/nvfp4_oracle.c`` (``-fsanitize=address,undefined``, any finding
aborts) and runs the oracle pins (``tests/test_oracle_*.py``) against it in a
child process with gcc's ASan runtime preloaded.  A heap overflow, use of
uninitialised shift counts, signed overflow or a misaligned access in any
oracle path that the pins exercise fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return os.path.realpath(p) if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(600)
def test_oracle_pins_under_asan_ubsan():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's libasan runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, sanitize=True)
    pins = sorted(p for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                  if not p.endswith("test_oracle_sanitized.py"))
    env = dict(os.environ)
    env.update({"NVFP4_ORACLE_SANITIZE": "1", "LD_PRELOAD": asan,
                # CPython keeps objects alive at exit by design: leak reports
                # would be about the interpreter, not the oracle
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *pins], cwd=ROOT, env=env, capture_output=True, text=True, timeout=560)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
