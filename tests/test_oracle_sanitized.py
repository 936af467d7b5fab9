"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The whole pin suite (tests/test_oracle_pins.py) runs again in a child process
against a build of oracle/attn_oracle.c instrumented with
-fsanitize=address,undefined, where any out-of-bounds read or write, use after
free or undefined operation aborts the process. The sanitizer runtimes are
gcc's own; the child preloads the ASan runtime, which must come first.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        path = subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_oracle_pins_under_address_and_undefined_sanitizers():
    lib = oracle.build_sanitized()
    env = dict(os.environ)
    env.update({
        "ORACLE_LIB": lib,
        "LD_PRELOAD": _runtime("libasan.so"),
        # Python and torch are not instrumented and keep some memory to the
        # end: leak reports would be about them, not about the oracle.
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join("tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, "sanitized pin run failed:\n" + tail
    assert " passed" in tail and "ERROR" not in tail, tail
