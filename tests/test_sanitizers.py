"""The oracle's pins once more, against an AddressSanitizer + UndefinedBehavior
Sanitizer build of the oracle (host code only; any report aborts the run).

Out-of-bounds reads or writes in the oracle's loops, and undefined behaviour
such as signed overflow in its index arithmetic (a hist_len near INT32_MAX,
for instance), end the subprocess with a sanitizer report instead of passing
silently.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(os.environ.get("KDA_ORACLE_LIB") is not None,
                    reason="already running under the sanitizer build")
def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's libasan runtime is not installed")
    lib = oracle.build(force=True, sanitize=True)
    env = dict(os.environ)
    env.update(KDA_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report is written to fd 2 as the process ends, which
    # pytest's own capture would swallow
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:]).strip()
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and \
        "runtime error" not in r.stderr, tail
