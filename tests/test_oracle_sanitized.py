"""The oracle's pins, run again against an AddressSanitizer + UndefinedBehavior
Sanitizer build of oracle/dlm_oracle.c (CPU only).

The oracle allocates scratch with malloc and runs threads across rows and
sequences; this run fails on any out-of-bounds access, use after free or
undefined behaviour (signed overflow, bad shifts, misaligned access) that the
pins reach.  It starts a child pytest over the oracle's own test files with
the sanitizer runtimes preloaded (the Python interpreter itself is not
instrumented) and DLM_ORACLE_SANITIZED=1, which makes the oracle package load
the sanitized library.  Leak checking is off: the interpreter's own
allocations outlive the run by design.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_stats.py", "tests/test_oracle_rules.py",
             "tests/test_oracle_next.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, sanitized=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{asan}:{ubsan}", DLM_ORACLE_SANITIZED="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized oracle run failed:\n{tail}"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and \
        "runtime error" not in r.stderr, tail
    print(r.stdout.strip().splitlines()[-1])
