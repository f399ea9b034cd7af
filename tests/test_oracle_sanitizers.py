"""The oracle's own pins, run once more with the oracle built under
AddressSanitizer and UndefinedBehaviorSanitizer (liboracle_san.so): any
out-of-bounds access, use after free or undefined behaviour in oracle.cpp
aborts the run. The sanitizer runtimes are preloaded into a child Python
that runs the oracle test files (CPU only; no GPU code is involved)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    oracle.build(sanitize=True)
    files = sorted(os.path.join(TESTS, f) for f in os.listdir(TESTS)
                   if f.startswith("test_oracle_") and f.endswith(".py")
                   and f != os.path.basename(__file__))
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    check = ("import oracle, sys; oracle._load(); "
             "assert oracle._lib._name.endswith('liboracle_san.so'), oracle._lib._name")
    subprocess.run([sys.executable, "-c", check], env=env, cwd=ROOT, check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=1500)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
