"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
runs every pin without a report: no out-of-bounds access, use after free,
signed overflow, bad shift or misaligned access on the paths the pins take
(every entry point of the oracle, at tiny and ragged shapes).  The
sanitized library is loaded into a fresh Python process started with
libasan preloaded; any report aborts that process and fails this test."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name: str) -> str:
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else ""


def test_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.build(oracle.LIB_SANITIZED, sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ORACLE_SANITIZE="1", OMP_NUM_THREADS="2",
               # CPython's own allocations are not freed at exit: leak checks off
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, f"sanitized oracle run failed:\n{tail}"
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error:" not in res.stderr, tail
    assert " passed" in res.stdout, tail
