"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the host, no GPU:
the CPU oracle driven through every entry point (small inputs and rejected
arguments), and the C-ABI's host-side argument checks driven through every
exported function.  A planted out-of-bounds read in the oracle's driver shows
the instrumented build reports one."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "helpers"))
import build as helpers  # noqa: E402

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe, env=ENV):
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_oracle_under_address_and_ub_sanitizers():
    r = _run(helpers.build_sanitized_oracle())
    assert r.returncode == 0, r.stderr[-3000:]
    assert "clean" in r.stdout and "runtime error" not in r.stderr


def test_sanitizer_reports_a_planted_out_of_bounds_read():
    r = _run(helpers.build_sanitized_oracle(planted=True))
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr


def test_abi_host_checks_under_address_and_ub_sanitizers():
    # the HIP runtime keeps allocations until exit by design: leaks not checked
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    r = _run(helpers.build_sanitized_abi(), env)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "clean" in r.stdout and "runtime error" not in r.stderr
