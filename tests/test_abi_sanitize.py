"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): tests/abi_sanitize/abi_fuzz, built by __graft_entry__.build() (or
python tests/abi_sanitize/build_check.py), calls every entry point on edge-value
problems with stand-in kernel launchers and checks statuses and workspace
layout; any memory error or undefined behaviour aborts it."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "io_aware_exact_fwd_amd", "_build", "abi_fuzz")


@pytest.mark.skipif(not os.path.exists(BIN), reason="abi_fuzz not built (run __graft_entry__.build())")
def test_abi_host_code_under_sanitizers():
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([BIN, "1000000"], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failures" in r.stdout
