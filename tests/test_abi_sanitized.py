"""The C ABI checks of test_abi.py, run against a host-sanitized libtq.

Argument validation, workspace sizing and the host codebook builder are
compiled with AddressSanitizer and UndefinedBehaviorSanitizer; any report
ends the child process with a non-zero status. CPU only (no kernel runs).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_checks_under_address_and_undefined_behaviour_sanitizers():
    from decode_tq_quantize_amd import build_sanitized as bs

    lib = bs.build_sanitized()
    env = dict(os.environ, TQ_LIBRARY=lib, LD_PRELOAD=bs.runtime_preload(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "libtq_san" in lib
