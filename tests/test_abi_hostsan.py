"""The host-side C ABI tests (tests/test_abi_host.py: validation, memory
accounting, error paths; no call reaches a GPU) run again against a build of
the library with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code, in a child process that preloads the sanitizer runtime.  Any report
aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_address_and_ub_sanitizers():
    sys.path.insert(0, ROOT)
    from hierarchical_autoregressive_lm_amd import build as b
    rt = b.sanitizer_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime next to hipcc")
    if not os.path.exists(b.SAN_OUT):
        b.build_hostsan()
    env = dict(os.environ, PHOTON_LIB=b.SAN_OUT, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
