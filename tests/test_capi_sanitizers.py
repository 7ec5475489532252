"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/asan/capi_check.cpp drives configuration checks, plane and workspace
sizing over many configurations and every argument error of the C ABI
(none of which reaches the GPU), built by the library build with the
sanitizers on the host side only."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_BIN = os.path.join(ROOT, "_build", "kvq_capi_asan")   # written by the library build


def test_capi_host_code_is_sanitizer_clean():
    if not os.path.exists(SAN_BIN):
        pytest.skip("sanitizer check not built (python -m decode_attention_rotate_amd.build)")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([SAN_BIN], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
