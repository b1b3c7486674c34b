"""The C-ABI layer under host AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): api.cpp is rebuilt with both, linked with the regular kernel
objects, and the ABI tests (host validation of every entry point, symbol
exports, the test hook) and the no-fallback tests run against it in a child
process with the sanitizer runtime preloaded; any report aborts that run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan_and_ubsan():
    from decode_kv_cache_evict_amd import build as b
    if not all(os.path.exists(os.path.join(b.LIBDIR, os.path.splitext(s)[0] + ".o")) for s in b.SOURCES):
        pytest.skip("the library is not built (python -m decode_kv_cache_evict_amd.build)")
    lib = b.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=b.sanitizer_runtime(), KVE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_no_fallback.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
