"""The bounds-checked build of the library (libkvevict_debug.so, every source
compiled with -DKVE_DEBUG): on the CPU it loads and passes the ABI tests; on
the GPU the parity suites of the select, compact, in-place and one-call
trigger kernels run against it in a child process, and every test must leave
the bounds-check flags at zero (tests/conftest.py checks them after each)."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GPU_FILES = ["tests/test_gpu_parity.py", "tests/test_gpu_inplace.py", "tests/test_gpu_step.py",
             "tests/test_gpu_budget_step.py", "tests/test_gpu_variants.py", "tests/test_gpu_graph.py"]


def _debug_lib():
    from decode_kv_cache_evict_amd import build as b
    return b.DEBUG_LIB


def _run(marker, files, timeout):
    env = dict(os.environ, KVE_LIB=_debug_lib())
    return subprocess.run([sys.executable, "-u", "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", marker,
                           *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def test_debug_library_loads_and_checks_arguments():
    if not os.path.exists(_debug_lib()):
        pytest.skip("the bounds-checked library is not built (python -m decode_kv_cache_evict_amd.build --debug)")
    r = _run("not gpu", ["tests/test_abi.py", "tests/test_no_fallback.py"], 600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and " passed" in out, out[-4000:]


@pytest.mark.gpu
def test_kernel_indices_stay_inside_their_segments():
    assert os.path.exists(_debug_lib()), f"{_debug_lib()} is missing: python -m decode_kv_cache_evict_amd.build --debug"
    r = _run("gpu", GPU_FILES, 900)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0 and "bounds checks fired" not in out, out[-6000:]
    m = re.search(r"(\d+) passed", out)
    assert m and int(m.group(1)) >= 60, out[-2000:]
