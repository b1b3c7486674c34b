"""The instrumented builds of the library.  The bounds-checked build
(libkvevict_debug.so, every source compiled with -DKVE_DEBUG): on the CPU it
loads and passes the ABI tests; on the GPU the parity suites of the select,
compact, in-place and one-call trigger kernels, and the random-shape sweeps,
run against it in a child process, and every test must leave the bounds-check flags at zero
(tests/conftest.py checks them after each).  The phase-stamping build
(libkvevict_stamps.so, -DKVE_STAMPS): on the CPU it loads and passes the ABI
tests; on the GPU the benchmark's --stamps run reports every work-group item
of the one-call trigger with its phases in order."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GPU_FILES = ["tests/test_gpu_parity.py", "tests/test_gpu_inplace.py", "tests/test_gpu_step.py",
             "tests/test_gpu_budget_step.py", "tests/test_gpu_variants.py", "tests/test_gpu_graph.py",
             "tests/test_gpu_fullsize.py", "tests/test_gpu_random.py"]


def _debug_lib():
    from decode_kv_cache_evict_amd import build as b
    return b.DEBUG_LIB


def _stamps_lib():
    from decode_kv_cache_evict_amd import build as b
    return b.STAMPS_LIB


def _run(marker, files, timeout, lib=None):
    env = dict(os.environ, KVE_LIB=lib or _debug_lib())
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


def test_stamps_library_loads_and_checks_arguments():
    if not os.path.exists(_stamps_lib()):
        pytest.skip("the phase-stamping library is not built (python -m decode_kv_cache_evict_amd.build --stamps)")
    r = _run("not gpu", ["tests/test_abi.py", "tests/test_no_fallback.py"], 600, lib=_stamps_lib())
    out = r.stdout + r.stderr
    assert r.returncode == 0 and " passed" in out, out[-4000:]


@pytest.mark.gpu
@pytest.mark.parametrize("args,phases,segments", [
    (["--workload", "qwen3-4b-1l"], 8, 14 * 8),                                  # copying one-call trigger
    (["--workload", "r1-llama-8b"], 8, 32 * 10 * 8),                             # with entropy budgets
    (["--workload", "qwen3-4b-36l", "--call", "inplace"], 4, 36 * 16 * 8)])      # in place: phases 1-4 only
def test_phase_stamps_cover_every_work_group_item(args, phases, segments):
    import json
    assert os.path.exists(_stamps_lib()), f"{_stamps_lib()} is missing: python -m decode_kv_cache_evict_amd.build --stamps"
    env = dict(os.environ, KVE_LIB=_stamps_lib())
    r = subprocess.run([sys.executable, "-u", "bench.py", *args, "--stamps", "--no-cpu-baseline", "--steps", "1",
                        "--warmup", "1"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    ph = json.loads(r.stdout.strip().splitlines()[-1])["phase_us"]
    # every item of the launch stamped, at least one per segment, each phase in order
    assert ph["items"] == ph["of_items"] and ph["items"] >= segments
    assert len(ph["mean_us"]) == phases and all(v >= 0 for v in ph["mean_us"].values())
    assert 0 < ph["item_life_us"] <= ph["span_us"]
