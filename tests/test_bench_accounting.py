"""bench.py's host-side contract (no GPU): the algorithmic bytes it reports
for the benchmark workload, and its refusal of more than one GPU."""
import subprocess
import sys
import os

import bench
from workloads import get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_benchmark_workload_bytes():
    """36 layers x 16 requests x 8 KV heads, d = 128, 4096 -> 3584: K 4.83 GB
    read once, the kept V rows read and the output K/V/pos written once, the
    queries, positions and scores once: 17.96 GB per one-call trigger, 18.19 GB
    with the beacon FPS."""
    w = get_workload("qwen3-4b-36l")
    b = bench.step_bytes(w, "fused")
    S, n, keep, row = 36 * 16 * 8, 4096, 3584, 256
    assert b["score_k"] == S * n * row == 4_831_838_208
    assert b["fused_step"] == 17_959_071_744
    assert b["total"] == 18_185_564_160
    # the in-place form moves at most min(K, n - K) rows per segment
    assert b["inplace_moves"] == 2 * S * min(keep, n - keep) * (2 * row + 4)
    assert bench.step_bytes(w, "inplace")["total"] < b["total"]


def test_benchmark_definition_bytes():
    """The benchmark definition's accounting of one trigger: K read once for
    scoring (4.832 GB), queries (0.227 GB), scores written and read (0.151 GB),
    kept K/V read and written (16.911 GB), kept positions read and written
    (0.132 GB), FPS buffers (0.227 GB): 22.48 GB, 4.01 ms at 70 % of 8 TB/s."""
    w = get_workload("qwen3-4b-36l")
    b = bench.step_bytes(w, "fused")
    S, n, keep, row = 36 * 16 * 8, 4096, 3584, 256
    assert b["compact_kv"] == 4 * S * keep * row == 16_911_433_728
    assert abs(b["definition_step"] - 22.48e9) < 0.01e9
    assert abs(b["definition_step"] / (0.7 * 8e12) * 1e3 - 4.01) < 0.01


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
