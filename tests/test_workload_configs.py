"""The five workload cases live in workloads/configs/<name>.json (shapes, seeds
and knobs); the loader takes every field from the file and rejects missing or
unknown ones (no GPU needed)."""
import json
import os

import pytest

from workloads.specs import CONFIG_DIR, WORKLOADS, load_workload


def test_each_file_names_its_case_and_the_five_cases_are_present():
    files = sorted(f for f in os.listdir(CONFIG_DIR) if f.endswith(".json"))
    assert [os.path.splitext(f)[0] for f in files] == sorted(WORKLOADS)
    assert sorted(WORKLOADS) == ["long-65k", "qwen3-4b-1l", "qwen3-4b-36l", "r1-llama-8b", "tiny-f32"]
    for f in files:
        assert load_workload(os.path.join(CONFIG_DIR, f)).name == os.path.splitext(f)[0]


def test_shapes_are_ones_the_library_accepts():
    for w in WORKLOADS.values():
        assert w.dtype in ("bf16", "f32") and w.head_dim in (64, 128)
        assert w.n_q_heads % w.n_kv_heads == 0
        assert 0 < w.len_lo <= w.len_hi
        assert w.budget == 0 or w.n_prefix + w.n_recent <= w.budget <= w.len_lo
        assert w.n_obs > 0 and w.n_recent_q <= w.n_obs
        assert w.fps_cap == 0 or 0 < w.fps_keep <= w.fps_cap


def test_loader_rejects_missing_and_unknown_fields(tmp_path):
    d = json.load(open(os.path.join(CONFIG_DIR, "tiny-f32.json")))
    bad = dict(d, surplus=1)
    p = tmp_path / "x.json"
    p.write_text(json.dumps(bad))
    with pytest.raises(ValueError, match="unknown fields"):
        load_workload(str(p))
    del d["seed_base"]
    p.write_text(json.dumps(d))
    with pytest.raises(ValueError, match="missing fields"):
        load_workload(str(p))
