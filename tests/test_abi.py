"""The C-ABI library loads, exports every declared entry point and rejects
bad arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

import decode_kv_cache_evict_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvevict.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(\w+)\(", src, flags=re.M)) - {"if", "while"})


def test_header_and_binding_agree():
    assert sorted(kv.EXPORTS) == _declared()


def test_every_declared_symbol_is_exported():
    L = kv.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert kv.kve_abi_version() == 2


def _fail(fn, *args):
    st = fn(*args)
    return st, kv.lib().kve_last_error().decode()


def test_host_validation_without_gpu():
    L = kv.lib()
    c = kv.KveCache(dtype=0, n_seg=8, n_kv_heads=8, head_dim=128, max_seg_len=64, n_rows=512,
                    k=0x1000, v=0x2000, pos=0x3000, seg_off=0x4000, seg_len=0x5000)
    o = kv.KveObs(q=0x6000, q_pos=0x7000, n_obs=None, n_q_heads=32, max_obs=48, rope_theta=1e6, causal=1)
    bad = kv.KveCache(**{f: getattr(c, f) for f, _ in kv.KveCache._fields_})
    bad.head_dim = 96
    st, msg = _fail(L.kv_evict_score, ctypes.byref(bad), ctypes.byref(o), 0x8000, None, None, 0, None)
    assert st == 2 and "head_dim" in msg
    o2 = kv.KveObs(q=0x6000, q_pos=0x7000, n_obs=None, n_q_heads=30, max_obs=48, rope_theta=1e6, causal=1)
    assert _fail(L.kv_evict_score, ctypes.byref(c), ctypes.byref(o2), 0x8000, None, None, 0, None)[0] == 2
    o3 = kv.KveObs(q=0x6000, q_pos=0x7000, n_obs=None, n_q_heads=32, max_obs=80, rope_theta=1e6, causal=1)
    assert _fail(L.kv_evict_score, ctypes.byref(c), ctypes.byref(o3), 0x8000, None, None, 0, None)[0] == 2
    need = L.kv_evict_score_workspace(ctypes.byref(c), ctypes.byref(o))
    assert need > 0
    st, msg = _fail(L.kv_evict_score, ctypes.byref(c), ctypes.byref(o), 0x8000, None, 0x100000, need - 1, None)
    assert st == 5
    # uniform budget below prefix + recent
    out = kv.KveCache(**{f: getattr(c, f) for f, _ in kv.KveCache._fields_})
    out.k, out.v, out.pos, out.seg_off, out.seg_len = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    st, msg = _fail(L.kv_evict_select_compact, ctypes.byref(c), 0x8000, None, 512, None, 19, 4, 16, 0x60000,
                    ctypes.byref(out), None, 0, None)
    assert st == 4
    # output aliasing the input keys
    out.k = c.k
    st, msg = _fail(L.kv_evict_select_compact, ctypes.byref(c), 0x8000, None, 512, None, 40, 4, 16, 0x60000,
                    ctypes.byref(out), None, 0, None)
    assert st == 3
    # FPS shapes
    assert _fail(L.beacon_fps_update, 0x1000, 0x1000, 0x2000, 0x2000, 4, 65, 16, 128, 0, None, None)[0] == 2
    assert _fail(L.beacon_fps_update, 0x1000, 0x1010, 0x2000, 0x3000, 4, 32, 16, 128, 0, None, None)[0] == 3
    # EPIKV shapes
    assert _fail(L.epikv_score, 0x1000, 0x2000, 2, 10, 4000, 256, 1e-6, 0, None, 0x3000, 0x4000, 1 << 20, None)[0] == 2
    assert _fail(L.epikv_score, 0x1000, 0x2000, 2, 10, 4096, 0, 1e-6, 0, None, 0x3000, 0x4000, 1 << 20, None)[0] == 2
    # budgets
    assert _fail(L.kv_evict_budgets, 0x1000, 0x2000, 0x3000, 4, 65, 64, 0x4000, None)[0] == 2
    assert _fail(L.kv_evict_wave_budgets, 32, 16.0, 6.0, 100, 64, 0x1000, None)[0] == 2
    # variant flags outside their enums
    o4 = kv.KveObs(q=0x6000, q_pos=0x7000, n_obs=None, n_q_heads=32, max_obs=48, rope_theta=1e6, causal=1,
                   aggregate=2)
    st, msg = _fail(L.kv_evict_score, ctypes.byref(c), ctypes.byref(o4), 0x8000, None, None, 0, None)
    assert st == 1 and "aggregate" in msg
    assert _fail(L.epikv_score, 0x1000, 0x2000, 2, 10, 4096, 256, 1e-6, 2, None, 0x3000, 0x4000, 1 << 20,
                 None)[0] == 1
    assert _fail(L.kv_evict_entropy_budgets, 0x1000, 2, 0x2000, 0x3000, 4, 8, 64, 0x4000, None)[0] == 1
    assert _fail(L.kv_evict_entropy_budgets, 0x1000, 1, 0x2000, 0x3000, 4, 65, 64, 0x4000, None)[0] == 2
    assert _fail(L.kv_rope_apply, 0x1000, 0x1000, 0x2000, 4, 128, 1e4, 0, None)[0] == 3
    # one-call entropy-budget trigger: direction flag, missing entropies, output capacity
    outb = kv.KveCache(**{f: getattr(out, f) for f, _ in kv.KveCache._fields_})
    outb.k, outb.max_seg_len = 0x10000, 64
    bw = L.kv_evict_score_budget_select_compact_workspace(ctypes.byref(c), ctypes.byref(o), ctypes.byref(outb), 1, 1)
    assert bw > 0
    args = lambda inv, ent, ob: (ctypes.byref(c), ctypes.byref(o), 0x8000, ent, inv, 0x9000, 64, None, 4, 16,  # noqa: E731
                                 0xA000, ctypes.byref(ob), 0x100000, bw, None)
    assert _fail(L.kv_evict_score_budget_select_compact, *args(2, 0x8800, outb))[0] == 1
    assert _fail(L.kv_evict_score_budget_select_compact, *args(0, None, outb))[0] == 1
    outs = kv.KveCache(**{f: getattr(outb, f) for f, _ in kv.KveCache._fields_})
    outs.max_seg_len = 63
    assert _fail(L.kv_evict_score_budget_select_compact, *args(0, 0x8800, outs))[0] == 4


def test_test_overrides_validate_and_reset():
    L = kv.lib()
    assert _fail(L.kve_set_test_overrides, 3, 0)[0] == 1
    assert _fail(L.kve_set_test_overrides, 0, -1)[0] == 1
    assert _fail(L.kve_set_test_overrides, 0, (1 << 30) + 1)[0] == 1
    assert L.kve_set_test_overrides(2, 5) == 0
    assert L.kve_set_test_overrides(0, 0) == 0


def test_debug_flags_call_outside_a_debug_build():
    if os.path.basename(kv.LIB_PATH) == "libkvevict_debug.so":
        pytest.skip("run against the bounds-checked library")
    L = kv.lib()
    assert _fail(L.kve_debug_flags, None)[0] == 1
    f = ctypes.c_uint32(7)
    st, msg = _fail(L.kve_debug_flags, ctypes.byref(f))
    assert st == 1 and "not a KVE_DEBUG build" in msg and f.value == 0


def test_stamps_call_outside_a_stamps_build():
    if os.path.basename(kv.LIB_PATH) == "libkvevict_stamps.so":
        pytest.skip("run against the phase-stamping library")
    L = kv.lib()
    n, tpu = ctypes.c_int64(5), ctypes.c_double(1.0)
    buf = (ctypes.c_uint64 * 9)()
    assert _fail(L.kve_debug_stamps, None, 1, ctypes.byref(n), ctypes.byref(tpu))[0] == 1
    assert _fail(L.kve_debug_stamps, buf, -1, ctypes.byref(n), ctypes.byref(tpu))[0] == 1
    st, msg = _fail(L.kve_debug_stamps, buf, 1, ctypes.byref(n), ctypes.byref(tpu))
    assert st == 1 and "not a KVE_STAMPS build" in msg and n.value == 0


def test_score_outputs_must_not_overlap_inputs_or_each_other():
    """kv_evict_score rejects, before any launch, scores, head_entropy or a
    workspace that overlaps an input (keys, positions, segment table, queries,
    query positions) or another output."""
    L = kv.lib()
    c = kv.KveCache(dtype=0, n_seg=8, n_kv_heads=8, head_dim=128, max_seg_len=64, n_rows=512,
                    k=0x100000, v=0x200000, pos=0x300000, seg_off=0x400000, seg_len=0x500000)
    o = kv.KveObs(q=0x600000, q_pos=0x700000, n_obs=None, n_q_heads=32, max_obs=48, rope_theta=1e6, causal=1)
    need = L.kv_evict_score_workspace(ctypes.byref(c), ctypes.byref(o))
    ws = 0x10000000
    call = lambda sc, ent, w: L.kv_evict_score(ctypes.byref(c), ctypes.byref(o), sc, ent, w, need, None)  # noqa: E731
    for sc, ent, w in ((0x500000, None, ws),          # scores over the segment lengths
                       (0x800000, 0x600100, ws),      # head_entropy inside the queries
                       (0x800000, None, 0x700000),    # workspace over the query positions
                       (0x800000, 0x800400, ws),      # head_entropy inside the scores
                       (0x800000, None, 0x300000)):   # workspace over the key positions
        st = call(sc, ent, w)
        assert st == 3, (hex(sc), ent, hex(w), st, L.kve_last_error().decode())
