"""MI355X-native decode-time KV-cache eviction step.

The work runs in libkvevict.so (hand-written HIP for gfx950); this package is
its Python face: ``_abi`` marshals torch tensors into the C entry points.
"""
from ._abi import (  # noqa: F401
    KveError, KveCache, KveObs, lib, make_cache, make_obs,
    kv_evict_score_workspace, kv_evict_score, kv_evict_budgets, kv_evict_entropy_budgets, kv_evict_wave_budgets,
    kv_evict_select_workspace, kv_evict_select_compact, kv_evict_select_compact_inplace,
    kv_evict_score_select_compact_workspace,
    kv_evict_score_select_compact, kv_evict_score_select_compact_noalloc,
    kv_evict_score_select_compact_inplace_workspace,
    kv_evict_score_select_compact_inplace, kv_evict_score_budget_select_compact_workspace,
    kv_evict_score_budget_select_compact, beacon_fps_update,
    epikv_workspace_size, epikv_score, skipkv_workspace_size, skipkv_sentence_scores, kv_decode_attention_workspace, kv_decode_attention, kv_rope_apply,
    kve_abi_version, kve_set_test_overrides, kve_debug_flags, kve_debug_stamps, EXPORTS, LIB_PATH,
    KVE_AGG_MAX, KVE_AGG_MEAN, KVE_EPIKV_Z, KVE_EPIKV_MEAN,
)
