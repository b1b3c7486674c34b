"""ctypes binding of libkvevict.so: argument marshalling only.

Every function here has the name of the C entry point it calls and turns
torch tensors into device pointers, the current HIP stream into a
``hipStream_t`` and C status codes into ``KveError``.  No arithmetic of the
eviction step happens in Python.  The library must have been built
(``python -m decode_kv_cache_evict_amd.build``); there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVE_LIB") or os.path.join(_HERE, "_lib", "libkvevict.so")

KVE_BF16, KVE_F32 = 0, 1
KVE_AGG_MAX, KVE_AGG_MEAN = 0, 1
KVE_EPIKV_Z, KVE_EPIKV_MEAN = 0, 1
STATUS = {0: "KVE_OK", 1: "KVE_EINVAL", 2: "KVE_ESHAPE", 3: "KVE_EALIAS", 4: "KVE_EBUDGET",
          5: "KVE_EWORKSPACE", 6: "KVE_EDEVICE"}
EXPORTS = ["kv_evict_score_workspace", "kv_evict_score", "kv_evict_budgets", "kv_evict_entropy_budgets",
           "kv_evict_wave_budgets",
           "kv_evict_select_workspace", "kv_evict_select_compact", "kv_evict_select_compact_inplace",
           "kv_evict_score_select_compact_workspace",
           "kv_evict_score_select_compact", "kv_evict_score_select_compact_noalloc",
           "kv_evict_score_select_compact_inplace_workspace",
           "kv_evict_score_select_compact_inplace", "kv_evict_score_budget_select_compact_workspace",
           "kv_evict_score_budget_select_compact", "beacon_fps_update",
           "epikv_workspace_size", "epikv_score", "skipkv_workspace_size", "skipkv_sentence_scores",
           "kv_decode_attention_workspace", "kv_decode_attention",
           "kv_rope_apply", "kve_set_test_overrides", "kve_debug_flags", "kve_debug_stamps", "kve_last_error",
           "kve_abi_version"]


class KveError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class KveCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_seg", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seg_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_rows", ctypes.c_int64), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("seg_off", ctypes.c_void_p), ("seg_len", ctypes.c_void_p)]


class KveObs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_pos", ctypes.c_void_p), ("n_obs", ctypes.c_void_p),
                ("n_q_heads", ctypes.c_int32), ("max_obs", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("causal", ctypes.c_int32), ("aggregate", ctypes.c_int32)]


_lib = None


def lib():
    """Load libkvevict.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m decode_kv_cache_evict_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, D, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                 ctypes.c_double, ctypes.c_float)
        CP, OP = ctypes.POINTER(KveCache), ctypes.POINTER(KveObs)
        sig = {
            "kv_evict_score_workspace": (SZ, [CP, OP]),
            "kv_evict_score": (I32, [CP, OP, P, P, P, SZ, P]),
            "kv_evict_budgets": (I32, [P, P, P, I32, I32, I32, P, P]),
            "kv_evict_entropy_budgets": (I32, [P, I32, P, P, I32, I32, I32, P, P]),
            "kv_evict_wave_budgets": (I32, [I32, D, D, I32, I32, P, P]),
            "kv_evict_select_workspace": (SZ, [CP, I32]),
            "kv_evict_select_compact": (I32, [CP, P, P, I64, P, I32, I32, I32, P, CP, P, SZ, P]),
            "kv_evict_select_compact_inplace": (I32, [CP, P, P, I64, P, I32, I32, I32, P, P]),
            "kv_evict_score_select_compact_workspace": (SZ, [CP, OP, CP, I32]),
            "kv_evict_score_select_compact": (I32, [CP, OP, P, P, I32, I32, I32, P, CP, P, SZ, P]),
            "kv_evict_score_select_compact_noalloc": (I32, [CP, OP, P, P, I32, I32, I32, P, CP, P]),
            "kv_evict_score_select_compact_inplace_workspace": (SZ, [CP, OP]),
            "kv_evict_score_select_compact_inplace": (I32, [CP, OP, P, P, I32, I32, I32, P, P, SZ, P]),
            "kv_evict_score_budget_select_compact_workspace": (SZ, [CP, OP, CP, I32, I32]),
            "kv_evict_score_budget_select_compact": (I32, [CP, OP, P, P, I32, P, I32, P, I32, I32, P, CP, P, SZ, P]),
            "beacon_fps_update": (I32, [P, P, P, P, I32, I32, I32, I32, I32, P, P]),
            "epikv_workspace_size": (SZ, [I32, I32]),
            "epikv_score": (I32, [P, P, I32, I32, I32, I32, F, I32, P, P, P, SZ, P]),
            "skipkv_workspace_size": (SZ, [I32, I32, I32]),
            "skipkv_sentence_scores": (I32, [P, I32, I32, I32, P, P, I32, F, P, P, P, P, SZ, P]),
            "kv_decode_attention_workspace": (SZ, [CP, I32]),
            "kv_decode_attention": (I32, [CP, P, I32, P, P, P, SZ, P]),
            "kv_rope_apply": (I32, [P, P, P, I64, I32, D, I32, P]),
            "kve_set_test_overrides": (I32, [I32, I32]),
            "kve_debug_flags": (I32, [ctypes.POINTER(ctypes.c_uint32)]),
            "kve_debug_stamps": (I32, [P, I64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
            "kve_last_error": (ctypes.c_char_p, []),
            "kve_abi_version": (I32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    """None: torch's current stream; an int: a raw hipStream_t (0 = null stream)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st):
    if st != 0:
        raise KveError(st, lib().kve_last_error().decode())


def dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KVE_BF16
    if t.dtype == torch.float32:
        return KVE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_cache(k, v, pos, seg_off, seg_len, n_kv_heads, max_seg_len):
    """kve_cache over torch tensors k/v [rows, d], pos [rows] i32, seg_off [S] i64, seg_len [S] i32."""
    c = KveCache()
    c.dtype = dtype_code(k)
    c.n_seg = int(seg_off.numel())
    c.n_kv_heads = int(n_kv_heads)
    c.head_dim = int(k.shape[-1])
    c.max_seg_len = int(max_seg_len)
    c.n_rows = int(k.shape[0])
    c.k, c.v, c.pos = k.data_ptr(), (v.data_ptr() if v is not None else None), pos.data_ptr()
    c.seg_off, c.seg_len = seg_off.data_ptr(), seg_len.data_ptr()
    c._keep = (k, v, pos, seg_off, seg_len)
    return c


def make_obs(q, q_pos, n_obs, rope_theta, causal=True, aggregate=KVE_AGG_MAX):
    """kve_obs over q [B, Hq, max_obs, d] (pre-RoPE), q_pos [B, max_obs] i32, n_obs [B] i32 or None.
    aggregate: KVE_AGG_MAX (0) or KVE_AGG_MEAN (1)."""
    o = KveObs()
    o.q, o.q_pos = q.data_ptr(), q_pos.data_ptr()
    o.n_obs = n_obs.data_ptr() if n_obs is not None else None
    o.n_q_heads, o.max_obs = int(q.shape[1]), int(q.shape[2])
    o.rope_theta, o.causal = float(rope_theta), int(bool(causal))
    o.aggregate = int(aggregate)
    o._keep = (q, q_pos, n_obs)
    return o


def _ws(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)


def _aligned(buf):
    if buf is None:
        return None, 0
    p = buf.data_ptr()
    a = (p + 255) & ~255
    return ctypes.c_void_p(a), buf.numel() - (a - p)


def kv_evict_score_workspace(cache, obs):
    return int(lib().kv_evict_score_workspace(ctypes.byref(cache), ctypes.byref(obs)))


def kv_evict_score(cache, obs, scores, head_entropy=None, ws=None, stream=None):
    if ws is None:
        ws = _ws(kv_evict_score_workspace(cache, obs), scores.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_evict_score(ctypes.byref(cache), ctypes.byref(obs), _ptr(scores), _ptr(head_entropy),
                                wp, wn, _stream(stream)))


def kv_evict_budgets(weights, layer_total, cap, batch, n_heads, min_per_head, budget_out, stream=None):
    _check(lib().kv_evict_budgets(_ptr(weights), _ptr(layer_total), _ptr(cap), int(batch), int(n_heads),
                                  int(min_per_head), _ptr(budget_out), _stream(stream)))


def kv_evict_entropy_budgets(head_entropy, inverse, layer_total, cap, batch, n_heads, min_per_head, budget_out,
                             stream=None):
    _check(lib().kv_evict_entropy_budgets(_ptr(head_entropy), int(inverse), _ptr(layer_total), _ptr(cap), int(batch),
                                          int(n_heads), int(min_per_head), _ptr(budget_out), _stream(stream)))


def kv_evict_wave_budgets(n_layers, center, sigma, total, min_per_layer, out, stream=None):
    _check(lib().kv_evict_wave_budgets(int(n_layers), float(center), float(sigma), int(total),
                                       int(min_per_layer), _ptr(out), _stream(stream)))


def kv_evict_select_workspace(out_cache, have_kept_idx):
    return int(lib().kv_evict_select_workspace(ctypes.byref(out_cache), int(bool(have_kept_idx))))


def kv_evict_select_compact(cache_in, scores, budget, n_prefix, n_recent, cache_out, kept_idx=None,
                            score_off=None, uniform_budget=0, ws=None, stream=None):
    """budget: int32 tensor [n_seg] or None (then uniform_budget applies)."""
    if ws is None:
        ws = _ws(kv_evict_select_workspace(cache_out, kept_idx is not None), scores.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_evict_select_compact(ctypes.byref(cache_in), _ptr(scores), _ptr(score_off),
                                         int(scores.numel()), _ptr(budget), int(uniform_budget), int(n_prefix),
                                         int(n_recent), _ptr(kept_idx), ctypes.byref(cache_out), wp, wn,
                                         _stream(stream)))


def kv_evict_select_compact_inplace(cache, scores, budget, n_prefix, n_recent, new_len, score_off=None,
                                    uniform_budget=0, stream=None):
    """Hole-filling compaction within `cache`; new_len int32 [n_seg] (may be the cache's seg_len tensor)."""
    _check(lib().kv_evict_select_compact_inplace(ctypes.byref(cache), _ptr(scores), _ptr(score_off),
                                                 int(scores.numel()), _ptr(budget), int(uniform_budget),
                                                 int(n_prefix), int(n_recent), _ptr(new_len), _stream(stream)))


def kv_evict_score_select_compact_workspace(cache_in, obs, cache_out, have_kept_idx):
    return int(lib().kv_evict_score_select_compact_workspace(ctypes.byref(cache_in), ctypes.byref(obs),
                                                             ctypes.byref(cache_out), int(bool(have_kept_idx))))


def kv_evict_score_select_compact(cache_in, obs, scores, budget, n_prefix, n_recent, cache_out, kept_idx=None,
                                  uniform_budget=0, ws=None, stream=None):
    """One trigger: score, protected top-K and gather in a single call (scores fp32 [n_rows] is written)."""
    if ws is None:
        ws = _ws(kv_evict_score_select_compact_workspace(cache_in, obs, cache_out, kept_idx is not None),
                 scores.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_evict_score_select_compact(ctypes.byref(cache_in), ctypes.byref(obs), _ptr(scores), _ptr(budget),
                                               int(uniform_budget), int(n_prefix), int(n_recent), _ptr(kept_idx),
                                               ctypes.byref(cache_out), wp, wn, _stream(stream)))


def kv_evict_score_select_compact_noalloc(cache_in, obs, scores, budget, n_prefix, n_recent, cache_out, kept_idx=None,
                                          uniform_budget=0, stream=None):
    """kv_evict_score_select_compact with the library's static scratch in place of a workspace."""
    _check(lib().kv_evict_score_select_compact_noalloc(ctypes.byref(cache_in), ctypes.byref(obs), _ptr(scores),
                                                       _ptr(budget), int(uniform_budget), int(n_prefix),
                                                       int(n_recent), _ptr(kept_idx), ctypes.byref(cache_out),
                                                       _stream(stream)))


def kv_evict_score_select_compact_inplace_workspace(cache, obs):
    return int(lib().kv_evict_score_select_compact_inplace_workspace(ctypes.byref(cache), ctypes.byref(obs)))


def kv_evict_score_select_compact_inplace(cache, obs, scores, budget, n_prefix, n_recent, new_len, uniform_budget=0,
                                          ws=None, stream=None):
    """One trigger compacted in place by hole filling; new_len int32 [n_seg] (may be the cache's seg_len)."""
    if ws is None:
        ws = _ws(kv_evict_score_select_compact_inplace_workspace(cache, obs), scores.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_evict_score_select_compact_inplace(ctypes.byref(cache), ctypes.byref(obs), _ptr(scores),
                                                       _ptr(budget), int(uniform_budget), int(n_prefix),
                                                       int(n_recent), _ptr(new_len), wp, wn, _stream(stream)))


def kv_evict_score_budget_select_compact_workspace(cache_in, obs, cache_out, have_kept_idx, have_budget_out):
    return int(lib().kv_evict_score_budget_select_compact_workspace(
        ctypes.byref(cache_in), ctypes.byref(obs), ctypes.byref(cache_out), int(bool(have_kept_idx)),
        int(bool(have_budget_out))))


def kv_evict_score_budget_select_compact(cache_in, obs, scores, head_entropy, layer_total, min_per_head, n_prefix,
                                         n_recent, cache_out, inverse=0, budget_out=None, kept_idx=None, ws=None,
                                         stream=None):
    """One trigger with entropy-driven head budgets: scores, head_entropy (fp32 [n_seg], written), the
    request-layer totals layer_total (int32 [n_seg / n_kv_heads]), budgets (budget_out, optional) and the
    compacted output cache."""
    if ws is None:
        ws = _ws(kv_evict_score_budget_select_compact_workspace(cache_in, obs, cache_out, kept_idx is not None,
                                                                budget_out is not None), scores.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_evict_score_budget_select_compact(
        ctypes.byref(cache_in), ctypes.byref(obs), _ptr(scores), _ptr(head_entropy), int(inverse), _ptr(layer_total),
        int(min_per_head), _ptr(budget_out), int(n_prefix), int(n_recent), _ptr(kept_idx), ctypes.byref(cache_out),
        wp, wn, _stream(stream)))


def beacon_fps_update(q_in, q_out, count_in, count_out, k_keep, picks=None, stream=None):
    """q_in/q_out [n_buf, cap, d]; counts [n_buf] int32 (may be the same tensors: in place)."""
    n_buf, cap, d = q_in.shape
    _check(lib().beacon_fps_update(_ptr(q_in), _ptr(q_out), _ptr(count_in), _ptr(count_out), int(n_buf), int(cap),
                                   int(k_keep), int(d), dtype_code(q_in), _ptr(picks), _stream(stream)))


def epikv_workspace_size(batch, T):
    return int(lib().epikv_workspace_size(int(batch), int(T)))


def epikv_score(h_a, h_b, window, eps, scores, g_out=None, ws=None, stream=None, form=KVE_EPIKV_Z):
    """h_a/h_b bf16 [B, T, d_model]; scores fp32 [B, T]; g_out optional fp32 [2, B, T];
    form: KVE_EPIKV_Z (0) or KVE_EPIKV_MEAN (1)."""
    B, T, D = h_a.shape
    if ws is None and g_out is None:
        ws = _ws(epikv_workspace_size(B, T), scores.device)
    wp, wn = _aligned(ws)
    _check(lib().epikv_score(_ptr(h_a), _ptr(h_b), int(B), int(T), int(D), int(window), float(eps), int(form),
                             _ptr(g_out), _ptr(scores), wp, wn, _stream(stream)))


def skipkv_workspace_size(batch, max_sent, d_model):
    return int(lib().skipkv_workspace_size(int(batch), int(max_sent), int(d_model)))


def skipkv_sentence_scores(h, starts, n_sent, tau, pss_max, token_scores, marks=None, ws=None, stream=None):
    """h bf16 [B, T, d_model]; starts int32 [B, max_sent + 1]; n_sent int32 [B];
    pss_max fp32 [B, max_sent]; token_scores fp32 [B, T]; marks optional int32 [B, max_sent]."""
    B, T, Dm = h.shape
    max_sent = int(starts.shape[1]) - 1
    if ws is None:
        ws = _ws(skipkv_workspace_size(B, max_sent, Dm), token_scores.device)
    wp, wn = _aligned(ws)
    _check(lib().skipkv_sentence_scores(_ptr(h), int(B), int(T), int(Dm), _ptr(starts), _ptr(n_sent), max_sent,
                                        float(tau), _ptr(pss_max), _ptr(marks), _ptr(token_scores), wp, wn,
                                        _stream(stream)))


def kv_decode_attention_workspace(cache, n_q_heads):
    return int(lib().kv_decode_attention_workspace(ctypes.byref(cache), int(n_q_heads)))


def kv_decode_attention(cache, q, out, lse=None, ws=None, stream=None):
    """q [B, Hq, d] rotated (cache dtype); out fp32 [B, Hq, d]; lse optional fp32 [B, Hq]."""
    n_q = int(q.shape[1])
    if ws is None:
        ws = _ws(kv_decode_attention_workspace(cache, n_q), out.device)
    wp, wn = _aligned(ws)
    _check(lib().kv_decode_attention(ctypes.byref(cache), _ptr(q), n_q, _ptr(out), _ptr(lse), wp, wn,
                                     _stream(stream)))


def kv_rope_apply(src, dst, pos, rope_theta, stream=None):
    """src fp32 [rows, d] pre-RoPE -> dst (bf16 or fp32) [rows, d] rotated to pos [rows]."""
    _check(lib().kv_rope_apply(_ptr(src), _ptr(dst), _ptr(pos), int(src.shape[0]), int(src.shape[1]),
                               float(rope_theta), dtype_code(dst), _stream(stream)))


def kve_abi_version():
    return int(lib().kve_abi_version())


def kve_debug_flags():
    """Bounds-check flags of a KVE_DEBUG build since the last call (cleared);
    raises KveError on a regular build."""
    f = ctypes.c_uint32(0)
    _check(lib().kve_debug_flags(ctypes.byref(f)))
    return int(f.value)


def kve_debug_stamps(max_items=1 << 16):
    """Phase stamps of a KVE_STAMPS build since the last call (cleared):
    (uint64 array [rows, 9], ticks per microsecond); raises KveError on other builds."""
    import numpy as np
    buf = np.zeros((max_items, 9), dtype=np.uint64)
    n, tpu = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().kve_debug_stamps(buf.ctypes.data, int(max_items), ctypes.byref(n), ctypes.byref(tpu)))
    return buf[:n.value], tpu.value


SCORE_IMPLS = {"default": 0, "valu": 1, "fused": 2}


def kve_set_test_overrides(score_impl="default", spin_limit=0):
    """Test hook (process-wide): the scoring kernels to force ("default",
    "valu" or "fused") and the meetings' poll bound (0 = the default)."""
    _check(lib().kve_set_test_overrides(SCORE_IMPLS[score_impl], int(spin_limit)))
