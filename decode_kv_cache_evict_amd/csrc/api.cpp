// C ABI of the eviction-step library: argument checks, workspace carving and
// launches.  Every check runs on the host before anything is launched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.h"
#include "kvevict.h"

namespace {

thread_local std::string g_err;

kve_status fail(kve_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

kve_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVE_OK;
  return fail(KVE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_bytes(int32_t dtype) { return dtype == KVE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) overlap (empty ranges never do).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

kve_status check_cache(const kve_cache* c, const char* name, bool need_v) {
  if (!c) return fail(KVE_EINVAL, "%s: null cache", name);
  if (c->dtype != KVE_BF16 && c->dtype != KVE_F32) return fail(KVE_EINVAL, "%s: bad dtype %d", name, c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(KVE_ESHAPE, "%s: head_dim %d not 64/128", name, c->head_dim);
  if (c->n_kv_heads < 1 || c->n_seg < 0 || c->n_seg % c->n_kv_heads != 0 || c->n_seg > 65535)
    return fail(KVE_ESHAPE, "%s: n_seg %d / n_kv_heads %d", name, c->n_seg, c->n_kv_heads);
  if (c->max_seg_len < 0 || c->n_rows < 0) return fail(KVE_EINVAL, "%s: negative size", name);
  if (c->n_seg > 0 && (!c->k || !c->pos || !c->seg_off || !c->seg_len || (need_v && !c->v)))
    return fail(KVE_EINVAL, "%s: null pointer", name);
  if (!aligned16(c->k) || (need_v && !aligned16(c->v))) return fail(KVE_EINVAL, "%s: k/v not 16-byte aligned", name);
  return KVE_OK;
}

// Process-wide overrides set by kve_set_test_overrides (0: the default).
std::atomic<int32_t> g_score_impl{0}, g_spin_limit{0};

// Polls a single-read work-group makes at a segment barrier before it reports
// the segment failed (tests lower it to drive that path on purpose).
int32_t spin_limit() {
  const int32_t v = g_spin_limit.load(std::memory_order_relaxed);
  return v > 0 ? v : (1 << 22);
}

size_t rows_bytes(const kve_cache* c) { return size_t(c->n_rows) * c->head_dim * elem_bytes(c->dtype); }

// Scoring implementation for bf16 caches: two MFMA passes (default), the
// single-read MFMA kernel (2) or, for cross-checks, the plain VALU kernels (1).
int score_impl() { return g_score_impl.load(std::memory_order_relaxed); }

size_t valu_lds(int rows, int D, int dtype) {
  return size_t(rows) * D * elem_bytes(dtype) + size_t(rows) * (4 * sizeof(float2) + sizeof(float) + sizeof(int));
}

kve_status check_obs(const kve_cache* c, const kve_obs* o, int32_t* rows) {
  if (!o) return fail(KVE_EINVAL, "null obs");
  if (o->n_q_heads < c->n_kv_heads || o->n_q_heads % c->n_kv_heads != 0)
    return fail(KVE_ESHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", o->n_q_heads, c->n_kv_heads);
  if (o->max_obs < 1) return fail(KVE_ESHAPE, "max_obs %d", o->max_obs);
  const int64_t r = int64_t(o->n_q_heads / c->n_kv_heads) * o->max_obs;
  if (r > kve::kMaxObsRows) return fail(KVE_ESHAPE, "group*max_obs = %lld > %d", (long long)r, kve::kMaxObsRows);
  if (!(o->rope_theta > 0.0)) return fail(KVE_EINVAL, "rope_theta must be > 0");
  if (o->causal != 0 && o->causal != 1) return fail(KVE_EINVAL, "causal must be 0 or 1");
  if (o->aggregate != KVE_AGG_MAX && o->aggregate != KVE_AGG_MEAN) return fail(KVE_EINVAL, "aggregate must be 0 or 1");
  if (c->n_seg > 0 && (!o->q || !o->q_pos)) return fail(KVE_EINVAL, "null query pointers");
  if (!aligned16(o->q)) return fail(KVE_EINVAL, "queries not 16-byte aligned");
  *rows = int32_t(r);
  return KVE_OK;
}

kve::ScoreArgs score_args(const kve_cache* c, const kve_obs* o, int32_t rows, float* scores) {
  kve::ScoreArgs a{};
  a.k = c->k;
  a.pos = c->pos;
  a.seg_off = c->seg_off;
  a.seg_len = c->seg_len;
  a.n_rows = c->n_rows;
  a.n_seg = c->n_seg;
  a.n_kv = c->n_kv_heads;
  a.max_seg_len = c->max_seg_len;
  a.head_dim = c->head_dim;
  a.dtype = c->dtype;
  a.q = o->q;
  a.q_pos = o->q_pos;
  a.n_obs = o->n_obs;
  a.n_q = o->n_q_heads;
  a.max_obs = o->max_obs;
  a.group = o->n_q_heads / c->n_kv_heads;
  a.rows = rows;
  a.causal = o->causal;
  a.theta = o->rope_theta;
  a.aggregate = o->aggregate;
  a.scores = scores;
  a.spin_limit = spin_limit();
  return a;
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

size_t step_score_ws(const kve_cache* in, const kve_obs* o, int32_t rows) {
  return round256(kve::score_workspace_bytes(in->n_seg / in->n_kv_heads, o->n_q_heads, o->max_obs, in->head_dim,
                                             in->dtype, in->n_seg, in->max_seg_len, rows));
}

}  // namespace

extern "C" {

const char* kve_last_error(void) { return g_err.c_str(); }

kve_status kve_set_test_overrides(int32_t score_impl, int32_t spin_limit) {
  if (score_impl < 0 || score_impl > 2) return fail(KVE_EINVAL, "score_impl %d not 0, 1 or 2", score_impl);
  if (spin_limit < 0 || spin_limit > (1 << 30)) return fail(KVE_EINVAL, "spin_limit %d out of range", spin_limit);
  g_score_impl.store(score_impl, std::memory_order_relaxed);
  g_spin_limit.store(spin_limit, std::memory_order_relaxed);
  return KVE_OK;
}

kve_status kve_debug_flags(uint32_t* flags) {
  if (!flags) return fail(KVE_EINVAL, "flags is NULL");
#ifdef KVE_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return fail(KVE_EDEVICE, "kve_debug_flags: device synchronisation failed");
  const unsigned int a = kve::debug_take_score(), b = kve::debug_take_select();
  if (a == ~0u || b == ~0u) return fail(KVE_EDEVICE, "kve_debug_flags: flag words could not be read");
  *flags = a | b;
  return KVE_OK;
#else
  *flags = 0;
  return fail(KVE_EINVAL, "kve_debug_flags: not a KVE_DEBUG build");
#endif
}

kve_status kve_debug_stamps(uint64_t* stamps, int64_t max_items, int64_t* n_rows, double* ticks_per_us) {
  if (!stamps || !n_rows || !ticks_per_us || max_items < 0)
    return fail(KVE_EINVAL, "kve_debug_stamps: NULL pointer or negative max_items");
#ifdef KVE_STAMPS
  int dev = 0, khz = 0;
  if (hipDeviceSynchronize() != hipSuccess || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return fail(KVE_EDEVICE, "kve_debug_stamps: device synchronisation or clock query failed");
  static_assert(sizeof(unsigned long long) == sizeof(uint64_t), "64-bit stamps");
  const int64_t n = kve::debug_take_stamps(reinterpret_cast<unsigned long long*>(stamps), max_items);
  if (n < 0) return fail(KVE_EDEVICE, "kve_debug_stamps: stamps could not be copied");
  *n_rows = n;
  *ticks_per_us = double(khz) / 1000.0;
  return KVE_OK;
#else
  *n_rows = 0;
  *ticks_per_us = 0.0;
  return fail(KVE_EINVAL, "kve_debug_stamps: not a KVE_STAMPS build");
#endif
}

int32_t kve_abi_version(void) { return KVE_ABI_VERSION; }

size_t kv_evict_score_workspace(const kve_cache* c, const kve_obs* o) {
  int32_t rows = 0;
  if (check_cache(c, "cache", false) != KVE_OK || check_obs(c, o, &rows) != KVE_OK) return 0;
  return kve::score_workspace_bytes(c->n_seg / c->n_kv_heads, o->n_q_heads, o->max_obs, c->head_dim, c->dtype,
                                    c->n_seg, c->max_seg_len, rows);
}

kve_status kv_evict_score(const kve_cache* c, const kve_obs* o, float* scores, float* head_entropy, void* ws,
                          size_t ws_bytes, void* stream) {
  kve_status st = check_cache(c, "cache", false);
  if (st != KVE_OK) return st;
  int32_t rows = 0;
  if ((st = check_obs(c, o, &rows)) != KVE_OK) return st;
  if (c->n_seg > 0 && !scores) return fail(KVE_EINVAL, "null scores");
  const int impl = c->dtype == KVE_BF16 ? score_impl() : 1;
  if (impl == 1 && valu_lds(rows, c->head_dim, c->dtype) > 65536)
    return fail(KVE_ESHAPE, "rows*head_dim too large for the fp32 scoring path");
  const int batch = c->n_seg / c->n_kv_heads;
  const size_t need = kve::score_workspace_bytes(batch, o->n_q_heads, o->max_obs, c->head_dim, c->dtype, c->n_seg,
                                                 c->max_seg_len, rows);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(KVE_EWORKSPACE, "workspace not 256-byte aligned");
  const size_t ns = size_t(c->n_seg);
  const void* ins[] = {c->k, c->pos, c->seg_off, c->seg_len, o->q, o->q_pos, o->n_obs};
  const size_t insz[] = {rows_bytes(c), size_t(c->n_rows) * 4, ns * 8, ns * 4,
                         size_t(batch) * o->n_q_heads * o->max_obs * c->head_dim * elem_bytes(c->dtype),
                         size_t(batch) * o->max_obs * 4, o->n_obs ? size_t(batch) * 4 : 0};
  const void* outs[] = {scores, head_entropy, ws};
  const size_t outsz[] = {size_t(c->n_rows) * sizeof(float), head_entropy ? ns * 4 : 0, need};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (c->n_seg == 0) return KVE_OK;
  kve::ScoreArgs a = score_args(c, o, rows, scores);
  a.entropy = head_entropy;
  a.impl = impl;
  return device_status(kve::launch_score(a, ws, static_cast<hipStream_t>(stream)), "kv_evict_score");
}

kve_status kv_evict_budgets(const float* weights, const int32_t* layer_total, const int32_t* cap, int32_t batch,
                            int32_t n_heads, int32_t min_per_head, int32_t* budget_out, void* stream) {
  if (batch < 0 || min_per_head < 0) return fail(KVE_EINVAL, "negative batch or floor");
  if (n_heads < 1 || n_heads > 64) return fail(KVE_ESHAPE, "n_heads %d not in [1, 64]", n_heads);
  if (batch > 0 && (!weights || !layer_total || !cap || !budget_out)) return fail(KVE_EINVAL, "null pointer");
  const size_t nb = size_t(batch) * n_heads * 4;
  if (overlap(budget_out, nb, weights, nb) || overlap(budget_out, nb, cap, nb) ||
      overlap(budget_out, nb, layer_total, size_t(batch) * 4))
    return fail(KVE_EALIAS, "budget_out overlaps an input");
  return device_status(kve::launch_budgets(weights, layer_total, cap, batch, n_heads, min_per_head, budget_out,
                                           static_cast<hipStream_t>(stream)),
                       "kv_evict_budgets");
}

kve_status kv_evict_entropy_budgets(const float* head_entropy, int32_t inverse, const int32_t* layer_total,
                                    const int32_t* cap, int32_t batch, int32_t n_heads, int32_t min_per_head,
                                    int32_t* budget_out, void* stream) {
  if (inverse != 0 && inverse != 1) return fail(KVE_EINVAL, "inverse must be 0 or 1");
  if (batch < 0 || min_per_head < 0) return fail(KVE_EINVAL, "negative batch or floor");
  if (n_heads < 1 || n_heads > 64) return fail(KVE_ESHAPE, "n_heads %d not in [1, 64]", n_heads);
  if (batch > 0 && (!head_entropy || !layer_total || !cap || !budget_out)) return fail(KVE_EINVAL, "null pointer");
  const size_t nb = size_t(batch) * n_heads * 4;
  if (overlap(budget_out, nb, head_entropy, nb) || overlap(budget_out, nb, cap, nb) ||
      overlap(budget_out, nb, layer_total, size_t(batch) * 4))
    return fail(KVE_EALIAS, "budget_out overlaps an input");
  return device_status(kve::launch_budgets(head_entropy, layer_total, cap, batch, n_heads, min_per_head, budget_out,
                                           static_cast<hipStream_t>(stream), inverse),
                       "kv_evict_entropy_budgets");
}

kve_status kv_evict_wave_budgets(int32_t n_layers, double center, double sigma, int32_t total, int32_t min_per_layer,
                                 int32_t* out, void* stream) {
  if (!out) return fail(KVE_EINVAL, "null out");
  if (n_layers < 1 || n_layers > 64) return fail(KVE_ESHAPE, "n_layers %d not in [1, 64]", n_layers);
  if (!(sigma > 0.0) || min_per_layer < 0) return fail(KVE_EINVAL, "sigma must be > 0, floor >= 0");
  if (int64_t(total) < int64_t(n_layers) * min_per_layer)
    return fail(KVE_ESHAPE, "total %d below n_layers * floor", total);
  return device_status(
      kve::launch_wave_budgets(n_layers, center, sigma, total, min_per_layer, out, static_cast<hipStream_t>(stream)),
      "kv_evict_wave_budgets");
}

size_t kv_evict_select_workspace(const kve_cache* out, int32_t have_kept_idx) {
  if (!out || out->n_rows < 0 || out->n_seg < 0) return 0;
  // the kept-index list (when the caller passes none), then the control ints
  // of the several-work-groups-per-segment selection of few long segments
  const size_t kept = have_kept_idx ? 0 : round256(size_t(out->n_rows) * sizeof(int32_t));
  return kept + kve::split_ctl_ints(out->n_seg) * sizeof(int32_t);
}

kve_status kv_evict_select_compact(const kve_cache* in, const float* scores, const int64_t* score_off,
                                   int64_t n_scores, const int32_t* budget, int32_t uniform_budget, int32_t n_prefix,
                                   int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* ws, size_t ws_bytes,
                                   void* stream) {
  kve_status st = check_cache(in, "in", true);
  if (st != KVE_OK) return st;
  if ((st = check_cache(out, "out", true)) != KVE_OK) return st;
  if (in->dtype != out->dtype || in->head_dim != out->head_dim || in->n_seg != out->n_seg ||
      in->n_kv_heads != out->n_kv_heads)
    return fail(KVE_ESHAPE, "in/out cache shapes differ");
  if (n_prefix < 0 || n_recent < 0 || n_scores < 0) return fail(KVE_EINVAL, "negative prefix/recent/n_scores");
  if (in->n_seg > 0 && !scores) return fail(KVE_EINVAL, "null scores");
  if (!budget) {
    if (uniform_budget < n_prefix + n_recent)
      return fail(KVE_EBUDGET, "budget %d below prefix %d + recent %d", uniform_budget, n_prefix, n_recent);
    const int32_t most = uniform_budget < in->max_seg_len ? uniform_budget : in->max_seg_len;
    if (most > out->max_seg_len)
      return fail(KVE_EBUDGET, "budget %d exceeds the output capacity %d", most, out->max_seg_len);
  }
  const size_t need = kept_idx ? 0 : size_t(out->n_rows) * sizeof(int32_t);
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  int32_t* kept = kept_idx ? kept_idx : static_cast<int32_t*>(ws);
  // control ints of the split selection when the workspace holds them (a
  // smaller workspace only costs the one-work-group-per-segment form)
  const size_t ctl_at = kept_idx ? 0 : round256(need);
  const size_t ctl_b = kve::split_ctl_ints(in->n_seg) * sizeof(int32_t);
  int32_t* ctl = ws && ctl_b > 0 && ws_bytes >= ctl_at + ctl_b && (reinterpret_cast<uintptr_t>(ws) & 3u) == 0
                     ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ctl_at)
                     : nullptr;
  const size_t ib = rows_bytes(in), ob = rows_bytes(out);
  const size_t ipb = size_t(in->n_rows) * 4, opb = size_t(out->n_rows) * 4;
  const size_t kb = size_t(out->n_rows) * 4;
  const size_t sb = size_t(n_scores) * 4;
  const void* ins[] = {in->k, in->v, in->pos, scores, in->seg_off, in->seg_len, budget, score_off, out->seg_off};
  const size_t insz[] = {ib, ib, ipb, sb, size_t(in->n_seg) * 8, size_t(in->n_seg) * 4,
                         budget ? size_t(in->n_seg) * 4 : 0, score_off ? size_t(in->n_seg) * 8 : 0,
                         size_t(out->n_seg) * 8};
  const void* outs[] = {out->k, out->v, out->pos, out->seg_len, kept, ctl};
  const size_t outsz[] = {ob, ob, opb, size_t(out->n_seg) * 4, kb, ctl ? ctl_b : 0};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 9; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (in->n_seg == 0) return KVE_OK;
  kve::SelectArgs a{};
  a.k_in = in->k;
  a.v_in = in->v;
  a.pos_in = in->pos;
  a.in_off = in->seg_off;
  a.in_len = in->seg_len;
  a.in_rows = in->n_rows;
  a.in_max = in->max_seg_len;
  a.scores = scores;
  a.score_off = score_off;
  a.n_scores = n_scores;
  a.budget = budget;
  a.uniform_budget = uniform_budget;
  a.n_prefix = n_prefix;
  a.n_recent = n_recent;
  a.k_out = out->k;
  a.v_out = out->v;
  a.pos_out = out->pos;
  a.out_off = out->seg_off;
  a.out_len = out->seg_len;
  a.out_rows = out->n_rows;
  a.out_cap = out->max_seg_len;
  a.kept = kept;
  a.n_seg = in->n_seg;
  a.head_dim = in->head_dim;
  a.elem_bytes = int32_t(elem_bytes(in->dtype));
  a.split_ctl = ctl;
  a.spin_limit = spin_limit();
  return device_status(kve::launch_select_compact(a, static_cast<hipStream_t>(stream)), "kv_evict_select_compact");
}

kve_status kv_evict_select_compact_inplace(kve_cache* c, const float* scores, const int64_t* score_off,
                                           int64_t n_scores, const int32_t* budget, int32_t uniform_budget,
                                           int32_t n_prefix, int32_t n_recent, int32_t* new_len, void* stream) {
  kve_status st = check_cache(c, "cache", true);
  if (st != KVE_OK) return st;
  if (n_prefix < 0 || n_recent < 0 || n_scores < 0) return fail(KVE_EINVAL, "negative prefix/recent/n_scores");
  if (c->n_seg > 0 && (!scores || !new_len)) return fail(KVE_EINVAL, "null scores or new_len");
  if (!budget && uniform_budget < n_prefix + n_recent)
    return fail(KVE_EBUDGET, "budget %d below prefix %d + recent %d", uniform_budget, n_prefix, n_recent);
  const size_t rb = rows_bytes(c), pb = size_t(c->n_rows) * 4, ns = size_t(c->n_seg);
  const void* ins[] = {scores, c->seg_off, budget, score_off};
  const size_t insz[] = {size_t(n_scores) * 4, ns * 8, budget ? ns * 4 : 0, score_off ? ns * 8 : 0};
  const void* outs[] = {c->k, c->v, c->pos};
  const size_t outsz[] = {rb, rb, pb};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "cache array %d overlaps input %d", i, j);
  // new_len may be the cache's own seg_len (read before it is written, by the same work-group)
  if (new_len != c->seg_len) {
    const void* all[] = {c->k, c->v, c->pos, scores, c->seg_off, c->seg_len, budget, score_off};
    const size_t allsz[] = {rb, rb, pb, size_t(n_scores) * 4, ns * 8, ns * 4, budget ? ns * 4 : 0,
                            score_off ? ns * 8 : 0};
    for (int j = 0; j < 8; ++j)
      if (overlap(new_len, ns * 4, all[j], allsz[j])) return fail(KVE_EALIAS, "new_len overlaps argument %d", j);
  }
  if (c->n_seg == 0) return KVE_OK;
  kve::SelectArgs a{};
  a.k_in = c->k;
  a.v_in = c->v;
  a.pos_in = c->pos;
  a.in_off = c->seg_off;
  a.in_len = c->seg_len;
  a.in_rows = c->n_rows;
  a.in_max = c->max_seg_len;
  a.scores = scores;
  a.score_off = score_off;
  a.n_scores = n_scores;
  a.budget = budget;
  a.uniform_budget = uniform_budget;
  a.n_prefix = n_prefix;
  a.n_recent = n_recent;
  a.k_out = c->k;
  a.v_out = c->v;
  a.pos_out = c->pos;
  a.out_len = new_len;
  a.n_seg = c->n_seg;
  a.head_dim = c->head_dim;
  a.elem_bytes = int32_t(elem_bytes(c->dtype));
  return device_status(kve::launch_select_inplace(a, static_cast<hipStream_t>(stream)),
                       "kv_evict_select_compact_inplace");
}

size_t kv_evict_score_select_compact_workspace(const kve_cache* in, const kve_obs* o, const kve_cache* out,
                                               int32_t have_kept_idx) {
  int32_t rows = 0;
  if (check_cache(in, "in", true) != KVE_OK || check_obs(in, o, &rows) != KVE_OK || !out || out->n_rows < 0)
    return 0;
  return step_score_ws(in, o, rows) + (have_kept_idx ? 0 : size_t(out->n_rows) * sizeof(int32_t));
}

kve_status kv_evict_score_select_compact(const kve_cache* in, const kve_obs* o, float* scores,
                                         const int32_t* budget, int32_t uniform_budget, int32_t n_prefix,
                                         int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* ws,
                                         size_t ws_bytes, void* stream) {
  // every check of both halves runs before anything is launched
  kve_status st = check_cache(in, "in", true);
  if (st != KVE_OK) return st;
  if ((st = check_cache(out, "out", true)) != KVE_OK) return st;
  int32_t rows = 0;
  if ((st = check_obs(in, o, &rows)) != KVE_OK) return st;
  if (in->dtype != out->dtype || in->head_dim != out->head_dim || in->n_seg != out->n_seg ||
      in->n_kv_heads != out->n_kv_heads)
    return fail(KVE_ESHAPE, "in/out cache shapes differ");
  if (n_prefix < 0 || n_recent < 0) return fail(KVE_EINVAL, "negative prefix/recent");
  if (in->n_seg > 0 && !scores) return fail(KVE_EINVAL, "null scores");
  const bool fused = in->dtype == KVE_BF16 && score_impl() == 0 && in->max_seg_len > 0 &&
                     in->max_seg_len <= kve::step_max_seg(in->head_dim);
  const int impl = in->dtype == KVE_BF16 ? score_impl() : 1;
  if (!fused && impl == 1 && valu_lds(rows, in->head_dim, in->dtype) > 65536)
    return fail(KVE_ESHAPE, "rows*head_dim too large for the fp32 scoring path");
  if (!budget) {
    if (uniform_budget < n_prefix + n_recent)
      return fail(KVE_EBUDGET, "budget %d below prefix %d + recent %d", uniform_budget, n_prefix, n_recent);
    const int32_t most = uniform_budget < in->max_seg_len ? uniform_budget : in->max_seg_len;
    if (most > out->max_seg_len)
      return fail(KVE_EBUDGET, "budget %d exceeds the output capacity %d", most, out->max_seg_len);
  }
  const size_t sw = step_score_ws(in, o, rows);
  const size_t need = sw + (kept_idx ? 0 : size_t(out->n_rows) * sizeof(int32_t));
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(KVE_EWORKSPACE, "workspace not 256-byte aligned");
  int32_t* kept = kept_idx ? kept_idx : reinterpret_cast<int32_t*>(static_cast<char*>(ws) + sw);
  const int32_t batch = in->n_seg / in->n_kv_heads;
  const size_t ns = size_t(in->n_seg);
  const void* ins[] = {in->k, in->v, in->pos, in->seg_off, in->seg_len, o->q, o->q_pos, o->n_obs, budget,
                       out->seg_off};
  const size_t insz[] = {rows_bytes(in), rows_bytes(in), size_t(in->n_rows) * 4, ns * 8, ns * 4,
                         size_t(batch) * o->n_q_heads * o->max_obs * in->head_dim * elem_bytes(in->dtype),
                         size_t(batch) * o->max_obs * 4, size_t(batch) * 4, budget ? ns * 4 : 0, ns * 8};
  const void* outs[] = {scores, out->k, out->v, out->pos, out->seg_len, kept, ws};
  const size_t outsz[] = {size_t(in->n_rows) * 4, rows_bytes(out), rows_bytes(out), size_t(out->n_rows) * 4,
                          ns * 4, size_t(out->n_rows) * 4, sw};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 7; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (in->n_seg == 0) return KVE_OK;
  if (!fused) {
    if ((st = kv_evict_score(in, o, scores, nullptr, ws, sw, stream)) != KVE_OK) return st;
    // the scoring workspace is free again (stream order): the selection's control ints
    return kv_evict_select_compact(in, scores, nullptr, in->n_rows, budget, uniform_budget, n_prefix, n_recent, kept,
                                   out, ws, sw, stream);
  }
  kve::ScoreArgs a = score_args(in, o, rows, scores);
  a.v = in->v;
  a.k_out = out->k;
  a.v_out = out->v;
  a.pos_out = out->pos;
  a.out_off = out->seg_off;
  a.out_len = out->seg_len;
  a.out_rows = out->n_rows;
  a.out_cap = out->max_seg_len;
  a.kept = kept_idx;   // the fused kernel needs no index list of its own
  a.budget = budget;
  a.uniform_budget = uniform_budget;
  a.n_prefix = n_prefix;
  a.n_recent = n_recent;
  return device_status(kve::launch_score_select_compact(a, ws, static_cast<hipStream_t>(stream)),
                       "kv_evict_score_select_compact");
}

size_t kv_evict_score_budget_select_compact_workspace(const kve_cache* in, const kve_obs* o, const kve_cache* out,
                                                      int32_t have_kept_idx, int32_t have_budget_out) {
  int32_t rows = 0;
  if (check_cache(in, "in", true) != KVE_OK || check_obs(in, o, &rows) != KVE_OK || !out || out->n_rows < 0)
    return 0;
  return step_score_ws(in, o, rows) + (have_kept_idx ? 0 : round256(size_t(out->n_rows) * sizeof(int32_t))) +
         (have_budget_out ? 0 : round256(size_t(in->n_seg) * sizeof(int32_t)));
}

kve_status kv_evict_score_budget_select_compact(const kve_cache* in, const kve_obs* o, float* scores,
                                                float* head_entropy, int32_t inverse, const int32_t* layer_total,
                                                int32_t min_per_head, int32_t* budget_out, int32_t n_prefix,
                                                int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* ws,
                                                size_t ws_bytes, void* stream) {
  // every check of the three halves runs before anything is launched
  kve_status st = check_cache(in, "in", true);
  if (st != KVE_OK) return st;
  if ((st = check_cache(out, "out", true)) != KVE_OK) return st;
  int32_t rows = 0;
  if ((st = check_obs(in, o, &rows)) != KVE_OK) return st;
  if (in->dtype != out->dtype || in->head_dim != out->head_dim || in->n_seg != out->n_seg ||
      in->n_kv_heads != out->n_kv_heads)
    return fail(KVE_ESHAPE, "in/out cache shapes differ");
  if (inverse != 0 && inverse != 1) return fail(KVE_EINVAL, "inverse must be 0 or 1");
  if (n_prefix < 0 || n_recent < 0 || min_per_head < 0) return fail(KVE_EINVAL, "negative prefix/recent/floor");
  if (in->n_kv_heads > 64) return fail(KVE_ESHAPE, "n_kv_heads %d > 64", in->n_kv_heads);
  if (in->n_seg > 0 && (!scores || !head_entropy || !layer_total))
    return fail(KVE_EINVAL, "null scores, head_entropy or layer_total");
  if (in->max_seg_len > out->max_seg_len)
    return fail(KVE_EBUDGET, "output capacity %d below max_seg_len %d (a head may keep every row)",
                out->max_seg_len, in->max_seg_len);
  const bool fused = in->dtype == KVE_BF16 && score_impl() == 0 && in->max_seg_len > 0 &&
                     kve::budget_step_fits(in->n_seg, in->n_kv_heads, in->max_seg_len, in->head_dim);
  const int impl = in->dtype == KVE_BF16 ? score_impl() : 1;
  if (!fused && impl == 1 && valu_lds(rows, in->head_dim, in->dtype) > 65536)
    return fail(KVE_ESHAPE, "rows*head_dim too large for the fp32 scoring path");
  const size_t sw = step_score_ws(in, o, rows);
  const size_t kb = kept_idx ? 0 : round256(size_t(out->n_rows) * sizeof(int32_t));
  const size_t bb = budget_out ? 0 : round256(size_t(in->n_seg) * sizeof(int32_t));
  const size_t need = sw + kb + bb;
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(KVE_EWORKSPACE, "workspace not 256-byte aligned");
  char* wsc = static_cast<char*>(ws);
  int32_t* kept = kept_idx ? kept_idx : reinterpret_cast<int32_t*>(wsc + sw);
  int32_t* budget = budget_out ? budget_out : reinterpret_cast<int32_t*>(wsc + sw + kb);
  const int32_t batch = in->n_seg / in->n_kv_heads;
  const size_t ns = size_t(in->n_seg);
  const void* ins[] = {in->k, in->v, in->pos, in->seg_off, in->seg_len, o->q, o->q_pos, o->n_obs, layer_total,
                       out->seg_off};
  const size_t insz[] = {rows_bytes(in), rows_bytes(in), size_t(in->n_rows) * 4, ns * 8, ns * 4,
                         size_t(batch) * o->n_q_heads * o->max_obs * in->head_dim * elem_bytes(in->dtype),
                         size_t(batch) * o->max_obs * 4, size_t(batch) * 4, size_t(batch) * 4, ns * 8};
  const void* outs[] = {scores, head_entropy, budget, out->k, out->v, out->pos, out->seg_len, kept, ws};
  const size_t outsz[] = {size_t(in->n_rows) * 4, ns * 4, ns * 4, rows_bytes(out), rows_bytes(out),
                          size_t(out->n_rows) * 4, ns * 4, size_t(out->n_rows) * 4, sw};
  for (int i = 0; i < 9; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 9; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (in->n_seg == 0) return KVE_OK;
  if (!fused) {
    if ((st = kv_evict_score(in, o, scores, head_entropy, ws, sw, stream)) != KVE_OK) return st;
    if ((st = kv_evict_entropy_budgets(head_entropy, inverse, layer_total, in->seg_len, batch, in->n_kv_heads,
                                       min_per_head, budget, stream)) != KVE_OK)
      return st;
    // the scoring workspace is free again (stream order): the selection's control ints
    return kv_evict_select_compact(in, scores, nullptr, in->n_rows, budget, 0, n_prefix, n_recent, kept, out, ws, sw,
                                   stream);
  }
  kve::ScoreArgs a = score_args(in, o, rows, scores);
  a.entropy = head_entropy;
  a.v = in->v;
  a.k_out = out->k;
  a.v_out = out->v;
  a.pos_out = out->pos;
  a.out_off = out->seg_off;
  a.out_len = out->seg_len;
  a.out_rows = out->n_rows;
  a.out_cap = out->max_seg_len;
  a.kept = kept_idx;
  a.n_prefix = n_prefix;
  a.n_recent = n_recent;
  a.layer_total = layer_total;
  a.min_per_head = min_per_head;
  a.ent_form = inverse;
  a.budget_out = budget_out;
  return device_status(kve::launch_score_budget_select_compact(a, ws, static_cast<hipStream_t>(stream)),
                       "kv_evict_score_budget_select_compact");
}

kve_status kv_evict_score_select_compact_noalloc(const kve_cache* in, const kve_obs* o, float* scores,
                                                 const int32_t* budget, int32_t uniform_budget, int32_t n_prefix,
                                                 int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* stream) {
  // the scratch size this call needs, from the same checks as the workspace query
  int32_t rows = 0;
  kve_status st = check_cache(in, "in", true);
  if (st != KVE_OK) return st;
  if ((st = check_obs(in, o, &rows)) != KVE_OK) return st;
  if (!out) return fail(KVE_EINVAL, "out: null cache");
  const size_t need = kv_evict_score_select_compact_workspace(in, o, out, kept_idx ? 1 : 0);
  if (need > kve::kNoAllocScratchBytes)
    return fail(KVE_EWORKSPACE, "needs %zu bytes of scratch, more than the static %zu", need,
                kve::kNoAllocScratchBytes);
  void* p = nullptr;
  if ((st = device_status(kve::noalloc_scratch(&p), "static scratch address")) != KVE_OK) return st;
  return kv_evict_score_select_compact(in, o, scores, budget, uniform_budget, n_prefix, n_recent, kept_idx, out, p,
                                       kve::kNoAllocScratchBytes, stream);
}

size_t kv_evict_score_select_compact_inplace_workspace(const kve_cache* c, const kve_obs* o) {
  int32_t rows = 0;
  if (check_cache(c, "cache", true) != KVE_OK || check_obs(c, o, &rows) != KVE_OK) return 0;
  return step_score_ws(c, o, rows);
}

kve_status kv_evict_score_select_compact_inplace(kve_cache* c, const kve_obs* o, float* scores, const int32_t* budget,
                                                 int32_t uniform_budget, int32_t n_prefix, int32_t n_recent,
                                                 int32_t* new_len, void* ws, size_t ws_bytes, void* stream) {
  kve_status st = check_cache(c, "cache", true);
  if (st != KVE_OK) return st;
  int32_t rows = 0;
  if ((st = check_obs(c, o, &rows)) != KVE_OK) return st;
  if (n_prefix < 0 || n_recent < 0) return fail(KVE_EINVAL, "negative prefix/recent");
  if (c->n_seg > 0 && (!scores || !new_len)) return fail(KVE_EINVAL, "null scores or new_len");
  if (!budget && uniform_budget < n_prefix + n_recent)
    return fail(KVE_EBUDGET, "budget %d below prefix %d + recent %d", uniform_budget, n_prefix, n_recent);
  const bool fused = c->dtype == KVE_BF16 && score_impl() == 0 && c->max_seg_len > 0 &&
                     c->max_seg_len <= kve::step_max_seg(c->head_dim);
  const int impl = c->dtype == KVE_BF16 ? score_impl() : 1;
  if (!fused && impl == 1 && valu_lds(rows, c->head_dim, c->dtype) > 65536)
    return fail(KVE_ESHAPE, "rows*head_dim too large for the fp32 scoring path");
  const size_t sw = step_score_ws(c, o, rows);
  if (ws_bytes < sw || (sw > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, sw);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(KVE_EWORKSPACE, "workspace not 256-byte aligned");
  const int32_t batch = c->n_seg / c->n_kv_heads;
  const size_t ns = size_t(c->n_seg), rb = rows_bytes(c), pb = size_t(c->n_rows) * 4;
  // inputs that are only read, and the cache arrays that are read and rewritten
  const void* ins[] = {o->q, o->q_pos, o->n_obs, budget, c->seg_off};
  const size_t insz[] = {size_t(batch) * o->n_q_heads * o->max_obs * c->head_dim * elem_bytes(c->dtype),
                         size_t(batch) * o->max_obs * 4, size_t(batch) * 4, budget ? ns * 4 : 0, ns * 8};
  const void* cache[] = {c->k, c->v, c->pos};
  const size_t cachesz[] = {rb, rb, pb};
  const void* outs[] = {scores, ws};
  const size_t outsz[] = {size_t(c->n_rows) * 4, sw};
  for (int i = 0; i < 2; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], outsz[i], cache[j], cachesz[j]))
        return fail(KVE_EALIAS, "output %d overlaps cache array %d", i, j);
    if (overlap(outs[i], outsz[i], c->seg_len, ns * 4)) return fail(KVE_EALIAS, "output %d overlaps seg_len", i);
  }
  if (overlap(scores, outsz[0], ws, sw)) return fail(KVE_EALIAS, "scores overlap the workspace");
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 5; ++j)
      if (overlap(cache[i], cachesz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "cache array %d overlaps input %d", i, j);
  // new_len may be the cache's own seg_len (every work-group reads its length before any is written)
  if (new_len != c->seg_len) {
    const void* all[] = {c->k, c->v, c->pos, scores, c->seg_off, c->seg_len, budget, ws, o->q, o->q_pos, o->n_obs};
    const size_t allsz[] = {rb, rb, pb, size_t(c->n_rows) * 4, ns * 8, ns * 4, budget ? ns * 4 : 0, sw,
                            insz[0], insz[1], insz[2]};
    for (int j = 0; j < 11; ++j)
      if (overlap(new_len, ns * 4, all[j], allsz[j])) return fail(KVE_EALIAS, "new_len overlaps argument %d", j);
  }
  if (c->n_seg == 0) return KVE_OK;
  if (!fused) {
    if ((st = kv_evict_score(c, o, scores, nullptr, ws, sw, stream)) != KVE_OK) return st;
    return kv_evict_select_compact_inplace(c, scores, nullptr, c->n_rows, budget, uniform_budget, n_prefix, n_recent,
                                           new_len, stream);
  }
  kve::ScoreArgs a = score_args(c, o, rows, scores);
  a.v = c->v;
  a.k_out = c->k;
  a.v_out = c->v;
  a.pos_out = c->pos;
  a.out_off = c->seg_off;
  a.out_len = new_len;
  a.out_rows = c->n_rows;
  a.out_cap = c->max_seg_len;
  a.kept = nullptr;
  a.budget = budget;
  a.uniform_budget = uniform_budget;
  a.n_prefix = n_prefix;
  a.n_recent = n_recent;
  a.inplace = 1;
  return device_status(kve::launch_score_select_compact(a, ws, static_cast<hipStream_t>(stream)),
                       "kv_evict_score_select_compact_inplace");
}

kve_status beacon_fps_update(const void* q_in, void* q_out, const int32_t* count_in, int32_t* count_out, int32_t n_buf,
                             int32_t cap, int32_t k_keep, int32_t head_dim, int32_t dtype, int32_t* picks,
                             void* stream) {
  if (dtype != KVE_BF16 && dtype != KVE_F32) return fail(KVE_EINVAL, "bad dtype %d", dtype);
  if (n_buf < 0) return fail(KVE_EINVAL, "negative n_buf");
  if (head_dim != 64 && head_dim != 128) return fail(KVE_ESHAPE, "head_dim %d", head_dim);
  if (cap < 1 || cap > 64 || k_keep < 1 || k_keep > cap)
    return fail(KVE_ESHAPE, "cap %d / k_keep %d (need 1 <= k_keep <= cap <= 64)", cap, k_keep);
  if (size_t(4) * cap * head_dim * elem_bytes(dtype) > 65536) return fail(KVE_ESHAPE, "cap*head_dim too large");
  if (n_buf > 0 && (!q_in || !q_out || !count_in || !count_out)) return fail(KVE_EINVAL, "null pointer");
  if (!aligned16(q_in) || !aligned16(q_out)) return fail(KVE_EINVAL, "buffers not 16-byte aligned");
  const size_t qb = size_t(n_buf) * cap * head_dim * elem_bytes(dtype);
  const size_t cb = size_t(n_buf) * 4;
  if (q_in != q_out && overlap(q_in, qb, q_out, qb)) return fail(KVE_EALIAS, "q_out partially overlaps q_in");
  if (count_in != count_out && overlap(count_in, cb, count_out, cb))
    return fail(KVE_EALIAS, "count_out partially overlaps count_in");
  const size_t pb = size_t(n_buf) * k_keep * 4;
  if (overlap(picks, pb, q_in, qb) || overlap(picks, pb, q_out, qb) || overlap(picks, pb, count_in, cb) ||
      overlap(picks, pb, count_out, cb) || overlap(count_out, cb, q_in, qb) || overlap(count_out, cb, q_out, qb))
    return fail(KVE_EALIAS, "picks/counts overlap the buffers");
  return device_status(kve::launch_fps(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, head_dim, dtype, picks,
                                       static_cast<hipStream_t>(stream)),
                       "beacon_fps_update");
}

size_t epikv_workspace_size(int32_t batch, int32_t T) {
  if (batch < 0 || T < 0) return 0;
  return kve::epikv_ws_bytes(batch, T);
}

kve_status epikv_score(const void* h_a, const void* h_b, int32_t batch, int32_t T, int32_t d_model, int32_t window,
                       float eps, int32_t form, float* g_out, float* scores, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 0 || T < 0) return fail(KVE_EINVAL, "negative batch or T");
  if (form != KVE_EPIKV_Z && form != KVE_EPIKV_MEAN) return fail(KVE_EINVAL, "form must be 0 (z) or 1 (rolling mean)");
  if (d_model != 512 && d_model != 1024 && d_model != 2048 && d_model != 4096 && d_model != 8192)
    return fail(KVE_ESHAPE, "d_model %d", d_model);
  if (window < 1 || window > 2048) return fail(KVE_ESHAPE, "window %d not in [1, 2048]", window);
  if (!(eps >= 0.f)) return fail(KVE_EINVAL, "eps must be >= 0");
  const size_t n = size_t(batch) * T;
  if (n > 0 && (!h_a || !h_b || !scores)) return fail(KVE_EINVAL, "null pointer");
  if (!aligned16(h_a) || !aligned16(h_b)) return fail(KVE_EINVAL, "traces not 16-byte aligned");
  const size_t need = g_out ? 0 : kve::epikv_ws_bytes(batch, T);
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  const size_t hb = n * d_model * 2;
  const size_t gb = 2 * n * 4;
  const float* gbuf = g_out ? g_out : static_cast<const float*>(ws);
  if (overlap(scores, n * 4, h_a, hb) || overlap(scores, n * 4, h_b, hb) || overlap(gbuf, gb, h_a, hb) ||
      overlap(gbuf, gb, h_b, hb) || overlap(gbuf, gb, scores, n * 4))
    return fail(KVE_EALIAS, "an output of epikv_score overlaps an input");
  return device_status(kve::launch_epikv(h_a, h_b, batch, T, d_model, window, eps, form, g_out, scores, ws,
                                         static_cast<hipStream_t>(stream)),
                       "epikv_score");
}

size_t skipkv_workspace_size(int32_t batch, int32_t max_sent, int32_t d_model) {
  if (batch < 0 || max_sent < 0 || d_model < 0) return 0;
  return kve::skipkv_ws_bytes(batch, max_sent, d_model);
}

kve_status skipkv_sentence_scores(const void* h, int32_t batch, int32_t T, int32_t d_model, const int32_t* starts,
                                  const int32_t* n_sent, int32_t max_sent, float tau, float* pss_max, int32_t* marks,
                                  float* token_scores, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 0 || T < 0 || max_sent < 0) return fail(KVE_EINVAL, "negative batch, T or max_sent");
  if (d_model < 64 || d_model > 16384 || d_model % 64 != 0)
    return fail(KVE_ESHAPE, "d_model %d not a multiple of 64 in [64, 16384]", d_model);
  if (max_sent > 65535) return fail(KVE_ESHAPE, "max_sent %d > 65535", max_sent);
  if (!(tau == tau)) return fail(KVE_EINVAL, "tau is NaN");
  const size_t nt = size_t(batch) * T, nsnt = size_t(batch) * max_sent;
  if (batch > 0 && (!starts || !n_sent || !token_scores || (nsnt > 0 && !pss_max) || (T > 0 && !h)))
    return fail(KVE_EINVAL, "null pointer");
  if (!aligned16(h)) return fail(KVE_EINVAL, "hidden states not 16-byte aligned");
  const size_t need = kve::skipkv_ws_bytes(batch, max_sent, d_model);
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(KVE_EWORKSPACE, "workspace not 256-byte aligned");
  const void* ins[] = {h, starts, n_sent};
  const size_t insz[] = {nt * d_model * 2, nsnt + batch, size_t(batch) * 4};
  const void* outs[] = {pss_max, marks, token_scores, ws};
  const size_t outsz[] = {nsnt * 4, marks ? nsnt * 4 : 0, nt * 4, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], outsz[i], ins[j], j == 1 ? insz[j] * 4 : insz[j]))
        return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (batch == 0) return KVE_OK;
  kve::SkipArgs a{};
  a.h = h;
  a.starts = starts;
  a.n_sent = n_sent;
  a.batch = batch;
  a.T = T;
  a.d_model = d_model;
  a.max_sent = max_sent;
  a.tau = tau;
  a.pss_max = pss_max;
  a.marks = marks;
  a.token_scores = token_scores;
  return device_status(kve::launch_skipkv(a, ws, static_cast<hipStream_t>(stream)), "skipkv_sentence_scores");
}

size_t kv_decode_attention_workspace(const kve_cache* c, int32_t n_q_heads) {
  if (check_cache(c, "cache", true) != KVE_OK || n_q_heads < c->n_kv_heads || n_q_heads % c->n_kv_heads) return 0;
  return kve::attn_workspace_bytes(c->n_seg, c->max_seg_len, n_q_heads / c->n_kv_heads, c->head_dim);
}

kve_status kv_decode_attention(const kve_cache* c, const void* q, int32_t n_q_heads, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  kve_status st = check_cache(c, "cache", true);
  if (st != KVE_OK) return st;
  if (n_q_heads < c->n_kv_heads || n_q_heads % c->n_kv_heads != 0)
    return fail(KVE_ESHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", n_q_heads, c->n_kv_heads);
  const int32_t group = n_q_heads / c->n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return fail(KVE_ESHAPE, "group %d not 1, 2, 4 or 8", group);
  if (c->n_seg > 0 && (!q || !out)) return fail(KVE_EINVAL, "null q or out");
  const size_t need = kve::attn_workspace_bytes(c->n_seg, c->max_seg_len, group, c->head_dim);
  if (ws_bytes < need || (need > 0 && !ws)) return fail(KVE_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  const size_t batch = size_t(c->n_seg / c->n_kv_heads);
  const size_t ob = batch * n_q_heads * c->head_dim * 4, lb = batch * n_q_heads * 4;
  const size_t qb = batch * n_q_heads * c->head_dim * elem_bytes(c->dtype);
  const void* ins[] = {c->k, c->v, c->seg_off, c->seg_len, q};
  const size_t insz[] = {rows_bytes(c), rows_bytes(c), size_t(c->n_seg) * 8, size_t(c->n_seg) * 4, qb};
  const void* outs[] = {out, lse, ws};
  const size_t outsz[] = {ob, lse ? lb : 0, need};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(KVE_EALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(KVE_EALIAS, "outputs %d and %d overlap", i, j);
  }
  if (c->n_seg == 0) return KVE_OK;
  kve::AttnArgs a{};
  a.k = c->k;
  a.v = c->v;
  a.seg_off = c->seg_off;
  a.seg_len = c->seg_len;
  a.n_rows = c->n_rows;
  a.n_seg = c->n_seg;
  a.n_kv = c->n_kv_heads;
  a.max_seg_len = c->max_seg_len;
  a.head_dim = c->head_dim;
  a.dtype = c->dtype;
  a.q = q;
  a.n_q = n_q_heads;
  a.group = group;
  a.out = out;
  a.lse = lse;
  a.part = static_cast<float*>(ws);
  return device_status(kve::launch_decode_attention(a, static_cast<hipStream_t>(stream)), "kv_decode_attention");
}

kve_status kv_rope_apply(const float* src, void* dst, const int32_t* pos, int64_t n_rows, int32_t head_dim,
                         double rope_theta, int32_t dtype, void* stream) {
  if (dtype != KVE_BF16 && dtype != KVE_F32) return fail(KVE_EINVAL, "bad dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(KVE_ESHAPE, "head_dim %d", head_dim);
  if (n_rows < 0) return fail(KVE_EINVAL, "negative n_rows");
  if (!(rope_theta > 0.0)) return fail(KVE_EINVAL, "rope_theta must be > 0");
  if (n_rows > 0 && (!src || !dst || !pos)) return fail(KVE_EINVAL, "null pointer");
  if (overlap(src, size_t(n_rows) * head_dim * 4, dst, size_t(n_rows) * head_dim * elem_bytes(dtype)))
    return fail(KVE_EALIAS, "dst overlaps src");
  return device_status(
      kve::launch_rope_rows(src, dst, pos, n_rows, head_dim, rope_theta, dtype, static_cast<hipStream_t>(stream)),
      "kv_rope_apply");
}

}  // extern "C"
