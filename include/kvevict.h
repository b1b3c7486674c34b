/*
 * kvevict.h — C ABI of the decode-time KV-cache eviction step for MI355X (gfx950).
 *
 * The step, as the BeaconKV page describes it (sections "观察 query 集 = 最近查询 +
 * 信标查询", "Continual FPS：有界内存的在线最远点采样", "打分时的 RoPE 对齐" and
 * "📊 实验"): every cached key of every KV head is scored by a small observation
 * set of queries (recent queries at their own RoPE positions, beacon queries kept
 * pre-RoPE and rotated to the current step t), by a per-row softmax of q.k/sqrt(d)
 * max-aggregated over the queries and the GQA group; the prefix and the recent
 * window are always kept, the remaining budget goes to the top scores, and the
 * cache is compacted.  Per-head budgets may follow the ReasonAlloc page ("Core
 * Mechanism", "Key Concepts"); the EPIKV page (方法论 parts 1 and 3) supplies an
 * attention-free alternative score.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     keeps no state (apart from the test overrides of kve_set_test_overrides,
 *     the per-thread error message, the static scratch array of
 *     kv_evict_score_select_compact_noalloc and, in the bounds-checked build
 *     only, the flag word of kve_debug_flags) and allocates no device memory;
 *     scratch comes from a caller-provided workspace whose size the
 *     *_workspace_size calls return.
 *   - Every call is asynchronous and stream-ordered on `stream` (a hipStream_t;
 *     NULL is the null stream).  No call synchronises (kve_debug_flags, a test
 *     call, synchronises the device).
 *   - Arguments are checked on the host BEFORE any launch; on an error status
 *     nothing is launched and nothing is written.  Values that live in device
 *     memory (segment offsets, lengths, budgets) are checked by the kernels,
 *     which never read or write outside the declared buffers: a segment whose
 *     metadata is out of range is skipped, and select/compact report it by
 *     writing -1 as that segment's output length.
 *   - Launch failures return KVE_EDEVICE.  No C++ exception crosses the ABI.
 *     kve_last_error() returns a message for the last non-OK status of the
 *     calling thread.
 *   - Storage dtypes: KVE_BF16 (bfloat16) or KVE_F32.  head_dim is 64 or 128.
 *
 * Cache layout (one layer, or several layers folded into the batch)
 *   A cache is a set of segments, one per (request b, KV head g), s = b*n_kv_heads+g.
 *   Segment s owns rows seg_off[s] .. seg_off[s]+seg_len[s]-1 of k, v and pos; a
 *   row of k or v is head_dim contiguous elements.  K is stored post-RoPE at the
 *   row's original position pos[row].  Every segment must have room for
 *   max_seg_len rows (seg_off[s] + max_seg_len <= n_rows) when the cache is an
 *   output; as an input seg_len[s] <= max_seg_len.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVE_ABI_VERSION 2

typedef enum {
  KVE_OK = 0,
  KVE_EINVAL = 1,      /* null pointer, bad enum, negative size */
  KVE_ESHAPE = 2,      /* unsupported or inconsistent shape */
  KVE_EALIAS = 3,      /* an output overlaps an input it must not overlap */
  KVE_EBUDGET = 4,     /* budget below the protected prefix + recent window */
  KVE_EWORKSPACE = 5,  /* workspace missing or too small */
  KVE_EDEVICE = 6      /* HIP runtime / launch failure */
} kve_status;

typedef enum { KVE_BF16 = 0, KVE_F32 = 1 } kve_dtype;

/* Aggregation of the observation rows' softmax probabilities into a key's score. */
typedef enum { KVE_AGG_MAX = 0, KVE_AGG_MEAN = 1 } kve_aggregate;

/* Form of the attention-free score. */
typedef enum { KVE_EPIKV_Z = 0, KVE_EPIKV_MEAN = 1 } kve_epikv_form;

typedef struct kve_cache {
  int32_t dtype;            /* kve_dtype of k and v */
  int32_t n_seg;            /* segments = batch * n_kv_heads */
  int32_t n_kv_heads;
  int32_t head_dim;         /* 64 or 128 */
  int32_t max_seg_len;      /* bound on every seg_len; per-segment row capacity of an output */
  int32_t reserved;
  int64_t n_rows;           /* rows allocated in k, v and pos */
  void* k;                  /* [n_rows, head_dim] post-RoPE keys */
  void* v;                  /* [n_rows, head_dim] values */
  int32_t* pos;             /* [n_rows] original token position of each row */
  const int64_t* seg_off;   /* [n_seg] first row of each segment */
  int32_t* seg_len;         /* [n_seg] valid rows (written by kv_evict_select_compact on an output) */
} kve_cache;

typedef struct kve_obs {
  const void* q;            /* [batch, n_q_heads, max_obs, head_dim] PRE-RoPE queries, cache dtype */
  const int32_t* q_pos;     /* [batch, max_obs] position each row is rotated to:
                               tau_i for a recent query, the current step t for a beacon */
  const int32_t* n_obs;     /* [batch] valid rows per request (<= max_obs), or NULL = max_obs */
  int32_t n_q_heads;        /* multiple of n_kv_heads; query head h scores KV head h / (n_q_heads/n_kv_heads) */
  int32_t max_obs;          /* (n_q_heads/n_kv_heads) * max_obs <= 256 */
  double rope_theta;        /* RoPE base; pairs (x_i, x_{i+d/2}), frequency theta^(-2i/d) */
  int32_t causal;           /* 1: key j visible to row i iff pos[j] <= q_pos[i]; 0: all keys visible */
  int32_t aggregate;        /* kve_aggregate: KVE_AGG_MAX (BeaconKV's choice) or KVE_AGG_MEAN (its ablation) */
} kve_obs;

/* Workspace bytes kv_evict_score needs for this cache/observation shape. */
size_t kv_evict_score_workspace(const kve_cache* c, const kve_obs* o);

/*
 * kv_evict_score — BeaconKV "打分时的 RoPE 对齐": rotate each observation query to
 * its q_pos (angle formed in double precision, rotated value rounded to the cache
 * dtype), take logits q.k/sqrt(d) in fp32 over every visible cached key of the
 * segment, a per-row softmax over the segment, and
 *   scores[row] = max over the group's query heads and observation rows of p
 * (o->aggregate = KVE_AGG_MAX), or, for the max-vs-mean ablation of BeaconKV's
 * "📊 实验", the mean over those rows (KVE_AGG_MEAN: every existing row counts,
 * a key a row cannot see contributes 0 for that row).
 * scores: [c->n_rows] fp32, aligned with the cache rows (rows outside every
 * segment are not written).  head_entropy: optional [n_seg] fp32, the
 * normalised entropy of each segment's score distribution (ReasonAlloc "Key
 * Concepts": head utility), or NULL.
 * Errors: EINVAL (null pointers), ESHAPE (head_dim, group, rows > 256),
 * EWORKSPACE, EALIAS (scores, head_entropy or the workspace overlapping an
 * input or each other), EDEVICE.
 */
kve_status kv_evict_score(const kve_cache* c, const kve_obs* o, float* scores, float* head_entropy,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * kv_evict_budgets — ReasonAlloc "Core Mechanism" (online head-wise
 * reallocation): per request b, split layer_total[b] over the n_heads heads
 * proportionally to weights[b*n_heads+g] with floor min_per_head and cap
 * cap[b*n_heads+g] (x_g = clamp(lam*w_g, min(floor,cap_g), cap_g), sum =
 * min(total, sum cap)), then round by largest remainder (ties to the lower
 * head).  All-zero weights split equally.  A head of weight 0 keeps its floor
 * while some lam meets the total; once every weighted head is at its cap, the
 * rest is split equally over the weightless heads (under their caps).
 * Computed in double precision.
 * budget_out: [batch*n_heads] int32.  A request whose total is below the sum of
 * its floors gets -1 in every head.  Errors: EINVAL, ESHAPE (n_heads > 64), EDEVICE.
 */
kve_status kv_evict_budgets(const float* weights, const int32_t* layer_total, const int32_t* cap,
                            int32_t batch, int32_t n_heads, int32_t min_per_head,
                            int32_t* budget_out, void* stream);

/*
 * kv_evict_wave_budgets — ReasonAlloc "Core Mechanism" (offline layer-wise
 * preallocation, the mid-peaked "Reasoning Wave"): per-layer base budgets
 * proportional to exp(-(l-center)^2 / (2 sigma^2)), floor min_per_layer,
 * summing exactly to total, largest-remainder rounding.  out: [n_layers] int32
 * device.  Errors: EINVAL, ESHAPE (n_layers > 64 or total < n_layers*floor), EDEVICE.
 */
kve_status kv_evict_wave_budgets(int32_t n_layers, double center, double sigma, int32_t total,
                                 int32_t min_per_layer, int32_t* out, void* stream);

/*
 * kv_evict_entropy_budgets — kv_evict_budgets with the weights formed from the
 * heads' normalised score entropy E (kv_evict_score's head_entropy, [batch *
 * n_heads] fp32): weight = E (inverse = 0) or 1 - E (inverse = 1, ReasonAlloc
 * "Key Concepts": low-entropy, focused heads are the useful ones and gain
 * budget).  Every other argument and rule as kv_evict_budgets.
 * Errors: EINVAL (inverse not 0/1, null pointers), ESHAPE, EALIAS, EDEVICE.
 */
kve_status kv_evict_entropy_budgets(const float* head_entropy, int32_t inverse, const int32_t* layer_total,
                                    const int32_t* cap, int32_t batch, int32_t n_heads, int32_t min_per_head,
                                    int32_t* budget_out, void* stream);

/* Workspace bytes kv_evict_select_compact asks for: the kept-index list when
 * kept_idx is not supplied (the part it requires), then, for at most 128
 * segments, a control area of about 4.3 KB per segment that lets segments too
 * long for one work-group's on-chip keys be selected by several work-groups
 * each (with less, those run one work-group per segment). */
size_t kv_evict_select_workspace(const kve_cache* out, int32_t have_kept_idx);

/*
 * kv_evict_select_compact — BeaconKV "打分时的 RoPE 对齐" and "📊 实验": per segment
 * with n rows and budget K: if K >= n keep every row; otherwise keep slots
 * [0, n_prefix) and [n-n_recent, n) and the K-n_prefix-n_recent other slots with
 * the highest score (score descending, slot ascending; scores compared as fp32
 * values, so -0.0 ties with +0.0; NaN is not supported), then gather-compact K, V and pos, in ascending slot order,
 * into the output segment and set out->seg_len[s].
 *   scores: fp32 [n_scores]; the score of slot j of segment s is
 *           scores[(score_off ? score_off[s] : in->seg_off[s]) + j]
 *           (score_off lets one per-token score serve every KV head of a request;
 *           a segment whose scores would fall outside [0, n_scores) is rejected).
 *   budget: [n_seg] device int32, or NULL to use uniform_budget for every segment.
 *   kept_idx: optional [out->n_rows] int32; row out->seg_off[s]+i receives the
 *           source slot of output row i.
 * The output must not overlap the input (EALIAS); out->max_seg_len is each output
 * segment's capacity.  A segment whose budget is below n_prefix+n_recent (and
 * below n), or larger than the output capacity, or whose metadata is out of
 * range, gets out->seg_len[s] = -1 and no rows.  Work-groups that share a long
 * segment meet with bounded polling; a segment whose work-groups could not all
 * run within that bound (only on a device busy with other work for that long)
 * also gets -1.
 * Errors: EINVAL, ESHAPE (dtype/head_dim/n_seg mismatch), EALIAS,
 * EBUDGET (uniform_budget < n_prefix+n_recent, or > out->max_seg_len), EWORKSPACE, EDEVICE.
 */
kve_status kv_evict_select_compact(const kve_cache* in, const float* scores, const int64_t* score_off,
                                   int64_t n_scores, const int32_t* budget, int32_t uniform_budget,
                                   int32_t n_prefix, int32_t n_recent, int32_t* kept_idx,
                                   kve_cache* out, void* ws, size_t ws_bytes, void* stream);

/*
 * kv_evict_select_compact_inplace — the same per-segment selection as
 * kv_evict_select_compact (same budget, protection and tie rules), compacted
 * within the cache c itself by hole filling: with K survivors, those already
 * in slots [0, K) stay, and the survivors in [K, n), in ascending slot order,
 * move into the evicted slots of [0, K), in ascending slot order (K, V and pos
 * rows; at most min(K, n-K) rows move per segment).  Rows [K, n) are left as
 * they were.  The survivors are therefore not in slot order; attention does
 * not depend on the order of the cached rows (BeaconKV "📊 实验": eviction is
 * permanent; each row keeps its position, which carries RoPE and causality).
 * Protection is by slot, as in kv_evict_select_compact: once a segment has been
 * hole-filled its slot order no longer follows position, so a later call
 * protects the n_recent most recent tokens only if at least n_recent tokens
 * were appended at the end of the segment since the hole filling (with fewer,
 * the protected window also covers the last slots of the hole-filled rows,
 * whatever their positions).
 * new_len: [n_seg] int32, receives K (n when K >= n, -1 for a segment rejected
 * as in kv_evict_select_compact); it may be c->seg_len itself.  No workspace.
 * Errors: EINVAL, ESHAPE, EALIAS (scores/budget/score_off/seg_off overlapping the
 * cache rows; new_len overlapping anything but c->seg_len), EBUDGET, EDEVICE.
 */
kve_status kv_evict_select_compact_inplace(kve_cache* c, const float* scores, const int64_t* score_off,
                                           int64_t n_scores, const int32_t* budget, int32_t uniform_budget,
                                           int32_t n_prefix, int32_t n_recent, int32_t* new_len, void* stream);

/* Workspace bytes kv_evict_score_select_compact needs. */
size_t kv_evict_score_select_compact_workspace(const kve_cache* in, const kve_obs* o, const kve_cache* out,
                                               int32_t have_kept_idx);

/*
 * kv_evict_score_select_compact — one eviction trigger of BeaconKV ("打分时的
 * RoPE 对齐" for the score, "📊 实验" for dropping the evicted rows): the
 * result of kv_evict_score(in, o, scores, NULL) followed by
 * kv_evict_select_compact(in, scores, NULL, in->n_rows, budget, ...), with the
 * same meaning of every argument.  For bf16 caches whose max_seg_len fits the
 * on-chip selection (9216 rows at head_dim 128, 5120 at 64) it runs as one
 * kernel: each segment's work-groups score their chunk, wait for the segment's
 * other chunks, select, and gather their own chunk's kept rows while those are
 * still in cache; otherwise it makes the two calls.  scores ([in->n_rows] fp32)
 * is written as by kv_evict_score.  Budgets must be known before the call
 * (uniform, or a device array from an earlier step); the per-head entropy that
 * ReasonAlloc's reallocation needs comes from kv_evict_score.  Ties between
 * near-equal scores may resolve differently from the two-call form, since the
 * softmax normaliser is summed in another order (scores agree to fp32 rounding).
 * A segment's work-groups wait for each other with bounded polling; a segment
 * whose work-groups could not all run within that bound (only possible on a
 * device stalled for a long time) gets out->seg_len[s] = -1 like a rejected one.
 * Errors: the union of kv_evict_score's and kv_evict_select_compact's; scores,
 * the output cache, kept_idx and the workspace must not overlap any input or
 * each other (EALIAS).
 */
kve_status kv_evict_score_select_compact(const kve_cache* in, const kve_obs* o, float* scores,
                                         const int32_t* budget, int32_t uniform_budget, int32_t n_prefix,
                                         int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* ws,
                                         size_t ws_bytes, void* stream);

/*
 * kv_evict_score_select_compact_noalloc — for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): kv_evict_score_select_compact with the same
 * arguments and results, minus the workspace, which comes instead from a
 * static device array of 32 MiB that every GPU the library runs on holds until
 * the process ends.  It calls no allocating routine.  Calls on one GPU share
 * that array: two such calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and give undefined results;
 * calls ordered on one stream do not.  What must start at zero is cleared by
 * each call.  A call whose workspace (kv_evict_score_select_compact_workspace
 * with have_kept_idx = kept_idx != NULL) exceeds 32 MiB is rejected
 * (EWORKSPACE) before anything is launched: a Qwen3-4B-shaped layer of 16
 * requests needs about 10 MB, so one call covers up to three such layers.
 * Errors: those of kv_evict_score_select_compact, EWORKSPACE when the scratch
 * is too small.
 */
kve_status kv_evict_score_select_compact_noalloc(const kve_cache* in, const kve_obs* o, float* scores,
                                                 const int32_t* budget, int32_t uniform_budget, int32_t n_prefix,
                                                 int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* stream);

/* Workspace bytes kv_evict_score_select_compact_inplace needs. */
size_t kv_evict_score_select_compact_inplace_workspace(const kve_cache* c, const kve_obs* o);

/*
 * kv_evict_score_select_compact_inplace — one eviction trigger of BeaconKV
 * ("打分时的 RoPE 对齐" for the score; "📊 实验": eviction is permanent) compacted
 * within the cache itself: the result of kv_evict_score(c, o, scores, NULL)
 * followed by kv_evict_select_compact_inplace(c, scores, NULL, c->n_rows, budget,
 * uniform_budget, n_prefix, n_recent, new_len), with the same meaning of every
 * argument (hole filling: the survivors in [K, n), in ascending slot order,
 * move into the evicted slots of [0, K), in ascending slot order).  For bf16
 * caches whose max_seg_len fits the on-chip selection (9216 rows at head_dim
 * 128, 5120 at 64) it runs as one kernel (a segment's work-groups score their
 * chunks, usually the whole segment in one; the last of them to finish selects
 * and moves the segment's survivors); otherwise it makes the two calls.  The kept
 * sets may differ from the two-call form's only where scores tie to fp32
 * rounding (the softmax normaliser is summed in another order).  new_len may
 * be c->seg_len itself; a segment whose work-groups could not meet within the
 * barrier's poll bound gets -1.
 * Errors: the union of kv_evict_score's and kv_evict_select_compact_inplace's;
 * scores and the workspace must not overlap the cache or any input (EALIAS).
 */
kve_status kv_evict_score_select_compact_inplace(kve_cache* c, const kve_obs* o, float* scores, const int32_t* budget,
                                                 int32_t uniform_budget, int32_t n_prefix, int32_t n_recent,
                                                 int32_t* new_len, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes kv_evict_score_budget_select_compact needs. */
size_t kv_evict_score_budget_select_compact_workspace(const kve_cache* in, const kve_obs* o, const kve_cache* out,
                                                      int32_t have_kept_idx, int32_t have_budget_out);

/*
 * kv_evict_score_budget_select_compact — one eviction trigger with ReasonAlloc's
 * entropy-driven head budgets ("Core Mechanism": online head-wise reallocation;
 * "Key Concepts": normalised attention entropy): the result of
 *   kv_evict_score(in, o, scores, head_entropy, ...),
 *   kv_evict_entropy_budgets(head_entropy, inverse, layer_total, in->seg_len,
 *                            in->n_seg / in->n_kv_heads, in->n_kv_heads, min_per_head, budget, ...),
 *   kv_evict_select_compact(in, scores, NULL, in->n_rows, budget, 0, n_prefix, n_recent, kept_idx, out, ...)
 * with the same meaning of every argument.  The segments of one request-layer
 * are the in->n_kv_heads consecutive segments b*n_kv_heads .. b*n_kv_heads +
 * n_kv_heads - 1, and layer_total[b] is their total ([n_seg / n_kv_heads] device
 * int32, e.g. n_kv_heads times the layer's kv_evict_wave_budgets entry).
 * head_entropy ([n_seg] fp32) is required and written; budget_out ([n_seg] int32)
 * is optional and receives the head budgets.  out->max_seg_len must be at least
 * in->max_seg_len (a head may keep every row).  For bf16 caches whose segments fit
 * the on-chip selection (9216 rows at head_dim 128, 5120 at 64) and whose heads'
 * work-groups fit its dispatch bound (about 96 per request-layer, so at most 10
 * heads of up to 9216 rows) it runs as one kernel: every head's chunks are
 * scored and its entropy published, and later work-groups of the same launch,
 * once all of a request-layer's heads are in, solve the same head budgets
 * with the budget kernel's solver and select and gather each chunk's kept
 * rows; otherwise it makes the three calls.  The entropies
 * are summed in another order than the stand-alone scoring's (equal to fp32
 * rounding), so budgets can differ from the three-call form's only where
 * largest-remainder fractions tie to that rounding.  A request-layer whose
 * heads could not meet within the poll bound (only on a device stalled that
 * long), or whose floors exceed its total, gets out->seg_len = -1 in every head.
 * Errors: the union of the three calls' (EINVAL for inverse not 0/1 or a null
 * head_entropy/layer_total, ESHAPE, EALIAS, EBUDGET when out->max_seg_len <
 * in->max_seg_len, EWORKSPACE, EDEVICE).
 */
kve_status kv_evict_score_budget_select_compact(const kve_cache* in, const kve_obs* o, float* scores,
                                                float* head_entropy, int32_t inverse, const int32_t* layer_total,
                                                int32_t min_per_head, int32_t* budget_out, int32_t n_prefix,
                                                int32_t n_recent, int32_t* kept_idx, kve_cache* out, void* ws,
                                                size_t ws_bytes, void* stream);

/*
 * beacon_fps_update — BeaconKV "Continual FPS": for each of n_buf buffers of
 * pre-RoPE queries ([n_buf, cap, head_dim], dtype) whose count_in equals cap, run
 * farthest-point sampling under the cosine distance 1 - cos: first pick row 0,
 * then repeatedly the unpicked row farthest (fp32) from the picked set, ties to
 * the lower row, until k_keep rows are picked; write the picked rows in
 * ascending row order to rows 0..k_keep-1 of q_out and set count_out = k_keep.
 * Buffers with count_in != cap are copied unchanged (count_out = count_in).
 * q_out may equal q_in and count_out may equal count_in (in place); partial
 * overlap is EALIAS.  picks: optional [n_buf, k_keep] int32, the picks in
 * selection order (-1 for buffers that were not full).
 * Errors: EINVAL, ESHAPE (cap > 64, 1 <= k_keep <= cap, head_dim, and for fp32
 * cap*head_dim <= 4096), EALIAS, EDEVICE.
 */
kve_status beacon_fps_update(const void* q_in, void* q_out, const int32_t* count_in, int32_t* count_out,
                             int32_t n_buf, int32_t cap, int32_t k_keep, int32_t head_dim, int32_t dtype,
                             int32_t* picks, void* stream);

/* Workspace bytes epikv_score needs. */
size_t epikv_workspace_size(int32_t batch, int32_t T);

/*
 * epikv_score — EPIKV page (方法论 part 1 顿悟得分 and part 3 时间趋势校正): for the
 * two monitored layers a and b (bf16 traces [batch, T, d_model]),
 *   g(t) = ||h(t) - h(t-1)||_2 (t >= 1), g(0) = 0,
 *   z(t) = (g(t) - mean) / (std + eps) over the causal window
 *          {max(1, t-window+1) .. t} (population std), z(0) = 0,
 *   scores[b*T + t] = z_a(t) - z_b(t)   (higher keeps; form = KVE_EPIKV_Z), or
 *   scores[b*T + t] = gbar_a(t) - gbar_b(t), the rolling means of g over the
 *   same window (form = KVE_EPIKV_MEAN; 方法论 part 2), gbar(0) = 0.
 * g_out: optional [2, batch, T] fp32 (the two g series).  Window sums in double.
 * d_model is 512, 1024, 2048, 4096 or 8192; the traces and scores are 16-byte aligned.
 * Errors: EINVAL (form, null pointers), ESHAPE (d_model, window < 1 or > 2048), EWORKSPACE, EDEVICE.
 */
kve_status epikv_score(const void* h_a, const void* h_b, int32_t batch, int32_t T, int32_t d_model,
                       int32_t window, float eps, int32_t form, float* g_out, float* scores,
                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes skipkv_sentence_scores needs. */
size_t skipkv_workspace_size(int32_t batch, int32_t max_sent, int32_t d_model);

/*
 * skipkv_sentence_scores — SkipKV page (核心方法 §4.1): sentence-level
 * redundancy.  Sentence i of request b covers tokens [starts[b][i],
 * starts[b][i+1]) (starts: [batch, max_sent + 1] int32 device, n_sent[b] <=
 * max_sent complete sentences; a reversed or out-of-range span counts as an
 * empty sentence).  Its embedding is the mean of its tokens' last-layer hidden
 * states h ([batch, T, d_model] bf16, fp32 sums); the pairwise sentence
 * similarity (PSS) is the cosine of two embeddings (0 for an empty or zero
 * embedding).  Outputs:
 *   pss_max[b][i]      the largest PSS of sentence i with a later sentence j > i
 *                      (-1 when there is none, also for i >= n_sent[b]);
 *   marks[b][i]        optional: 1 if pss_max >= tau (the earlier sentence of a
 *                      redundant pair is the evictable one; the page uses 0.95);
 *   token_scores[b][t] 1 - max(0, pss_max) of token t's sentence, 1 after the
 *                      last complete sentence — higher keeps, whole sentences
 *                      go together.  The page's combined score (its eq. 6,
 *                      with token importance weighted by lambda) is not
 *                      printed; this is the sentence term alone.
 * token_scores feeds kv_evict_select_compact through score_off (one score per
 * token shared by every KV head of a request).  d_model: a multiple of 64 in
 * [64, 16384]; h 16-byte aligned.
 * Errors: EINVAL, ESHAPE, EALIAS, EWORKSPACE, EDEVICE.
 */
kve_status skipkv_sentence_scores(const void* h, int32_t batch, int32_t T, int32_t d_model, const int32_t* starts,
                                  const int32_t* n_sent, int32_t max_sent, float tau, float* pss_max,
                                  int32_t* marks, float* token_scores, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes kv_decode_attention needs. */
size_t kv_decode_attention_workspace(const kve_cache* c, int32_t n_q_heads);

/*
 * kv_decode_attention — the decode step's attention over the (compacted) cache,
 * the step that follows eviction (EPIKV 方法论 part 4: the eviction score stays
 * compatible with a fused attention kernel; BeaconKV "📊 实验" reports decode
 * throughput over the compacted cache): for every request b and query head h,
 *   out[b, h] = softmax_j(q[b, h] . k_j / sqrt(head_dim)) v_j
 * over all rows j of segment b*n_kv_heads + h/(n_q_heads/n_kv_heads), in any
 * row order (the in-place compaction's layout works as is).  q: [batch,
 * n_q_heads, head_dim] rotated queries of the new token, cache dtype.  out:
 * fp32 [batch, n_q_heads, head_dim]; lse: optional fp32 [batch, n_q_heads],
 * natural-log normaliser.  fp32 accumulation.  An empty segment (or one whose
 * metadata is out of range) gives zeros and lse = -inf.  n_q_heads/n_kv_heads
 * must be 1, 2, 4 or 8.
 * Errors: EINVAL, ESHAPE, EALIAS, EWORKSPACE, EDEVICE.
 */
kve_status kv_decode_attention(const kve_cache* c, const void* q, int32_t n_q_heads, float* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * kv_rope_apply — write keys into a cache the way a decoder layer does: rotate
 * fp32 pre-RoPE rows src[n_rows, head_dim] to positions pos[n_rows] (half-split
 * pairs, angle in double precision, rotation in double) and round to dtype into
 * dst[n_rows, head_dim].  src and dst must not overlap.
 * Errors: EINVAL, ESHAPE, EALIAS, EDEVICE.
 */
kve_status kv_rope_apply(const float* src, void* dst, const int32_t* pos, int64_t n_rows,
                         int32_t head_dim, double rope_theta, int32_t dtype, void* stream);

/*
 * kve_set_test_overrides — for the library's own tests, not for production
 * callers: two process-wide overrides of internal choices, both 0 (off) when
 * the library loads.  Every later call of any entry point, on any thread, sees
 * the values set last; set them while no other thread is calling the library.
 *   score_impl  0: default dispatch.  1: the plain VALU scoring kernels for
 *               bf16 caches as well (a cross-check of the MFMA kernels).  2: the
 *               single-read MFMA scoring kernel in kv_evict_score.  With 1 or 2
 *               the one-call entry points run their multi-call forms.
 *   spin_limit  0: the default poll bound of the work-group meetings (about
 *               four million polls).  > 0: that many polls, so that a test can
 *               make the meetings give up and check the failure reporting.
 * Errors: EINVAL (score_impl not 0..2, spin_limit outside [0, 2^30]).
 */
kve_status kve_set_test_overrides(int32_t score_impl, int32_t spin_limit);

/*
 * kve_debug_flags — bounds-check report of a library built with -DKVE_DEBUG
 * (libkvevict_debug.so), for the library's own tests.  That build checks every
 * global or LDS index of the select, compact and in-place kernels and of the
 * gather / hole-filling stages of the one-call triggers against its segment's
 * range before the access; an index out of range skips the access (nothing
 * traps) and sets one bit of a per-device flag word.  This call synchronises
 * the device, writes the OR of the flags set since the previous call to
 * *flags and clears them:
 *   bit 1  one-call trigger gather: a source slot outside [0, seg_len)
 *   bit 2  one-call trigger gather: an output row outside the segment's rows
 *          ([out_off, out_off + out_cap) compacting, [seg_off, seg_off + budget)
 *          hole filling)
 *   bit 3  select: a kept index at or past out_cap, or a kept slot past seg_len
 *   bit 4  compact: a kept slot outside the input rows, or a row past out_cap
 *   bit 5  in-place select: a mover outside [budget, seg_len) or a hole outside
 *          [0, budget)
 *   bit 6  one-call in-place trigger: a mover or hole list index outside its piece
 *   bit 7  one-call trigger: a kept-slot list index outside its chunk
 * Errors: EINVAL (flags NULL, or the library is not a debug build), EDEVICE
 * (the device could not be read).
 */
kve_status kve_debug_flags(uint32_t* flags);

/*
 * kve_debug_stamps — phase timestamps of a library built with -DKVE_STAMPS
 * (libkvevict_stamps.so), for measuring where the one-call trigger kernels
 * spend their time.  That build has every work-group item (ticket t, t below
 * 65536) of kv_evict_score_select_compact and
 * kv_evict_score_budget_select_compact record the memory-clock counter at
 * nine phase boundaries: 0 item taken, 1 pass 1 done, 2 first segment barrier
 * passed, 3 log-sum-exp merged, 4 pass 2 done, 5 second meeting passed (and
 * head budgets known), 6 threshold found, 7 output places ranked, 8 rows
 * gathered; the in-place kernel records phases 0-4.  This call synchronises
 * the device, copies rows 0 .. max_items-1 (9 values each, 0 where nothing was
 * recorded since the previous call) into host memory `stamps`, clears them,
 * and sets *n_rows to the rows copied and *ticks_per_us to the counter's rate.
 * Errors: EINVAL (a NULL pointer, max_items < 0, or not a KVE_STAMPS build),
 * EDEVICE (the device could not be read).
 */
kve_status kve_debug_stamps(uint64_t* stamps, int64_t max_items, int64_t* n_rows, double* ticks_per_us);

/* Message for the last non-OK status returned on the calling thread. */
const char* kve_last_error(void);

/* KVE_ABI_VERSION of the loaded library. */
int32_t kve_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVEVICT_H */
