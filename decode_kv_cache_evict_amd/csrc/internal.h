// Launch interfaces between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kve {

constexpr int kScoreChunk = 256;   // keys per work-group, VALU path (one key per thread)
constexpr int kMfmaChunk = 1024;   // keys per work-group, MFMA path
constexpr int kMaxObsRows = 256;   // group * max_obs

struct ScoreArgs {
  // cache
  const void* k;
  const int32_t* pos;
  const int64_t* seg_off;
  const int32_t* seg_len;
  int64_t n_rows;
  int32_t n_seg, n_kv, max_seg_len, head_dim, dtype;
  // observation queries
  const void* q;          // pre-RoPE [B, Hq, max_obs, D]
  const int32_t* q_pos;   // [B, max_obs]
  const int32_t* n_obs;   // [B] or null
  int32_t n_q, max_obs, group, rows, causal;
  int32_t aggregate;      // 0: max over the observation rows, 1: mean
  double theta;
  // outputs and workspace
  float* scores;
  float* entropy;
  void* qr;               // rotated queries [B, Hq, max_obs, D] (workspace)
  float2* stats;          // [n_seg, n_chunks, rows] (m * log2e/sqrt(D), l) (workspace)
  float* lse;             // [n_seg, rows] merged row log-sum-exp, log2 units (workspace)
  int32_t n_chunks;
  int32_t chunk;          // keys per work-group
  int32_t impl;           // 0: two-pass MFMA, 1: plain VALU, 2: single-read MFMA
  int32_t spin_limit;     // polls at a segment barrier (single-read kernels) before giving up
  // fused score -> select -> compact (kv_evict_score_select_compact) only
  const void* v;
  void* k_out; void* v_out; int32_t* pos_out;
  const int64_t* out_off; int32_t* out_len; int64_t out_rows; int32_t out_cap;
  int32_t* kept;          // optional, aligned with output rows
  const int32_t* budget;  // [n_seg] or null
  int32_t uniform_budget, n_prefix, n_recent;
  int32_t inplace;        // 1: hole filling within the input cache (k_out = k, out_len = new lengths)
  // entropy budgets in the one-kernel trigger (kv_evict_score_budget_select_compact) only
  const int32_t* layer_total;  // [n_seg / n_kv] request-layer totals
  int32_t min_per_head, ent_form;  // ent_form 1: weights 1 - entropy
  int32_t* budget_out;    // [n_seg] or null
};

// Largest segment the one-kernel step can select on chip: its order keys reuse the
// two 64-key tiles of padded bf16 rows (64 * (D + 16) 32-bit words).
constexpr int step_max_seg(int head_dim) { return 64 * (head_dim + 16); }
hipError_t launch_score_select_compact(ScoreArgs& a, void* ws, hipStream_t st);
// Static device scratch of kv_evict_score_select_compact_noalloc: its size,
// and its address on the current device (taken once per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);
// Debug build (KVE_DEBUG) only: read and clear the bounds-check flag word of
// the score / select kernel files (0 in the regular build, ~0u when the copy fails).
unsigned int debug_take_score();
// Phase-stamp build (KVE_STAMPS) only: copy up to n_items rows of
// kStampPhases memory-clock stamps of the one-call trigger's work-group items
// into host memory and clear them; returns the rows copied (-1 on a copy
// failure, 0 in the other builds).
constexpr int kStampPhases = 9;
int64_t debug_take_stamps(unsigned long long* host, int64_t n_items);
unsigned int debug_take_select();
// The one-kernel trigger with entropy budgets applies when every
// request-layer's work-groups fit the dispatch bound of its barrier.
bool budget_step_fits(int32_t n_seg, int32_t n_kv, int32_t max_seg_len, int32_t head_dim);
hipError_t launch_score_budget_select_compact(ScoreArgs& a, void* ws, hipStream_t st);

size_t score_workspace_bytes(int32_t batch, int32_t n_q, int32_t max_obs, int32_t head_dim, int32_t dtype,
                             int32_t n_seg, int32_t max_seg_len, int32_t rows);
hipError_t launch_score(ScoreArgs& a, void* ws, hipStream_t st);

struct SelectArgs {
  // input cache
  const void* k_in; const void* v_in; const int32_t* pos_in;
  const int64_t* in_off; const int32_t* in_len; int64_t in_rows; int32_t in_max;
  // scores
  const float* scores; const int64_t* score_off; int64_t n_scores;
  // budgets
  const int32_t* budget; int32_t uniform_budget; int32_t n_prefix, n_recent;
  // output cache
  void* k_out; void* v_out; int32_t* pos_out;
  const int64_t* out_off; int32_t* out_len; int64_t out_rows; int32_t out_cap;
  int32_t* kept;          // [out_rows]
  int32_t n_seg, head_dim, elem_bytes;
  int32_t* split_ctl;     // split_ctl_ints(n_seg) ints of workspace, or null (long segments, one work-group each)
  int32_t spin_limit;     // polls at a segment barrier before giving up
};
// Control ints the selection of few long segments over several work-groups
// per segment needs (0: that form is not used for n_seg segments).
size_t split_ctl_ints(int32_t n_seg);
hipError_t launch_select_compact(const SelectArgs& a, hipStream_t st);
// In place: k_out/v_out/pos_out are the input cache; out_len receives the new lengths.
hipError_t launch_select_inplace(const SelectArgs& a, hipStream_t st);

// weight_form 0: weights as given; 1: 1 - weight (inverse entropy).
hipError_t launch_budgets(const float* w, const int32_t* total, const int32_t* cap, int32_t batch,
                          int32_t n_heads, int32_t min_per_head, int32_t* out, hipStream_t st, int weight_form = 0);
hipError_t launch_wave_budgets(int32_t n_layers, double center, double sigma, int32_t total, int32_t lo,
                               int32_t* out, hipStream_t st);

hipError_t launch_fps(const void* q_in, void* q_out, const int32_t* count_in, int32_t* count_out,
                      int32_t n_buf, int32_t cap, int32_t k_keep, int32_t head_dim, int32_t dtype,
                      int32_t* picks, hipStream_t st);

size_t epikv_ws_bytes(int32_t batch, int32_t T);
// form 0: z_a - z_b; 1: rolling mean g_bar_a - g_bar_b.
hipError_t launch_epikv(const void* h_a, const void* h_b, int32_t batch, int32_t T, int32_t d_model,
                        int32_t window, float eps, int32_t form, float* g_out, float* scores, void* ws, hipStream_t st);

struct AttnArgs {
  const void* k; const void* v;
  const int64_t* seg_off; const int32_t* seg_len;
  int64_t n_rows; int32_t n_seg, n_kv, max_seg_len, head_dim, dtype;
  const void* q;          // [B, n_q, head_dim] rotated queries of the new token, cache dtype
  int32_t n_q, group;
  float* out;             // [B, n_q, head_dim]
  float* lse;             // [B, n_q] or null
  float* part;            // [n_seg, n_chunks, group, head_dim + 2] workspace
  int32_t n_chunks;
};
size_t attn_workspace_bytes(int32_t n_seg, int32_t max_seg_len, int32_t group, int32_t head_dim);
hipError_t launch_decode_attention(AttnArgs& a, hipStream_t st);

struct SkipArgs {
  const void* h;          // [batch, T, d_model] bf16 last-layer hidden states
  const int32_t* starts;  // [batch, max_sent + 1] sentence boundaries
  const int32_t* n_sent;  // [batch] complete sentences
  int32_t batch, T, d_model, max_sent;
  float tau;
  float* pss_max;         // [batch, max_sent]
  int32_t* marks;         // [batch, max_sent] or null
  float* token_scores;    // [batch, T]
  float* emb;             // [batch, max_sent, d_model] unit sentence means (workspace)
  uint32_t* pss_key;      // [batch, max_sent] order keys of the running maxima (workspace)
};
size_t skipkv_ws_bytes(int32_t batch, int32_t max_sent, int32_t d_model);
hipError_t launch_skipkv(SkipArgs& a, void* ws, hipStream_t st);

hipError_t launch_rope_rows(const float* src, void* dst, const int32_t* pos, int64_t n_rows, int32_t head_dim,
                            double theta, int32_t dtype, hipStream_t st);

}  // namespace kve
