// Protected top-K selection and gather compaction (BeaconKV, "打分时的 RoPE 对齐":
// the prefix and a short recent span are always kept and the rest of the
// budget goes to the highest scores; "📊 实验": evicted entries are dropped for
// good).
//
// select: one work-group per segment (segments longer than the LDS holds: a
// 1024-thread work-group re-reading the scores).  The K-th largest candidate score is found
// by an MSB-first radix select over order-preserving 32-bit keys (at most 8-bit
// digits over LDS histograms, starting below the leading bits that the
// candidates' minimum and maximum share); ties at the threshold go to the lower
// slots.  Kept slots are then emitted in ascending order by block-wide scans,
// 8 consecutive slots per thread and round.
// compact: a grid over (segment, share of its 128-row tiles) that gathers kept
// K/V rows with 16-byte loads and stores, and their positions.
// inplace: hole filling within the input cache (one work-group per segment).
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace kve {

namespace {

constexpr int kSelBlock = 512;
constexpr int kSelWaves = kSelBlock / kWave;

// Keys a select work-group holds in LDS (48 KB); the scores of longer segments
// are re-read from memory on each radix pass.
constexpr int kSelLdsKeys = 12288;

__global__ __launch_bounds__(kSelBlock) void select_kernel(SelectArgs a) {
  __shared__ uint32_t keys[kSelLdsKeys];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot[kSelWaves];
  __shared__ uint32_t mm[2 * kSelWaves];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;

  const int64_t oo = a.out_off[s];
  const bool out_ok = oo >= 0 && oo + a.out_cap <= a.out_rows;
  const int64_t io = a.in_off[s];
  const int n = a.in_len[s];
  const bool in_ok = n >= 0 && n <= a.in_max && io >= 0 && io + n <= a.in_rows;
  const int K = a.budget ? a.budget[s] : a.uniform_budget;
  const int P = a.n_prefix, R = a.n_recent;
  const int64_t so = a.score_off ? a.score_off[s] : io;
  const bool sc_ok = so >= 0 && so + n <= a.n_scores;
  const int keep_n = K >= n ? n : K;
  const bool bud_ok = K >= n || (K >= P + R && K >= 0);
  if (!(out_ok && in_ok && sc_ok && bud_ok) || keep_n > a.out_cap) {
    if (tid == 0) a.out_len[s] = -1;
    return;
  }
  if (K >= n) {
    for (int j = tid; j < n; j += kSelBlock) if (KVE_CHECK(j < a.out_cap, 3)) a.kept[oo + j] = j;
    if (tid == 0) a.out_len[s] = n;
    return;
  }
  const float* sc = a.scores + so;
  const bool in_lds = n <= kSelLdsKeys;
  const int c0 = P, c1 = n - R;              // candidate slots [c0, c1)
  // one read of the scores, eight loads in flight per thread (clamped
  // addresses): order keys into LDS when they fit, and the candidates' min and max
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int j0 = 0; j0 < n; j0 += 8 * kSelBlock) {
    float raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = sc[min(j0 + u * kSelBlock + tid, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kSelBlock + tid;
      if (j < n) {
        const uint32_t key = float_order_key(raw[u]);
        if (in_lds) keys[j] = key;
        if (j >= c0 && j < c1) {
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
      }
    }
  }
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  if ((tid & 63) == 0) {
    mm[tid >> 6] = kmin;
    mm[kSelWaves + (tid >> 6)] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSelWaves; ++q) {
    kmin = min(kmin, mm[q]);
    kmax = max(kmax, mm[kSelWaves + q]);
  }
  // every candidate shares the leading bits of its min and max: the radix digits start below them
  const int known = kmin == kmax ? 32 : __clz(int(kmin ^ kmax));
  uint32_t T, kk;
  radix_threshold_v<kSelBlock>(
      [&](const auto& f) {
        if (in_lds) {
          for (int j = c0 + tid; j < c1; j += kSelBlock) f(keys[j]);
        } else {
          for (int j0 = c0; j0 < c1; j0 += 8 * kSelBlock) {
            float raw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) raw[u] = sc[min(j0 + u * kSelBlock + tid, c1 - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (j0 + u * kSelBlock + tid < c1) f(float_order_key(raw[u]));
          }
        }
      },
      K - P - R, hist, sh, T, kk, kmin, known);
  // kept = protected, keys above T, and the first kk candidates equal to T, in
  // slot order; each thread takes 8 consecutive slots per round
  int base = 0, eq_seen = 0;
  for (int j0 = 0; j0 < n; j0 += 8 * kSelBlock) {
    const int jt = j0 + 8 * tid;
    uint32_t kv[8];
    if (in_lds) {
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = jt + u < n ? keys[jt + u] : 0u;
    } else {
      float raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = sc[min(jt + u, n - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = float_order_key(raw[u]);
    }
    int n_eq = 0, n_sure = 0;                  // ties at T; protected or above T
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      n_eq += cand && kv[u] == T;
      n_sure += j < n && (!cand || kv[u] > T);
    }
    int eq_tot;
    const int eq_before = eq_seen + block_scan<kSelBlock>(n_eq, wtot, eq_tot);
    const int n_keep = n_sure + min(n_eq, max(0, int(kk) - eq_before));
    int keep_tot;
    int at = base + block_scan<kSelBlock>(n_keep, wtot, keep_tot);
    int eq_rank = eq_before;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      const bool eq = cand && kv[u] == T;
      const bool keep = j < n && (!cand || kv[u] > T || (eq && eq_rank < int(kk)));
      eq_rank += eq;
      if (keep) {
        if (at < K && KVE_CHECK(at < a.out_cap && j < n, 3)) a.kept[oo + at] = j;
        ++at;
      }
    }
    base += keep_tot;
    eq_seen += eq_tot;
  }
  if (tid == 0) a.out_len[s] = K;
}

// Long segments (more keys than the LDS holds): one 1024-thread work-group per
// segment that re-reads the scores on each radix pass with sixteen loads in
// flight per thread (a 65,536-key segment is four rounds per pass), and emits
// the kept slots 8 consecutive slots per thread and round.
constexpr int kLongBlock = 1024;
constexpr int kLongUnr = 16;

__global__ __launch_bounds__(kLongBlock) void select_long_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot[kLongBlock / kWave];
  __shared__ uint32_t mm[2 * (kLongBlock / kWave)];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t oo = a.out_off[s];
  const bool out_ok = oo >= 0 && oo + a.out_cap <= a.out_rows;
  const int64_t io = a.in_off[s];
  const int n = a.in_len[s];
  const bool in_ok = n >= 0 && n <= a.in_max && io >= 0 && io + n <= a.in_rows;
  const int K = a.budget ? a.budget[s] : a.uniform_budget;
  const int P = a.n_prefix, R = a.n_recent;
  const int64_t so = a.score_off ? a.score_off[s] : io;
  const bool sc_ok = so >= 0 && so + n <= a.n_scores;
  const int keep_n = K >= n ? n : K;
  const bool bud_ok = K >= n || (K >= P + R && K >= 0);
  if (!(out_ok && in_ok && sc_ok && bud_ok) || keep_n > a.out_cap) {
    if (tid == 0) a.out_len[s] = -1;
    return;
  }
  if (K >= n) {
    for (int j = tid; j < n; j += kLongBlock) if (KVE_CHECK(j < a.out_cap, 3)) a.kept[oo + j] = j;
    if (tid == 0) a.out_len[s] = n;
    return;
  }
  const float* sc = a.scores + so;
  const int c0 = P, c1 = n - R;              // candidate slots [c0, c1)
  // visit the candidates' keys, kLongUnr loads in flight per thread (clamped addresses)
  auto visit_all = [&](const auto& f) {
    for (int b0 = c0; b0 < c1; b0 += kLongUnr * kLongBlock) {
      float raw[kLongUnr];
#pragma unroll
      for (int u = 0; u < kLongUnr; ++u) raw[u] = sc[min(b0 + u * kLongBlock + tid, c1 - 1)];
#pragma unroll
      for (int u = 0; u < kLongUnr; ++u)
        if (b0 + u * kLongBlock + tid < c1) f(float_order_key(raw[u]));
    }
  };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  visit_all([&](uint32_t key) {
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  });
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  constexpr int NW = kLongBlock / kWave;
  if ((tid & 63) == 0) {
    mm[tid >> 6] = kmin;
    mm[NW + (tid >> 6)] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    kmin = min(kmin, mm[q]);
    kmax = max(kmax, mm[NW + q]);
  }
  const int known = kmin == kmax ? 32 : __clz(int(kmin ^ kmax));
  uint32_t T, kk;
  radix_threshold_v<kLongBlock>(visit_all, K - P - R, hist, sh, T, kk, kmin, known);
  // kept = protected, keys above T, and the first kk candidates equal to T, in
  // slot order; each thread takes 8 consecutive slots per round
  int base = 0, eq_seen = 0;
  for (int r0 = 0; r0 < n; r0 += 8 * kLongBlock) {
    const int jt = r0 + 8 * tid;
    float raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = sc[min(jt + u, n - 1)];
    uint32_t kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = float_order_key(raw[u]);
    int n_eq = 0, n_sure = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      n_eq += cand && kv[u] == T;
      n_sure += j < n && (!cand || kv[u] > T);
    }
    int eq_tot;
    const int eq_before = eq_seen + block_scan<kLongBlock>(n_eq, wtot, eq_tot);
    const int n_keep = n_sure + min(n_eq, max(0, int(kk) - eq_before));
    int keep_tot;
    int at = base + block_scan<kLongBlock>(n_keep, wtot, keep_tot);
    int eq_rank = eq_before;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      const bool eq = cand && kv[u] == T;
      const bool keep = j < n && (!cand || kv[u] > T || (eq && eq_rank < int(kk)));
      eq_rank += eq;
      if (keep) {
        if (at < K && KVE_CHECK(at < a.out_cap && j < n, 3)) a.kept[oo + at] = j;
        ++at;
      }
    }
    base += keep_tot;
    eq_seen += eq_tot;
  }
  if (tid == 0) a.out_len[s] = K;
}

// Few long segments (the 65k workload has 32): one work-group per segment
// would leave most CUs idle, so G work-groups share each segment, each
// holding 1/G of its candidates.  Every digit pass's histogram is summed over
// the segment's work-groups in a per-segment control block with device-scope
// atomics, and the work-groups meet at a per-segment arrival counter after
// each sum (bounded polling).  Work-groups take their (segment, slice) from
// one ticket counter in launch order, so a waiting work-group only ever waits
// for slices of its own segment, all of them taken by running work-groups but
// at most G - 1 of the newest segment; on an idle device the whole launch (at
// most kSplitMaxWg work-groups, one per CU) is resident at once.  A last exchange of each work-group's
// kept and tied counts gives every work-group the kept rows before its slice
// of slots, which it then lists like the one-work-group form.  The segment's
// length is published by its last work-group to finish, so a segment whose
// work-groups did not all meet keeps -1.
// Control block of a segment (kSplitCtl ints): [0] arrivals, [1] finished
// work-groups, [2] / [3] the candidates' smallest / largest key, [8 + 2g] /
// [9 + 2g] work-group g's kept-for-sure / tied slot counts, [64 + 256p + d]
// the pass-p histogram.  One more int after the last block: the ticket counter.
constexpr int kSplitMaxWg = 256;
constexpr int kSplitMaxG = 16;
constexpr int kSplitHist = 64;
constexpr int kSplitCtl = kSplitHist + 4 * 256;

__device__ __forceinline__ int load_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 only: count this work-group in and poll until `target` arrivals,
// for at most `limit` polls; on a timeout push the counter far below any
// target, so that no work-group of the segment passes a later meeting.
__device__ __forceinline__ bool split_meet(int* arrive, int target, int limit) {
  atomicAdd(arrive, 1);
  int spins = 0;
  while (load_agent(arrive) < target && ++spins < limit) __builtin_amdgcn_s_sleep(1);
  if (spins < limit) return true;
  atomicAdd(arrive, -(1 << 24));
  return false;
}

__global__ void split_ctl_init_kernel(int* ctl, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) ctl[i] = i % kSplitCtl == 2 ? -1 : 0;    // [2] holds a minimum: all bits set
}

__global__ __launch_bounds__(kLongBlock) void select_split_kernel(SelectArgs a, int G) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot[kLongBlock / kWave];
  __shared__ uint32_t mm[2 * (kLongBlock / kWave)];
  __shared__ int met;
  const int tid = threadIdx.x;
  if (tid == 0) met = atomicAdd(&a.split_ctl[int64_t(a.n_seg) * kSplitCtl], 1);
  __syncthreads();
  const int item = met;
  __syncthreads();
  const int s = item / G, g = item % G;
  int* ctl = a.split_ctl + int64_t(s) * kSplitCtl;
  const int64_t oo = a.out_off[s];
  const bool out_ok = oo >= 0 && oo + a.out_cap <= a.out_rows;
  const int64_t io = a.in_off[s];
  const int n = a.in_len[s];
  const bool in_ok = n >= 0 && n <= a.in_max && io >= 0 && io + n <= a.in_rows;
  const int K = a.budget ? a.budget[s] : a.uniform_budget;
  const int P = a.n_prefix, R = a.n_recent;
  const int64_t so = a.score_off ? a.score_off[s] : io;
  const bool sc_ok = so >= 0 && so + n <= a.n_scores;
  const int keep_n = K >= n ? n : K;
  const bool bud_ok = K >= n || (K >= P + R && K >= 0);
  // every work-group of the segment takes the same branch below
  if (!(out_ok && in_ok && sc_ok && bud_ok) || keep_n > a.out_cap) {
    if (g == 0 && tid == 0) __hip_atomic_store(&a.out_len[s], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int ls = (n + G - 1) / G;                      // this work-group's slots [s0, s1)
  const int s0 = min(n, g * ls), s1 = min(n, s0 + ls);
  if (K >= n) {
    for (int j = s0 + tid; j < s1; j += kLongBlock) if (KVE_CHECK(j < a.out_cap, 3)) a.kept[oo + j] = j;
    if (g == 0 && tid == 0) __hip_atomic_store(&a.out_len[s], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (g == 0 && tid == 0) __hip_atomic_store(&a.out_len[s], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float* sc = a.scores + so;
  const int c0 = P, c1 = n - R;                      // candidate slots; this work-group's [b0, b1)
  const int lc = (c1 - c0 + G - 1) / G;
  const int b0 = min(c1, c0 + g * lc), b1 = min(c1, b0 + lc);
  auto visit = [&](const auto& f) {
    for (int j0 = b0; j0 < b1; j0 += kLongUnr * kLongBlock) {
      float raw[kLongUnr];
#pragma unroll
      for (int u = 0; u < kLongUnr; ++u) raw[u] = sc[min(j0 + u * kLongBlock + tid, b1 - 1)];
#pragma unroll
      for (int u = 0; u < kLongUnr; ++u)
        if (j0 + u * kLongBlock + tid < b1) f(float_order_key(raw[u]));
    }
  };
  int meetings = 0;
  // every thread; true when all G work-groups are in.  The device-scope
  // atomics and coherent stores before it are acknowledged first (a fence
  // would also write back and invalidate the whole L2).
  auto meet = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ++meetings;
    if (tid == 0) met = split_meet(&ctl[0], meetings * G, a.spin_limit);
    __syncthreads();
    return met != 0;
  };
  // the candidates' key range over the whole segment
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  visit([&](uint32_t key) {
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  });
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  constexpr int NW = kLongBlock / kWave;
  if ((tid & 63) == 0) {
    mm[tid >> 6] = kmin;
    mm[NW + (tid >> 6)] = kmax;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      kmin = min(kmin, mm[q]);
      kmax = max(kmax, mm[NW + q]);
    }
    atomicMin(reinterpret_cast<unsigned*>(&ctl[2]), kmin);
    atomicMax(reinterpret_cast<unsigned*>(&ctl[3]), kmax);
  }
  if (!meet()) return;
  kmin = uint32_t(load_agent(&ctl[2]));
  kmax = uint32_t(load_agent(&ctl[3]));
  const int known = kmin == kmax ? 32 : __clz(int(kmin ^ kmax));
  int pass = 0;
  auto merge = [&](uint32_t* h) {
    int* gh = &ctl[kSplitHist + 256 * pass++];
    if (tid < 256 && h[tid] != 0) atomicAdd(&gh[tid], int(h[tid]));
    if (!meet()) return false;
    if (tid < 256) h[tid] = uint32_t(load_agent(&gh[tid]));
    __syncthreads();
    return true;
  };
  uint32_t T, kk;
  if (!radix_threshold_v<kLongBlock>(visit, K - P - R, hist, sh, T, kk, kmin, known, merge)) return;
  // this work-group's slots kept for sure (protected, or above T) and tied at T
  int n_sure = 0, n_eq = 0;
  for (int j0 = s0; j0 < s1; j0 += kLongUnr * kLongBlock) {
    float raw[kLongUnr];
#pragma unroll
    for (int u = 0; u < kLongUnr; ++u) raw[u] = sc[min(j0 + u * kLongBlock + tid, s1 - 1)];
#pragma unroll
    for (int u = 0; u < kLongUnr; ++u) {
      const int j = j0 + u * kLongBlock + tid;
      const bool cand = j >= c0 && j < c1;
      const uint32_t key = float_order_key(raw[u]);
      n_sure += j < s1 && (!cand || key > T);
      n_eq += j < s1 && cand && key == T;
    }
  }
  n_sure = block_sum<kLongBlock>(n_sure, wtot);
  n_eq = block_sum<kLongBlock>(n_eq, wtot);
  if (tid == 0) {
    __hip_atomic_store(&ctl[8 + 2 * g], n_sure, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctl[9 + 2 * g], n_eq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!meet()) return;
  int base = 0, eq_seen = 0;                         // kept and tied slots before this work-group's
  for (int q = 0; q < g; ++q) {
    const int eq_q = load_agent(&ctl[9 + 2 * q]);
    base += load_agent(&ctl[8 + 2 * q]) + min(eq_q, max(0, int(kk) - eq_seen));
    eq_seen += eq_q;
  }
  // list this work-group's kept slots, 8 consecutive per thread and round
  for (int r0 = s0; r0 < s1; r0 += 8 * kLongBlock) {
    const int jt = r0 + 8 * tid;
    float raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = sc[min(jt + u, s1 - 1)];
    uint32_t kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = float_order_key(raw[u]);
    int r_eq = 0, r_sure = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      r_eq += j < s1 && cand && kv[u] == T;
      r_sure += j < s1 && (!cand || kv[u] > T);
    }
    int eq_tot;
    const int eq_before = eq_seen + block_scan<kLongBlock>(r_eq, wtot, eq_tot);
    const int r_keep = r_sure + min(r_eq, max(0, int(kk) - eq_before));
    int keep_tot;
    int at = base + block_scan<kLongBlock>(r_keep, wtot, keep_tot);
    int eq_rank = eq_before;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= c0 && j < c1;
      const bool eq = j < s1 && cand && kv[u] == T;
      const bool keep = j < s1 && (!cand || kv[u] > T || (eq && eq_rank < int(kk)));
      eq_rank += eq;
      if (keep) {
        if (at < K && KVE_CHECK(at < a.out_cap && j < n, 3)) a.kept[oo + at] = j;
        ++at;
      }
    }
    base += keep_tot;
    eq_seen += eq_tot;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0 && atomicAdd(&ctl[1], 1) == G - 1)
    __hip_atomic_store(&a.out_len[s], K, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Gather kept rows.  CPR 16-byte chunks per row; each thread moves UNR rows of
// K and V per pass (all loads issued before the stores), a tile is PASSES
// passes, and a work-group takes every gridDim.x-th tile of its segment.  Loads
// and stores are non-temporal: every byte is touched exactly once.
#ifndef KVE_COMPACT_UNR
#define KVE_COMPACT_UNR 4
#endif
#ifndef KVE_COMPACT_PASSES
#define KVE_COMPACT_PASSES 2
#endif
constexpr int kCompactUnr = KVE_COMPACT_UNR;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCompactPasses = KVE_COMPACT_PASSES;

template <int CPR>
__global__ __launch_bounds__(256) void compact_kernel(SelectArgs a) {
  constexpr int RPP = 256 / CPR;            // rows per sub-pass
  constexpr int UNR = kCompactUnr;
  constexpr int RPW = RPP * UNR * kCompactPasses;
  const int s = blockIdx.y;
  const int out_n = a.out_len[s];
  if (out_n <= 0 || out_n > a.out_cap || int(blockIdx.x) * RPW >= out_n) return;
  const int64_t io = a.in_off[s], oo = a.out_off[s];
  const int n_in = a.in_len[s];
  const int part = threadIdx.x % CPR;
  const int rsub = threadIdx.x / CPR;
  const u32x4* kin = static_cast<const u32x4*>(a.k_in);
  const u32x4* vin = static_cast<const u32x4*>(a.v_in);
  u32x4* kout = static_cast<u32x4*>(a.k_out);
  u32x4* vout = static_cast<u32x4*>(a.v_out);
  for (int rw = blockIdx.x * RPW; rw < out_n; rw += gridDim.x * RPW) {
    for (int p = 0; p < kCompactPasses; ++p) {
      const int r0 = rw + p * RPP * UNR;
      if (r0 >= out_n) break;
      u32x4 kb[UNR], vb[UNR];
      int src[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * RPP + rsub;
        int j = r < out_n ? a.kept[oo + r] : -1;
        if (j >= n_in) j = -1;
        if (j >= 0 && !KVE_CHECK(io + j < a.in_rows && r < a.out_cap, 4)) j = -1;
        src[u] = j;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (src[u] >= 0) {
          kb[u] = __builtin_nontemporal_load(&kin[(io + src[u]) * CPR + part]);
          vb[u] = __builtin_nontemporal_load(&vin[(io + src[u]) * CPR + part]);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * RPP + rsub;
        if (src[u] >= 0) {
          __builtin_nontemporal_store(kb[u], &kout[(oo + r) * CPR + part]);
          __builtin_nontemporal_store(vb[u], &vout[(oo + r) * CPR + part]);
          if (part == 0) a.pos_out[oo + r] = a.pos_in[io + src[u]];
        }
      }
    }
  }
}

template <int CPR>
hipError_t launch_compact(const SelectArgs& a, hipStream_t st) {
  constexpr int RPW = (256 / CPR) * kCompactUnr * kCompactPasses;
  // work-groups per segment: one per RPW-row tile when a uniform budget fixes
  // the kept counts; with per-segment budgets (known only on the device),
  // enough for about 32K work-groups in all, each looping over its share of
  // the segment's tiles, so that few are idle when the kept counts are far
  // below the output capacity
  const int tiles = (a.out_cap + RPW - 1) / RPW;
  const int per_seg = !a.budget ? (min(a.uniform_budget, a.out_cap) + RPW - 1) / RPW
                                : max(1, min(tiles, (32768 + a.n_seg - 1) / a.n_seg));
  if (per_seg <= 0) return hipSuccess;
  const dim3 grid(unsigned(per_seg), unsigned(a.n_seg));
  hipLaunchKernelGGL(compact_kernel<CPR>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// In-place compaction by hole filling, one work-group per segment: the same
// protected top-K threshold as select_kernel, then the survivors in [K, n)
// move, in ascending order, into the evicted slots of [0, K), in ascending
// order (survivors below K stay).  Slots are ranked block by block (512 at a
// time) into two short lists in LDS, pending holes and pending movers, which
// are paired and copied as they fill; at most min(K, n - K) rows move.  Mover
// rows are only read and hole rows only written, so no row is both.
template <int CPR>
__global__ __launch_bounds__(kSelBlock) void inplace_kernel(SelectArgs a) {
  constexpr int RPP = kSelBlock / CPR;      // rows per copy pass
  constexpr int UNR = 4;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot_a[kSelWaves], wtot_b[kSelWaves];
  __shared__ int hl[kSelBlock], ml[kSelBlock];   // pending holes / movers (slots), ascending
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t io = a.in_off[s];
  const int n = a.in_len[s];
  const bool in_ok = n >= 0 && n <= a.in_max && io >= 0 && io + n <= a.in_rows;
  const int K = a.budget ? a.budget[s] : a.uniform_budget;
  const int P = a.n_prefix, R = a.n_recent;
  const int64_t so = a.score_off ? a.score_off[s] : io;
  const bool sc_ok = so >= 0 && so + n <= a.n_scores;
  const bool bud_ok = K >= n || (K >= P + R && K >= 0);
  if (!(in_ok && sc_ok && bud_ok)) {
    if (tid == 0) a.out_len[s] = -1;
    return;
  }
  if (K >= n) {                              // every row survives where it is
    if (tid == 0) a.out_len[s] = n;
    return;
  }
  const float* sc = a.scores + so;
  auto key_at = [&](int j) { return float_order_key(sc[j]); };
  uint32_t T, kk;
  radix_threshold<kSelBlock>(key_at, P, n, R, K - P - R, hist, sh, T, kk);
  // candidates equal to T below K: the tie rank the mover scan starts from
  int eq_lo = 0;
  for (int j = P + tid; j < min(K, n - R); j += kSelBlock) eq_lo += key_at(j) == T;
  eq_lo = block_sum<kSelBlock>(eq_lo, wtot_a);

  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4* kc = static_cast<u32x4*>(a.k_out);
  u32x4* vc = static_cast<u32x4*>(a.v_out);
  const int part = tid % CPR, rsub = tid / CPR;
  // one block of slots [j0, j1): keep flags with running tie ranks; returns
  // this thread's flag for "wanted" (a hole below K or a survivor at or above K)
  auto scan_block = [&](int j0, int j1, int& eq_seen, bool want_kept, int* list, int& count) {
    const int j = j0 + tid;
    const bool in = j < j1;
    const bool cand = in && j >= P && j < n - R;
    const uint32_t key = cand ? key_at(j) : 0u;
    const bool eq = cand && key == T;
    int eq_tot;
    const int eq_rank = eq_seen + block_flag_scan<kSelBlock>(eq, wtot_a, eq_tot);
    const bool keep = !cand || key > T || (eq && uint32_t(eq_rank) < kk);
    const bool want = in && (keep == want_kept);
    int tot;
    const int at = block_flag_scan<kSelBlock>(want, wtot_b, tot);
    if (want) list[at] = j;
    count = tot;
    eq_seen += eq_tot;
  };
  int hc = 0, h_eq = 0, nH = 0;              // holes: next slot to scan, ties seen, pending
  int mc = K, m_eq = eq_lo, nM = 0;          // movers
  for (;;) {
    if (nH == 0 && hc < K) {
      scan_block(hc, min(hc + kSelBlock, K), h_eq, false, hl, nH);
      hc = min(hc + kSelBlock, K);
    }
    if (nM == 0 && mc < n) {
      scan_block(mc, min(mc + kSelBlock, n), m_eq, true, ml, nM);
      mc = min(mc + kSelBlock, n);
    }
    __syncthreads();
    if (nH == 0 || nM == 0) {
      if ((nH == 0 && hc >= K) || (nM == 0 && mc >= n)) break;
      continue;
    }
    const int p = min(nH, nM);
    for (int r0 = 0; r0 < p; r0 += RPP * UNR) {
      u32x4 kb[UNR], vb[UNR];
      int src[UNR], dst[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + u * RPP + rsub;
        src[u] = r < p ? ml[r] : -1;
        dst[u] = r < p ? hl[r] : -1;
        if (src[u] >= 0 && !KVE_CHECK(dst[u] >= 0 && dst[u] < K && src[u] >= K && src[u] < n, 5))
          src[u] = -1;
        if (src[u] >= 0) {
          kb[u] = __builtin_nontemporal_load(&kc[(io + src[u]) * CPR + part]);
          vb[u] = __builtin_nontemporal_load(&vc[(io + src[u]) * CPR + part]);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (src[u] >= 0) {
          __builtin_nontemporal_store(kb[u], &kc[(io + dst[u]) * CPR + part]);
          __builtin_nontemporal_store(vb[u], &vc[(io + dst[u]) * CPR + part]);
          if (part == 0) a.pos_out[io + dst[u]] = a.pos_in[io + src[u]];
        }
    }
    // drop the p paired entries from both lists
    const int h_rest = tid < nH - p ? hl[p + tid] : 0;
    const int m_rest = tid < nM - p ? ml[p + tid] : 0;
    __syncthreads();
    if (tid < nH - p) hl[tid] = h_rest;
    if (tid < nM - p) ml[tid] = m_rest;
    nH -= p;
    nM -= p;
    __syncthreads();
  }
  if (tid == 0) a.out_len[s] = K;
}

}  // namespace

hipError_t launch_select_inplace(const SelectArgs& a, hipStream_t st) {
  if (a.n_seg == 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_seg));
  switch (a.head_dim * a.elem_bytes / 16) {
    case 8: hipLaunchKernelGGL(inplace_kernel<8>, grid, dim3(kSelBlock), 0, st, a); break;
    case 16: hipLaunchKernelGGL(inplace_kernel<16>, grid, dim3(kSelBlock), 0, st, a); break;
    case 32: hipLaunchKernelGGL(inplace_kernel<32>, grid, dim3(kSelBlock), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t split_ctl_ints(int32_t n_seg) {
  return n_seg > 0 && 2 * n_seg <= kSplitMaxWg ? size_t(n_seg) * kSplitCtl + 1 : 0;
}

hipError_t launch_select_compact(const SelectArgs& a, hipStream_t st) {
  if (a.n_seg == 0) return hipSuccess;
  const int G = min(kSplitMaxG, kSplitMaxWg / a.n_seg);
  if (a.in_max > kSelLdsKeys && a.split_ctl && G >= 2) {
    const int64_t nc = int64_t(a.n_seg) * kSplitCtl + 1;
    hipLaunchKernelGGL(split_ctl_init_kernel, dim3(unsigned((nc + 255) / 256)), dim3(256), 0, st, a.split_ctl, nc);
    hipLaunchKernelGGL(select_split_kernel, dim3(unsigned(a.n_seg * G)), dim3(kLongBlock), 0, st, a, G);
  } else if (a.in_max > kSelLdsKeys)
    hipLaunchKernelGGL(select_long_kernel, dim3(unsigned(a.n_seg)), dim3(kLongBlock), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel, dim3(unsigned(a.n_seg)), dim3(kSelBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.out_cap == 0) return e;
  const int cpr = a.head_dim * a.elem_bytes / 16;
  switch (cpr) {
    case 8: return launch_compact<8>(a, st);
    case 16: return launch_compact<16>(a, st);
    case 32: return launch_compact<32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

unsigned int debug_take_select() {
#ifdef KVE_DEBUG
  unsigned int v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kve_debug_word), sizeof(v)) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(kve_debug_word), &z, sizeof(z)) != hipSuccess) return ~0u;
  return v;
#else
  return 0;
#endif
}

}  // namespace kve
