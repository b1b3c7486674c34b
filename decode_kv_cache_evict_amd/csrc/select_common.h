// Block-level pieces of the protected top-K selection, shared by the stand-alone
// select kernel and the fused score-select-compact kernel.
#pragma once

#include "common.h"

namespace kve {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (uint64_t(1) << lane) - 1; }

// Exclusive block scan of a 0/1 flag over BLOCK threads; returns this thread's
// prefix and sets `total`.  wtot: BLOCK/64 ints of LDS.
template <int BLOCK>
__device__ __forceinline__ int block_flag_scan(bool f, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const int in_wave = __popcll(m & lanemask_lt(lane));
  if (lane == 0) wtot[w] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < BLOCK / kWave; ++q) {
    const int t = wtot[q];
    before += q < w ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + in_wave;
}

// Exclusive block scan of a non-negative int over BLOCK threads; returns this
// thread's prefix and sets `total`.  wtot: BLOCK/64 ints of LDS.
template <int BLOCK>
__device__ __forceinline__ int block_scan(int x, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(x);
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < BLOCK / kWave; ++q) {
    const int t = wtot[q];
    before += q < w ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - x;
}

// Block sum of an int over BLOCK threads (wtot: BLOCK/64 ints of LDS).
template <int BLOCK>
__device__ __forceinline__ int block_sum(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_reduce(v, [](int x, int y) { return x + y; });
  if (lane == 0) wtot[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int q = 0; q < BLOCK / kWave; ++q) t += wtot[q];
  __syncthreads();
  return t;
}

// Row gather of a 256-thread work-group: output rows dst_at(r) <- input rows
// in_off + src_at(r) for r in [0, cnt), K and V (CPR 16-byte chunks per row)
// and the position; kept_out[dst_at(r)] = src_at(r) when kept_out is set.
// src_at and dst_at read LDS or registers (they must not issue memory loads).
// The debug build checks every source slot against [0, src_n) and every
// output row against [dst_lo, dst_hi).  GU rows per thread and batch, four batches in registers: the memory counter retires loads and
// stores in issue order and a batch's registers may only be reloaded once its
// stores are done, so the loads run two batches ahead of the stores and a
// batch is reloaded two batches after its stores, which leaves two batches in
// flight at every wait.  Loads past the last row repeat it (no branch).
// Every access is non-temporal: the rows are not touched again here, and
// keeping them out of L2 leaves it to the scoring passes of other work-groups.
template <int CPR, int GU = 2, typename SrcAt, typename DstAt>
__device__ __forceinline__ void gather_rows(const SrcAt& src_at, const DstAt& dst_at, int cnt, const void* k,
                                            const void* v, const int32_t* pos, int64_t in_off, void* k_out,
                                            void* v_out, int32_t* pos_out, int32_t* kept_out, int tid,
                                            int src_n, int64_t dst_lo, int64_t dst_hi) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int RPP = 256 / CPR;             // rows per thread-row
  constexpr int STEP = RPP * GU;
  if (cnt <= 0) return;
  const u32x4* kin = static_cast<const u32x4*>(k);
  const u32x4* vin = static_cast<const u32x4*>(v);
  u32x4* kout = static_cast<u32x4*>(k_out);
  u32x4* vout = static_cast<u32x4*>(v_out);
  const int part = tid % CPR, rsub = tid / CPR;
  struct Batch {
    u32x4 k[GU], v[GU];
    int src[GU], pos[GU];
  };
  auto load = [&](Batch& bt, int r0) {
#pragma unroll
    for (int u = 0; u < GU; ++u) bt.src[u] = src_at(min(r0 + u * RPP + rsub, cnt - 1));
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      if (!KVE_CHECK(bt.src[u] >= 0 && bt.src[u] < src_n, 1)) continue;
      bt.k[u] = __builtin_nontemporal_load(&kin[(in_off + bt.src[u]) * CPR + part]);
      bt.v[u] = __builtin_nontemporal_load(&vin[(in_off + bt.src[u]) * CPR + part]);
      bt.pos[u] = pos[in_off + bt.src[u]];
    }
  };
  auto store = [&](const Batch& bt, int r0) {
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int r = r0 + u * RPP + rsub;
      if (r < cnt) {
        const int64_t dst = dst_at(r);
        if (!KVE_CHECK(dst >= dst_lo && dst < dst_hi, 2)) continue;
        __builtin_nontemporal_store(bt.k[u], &kout[dst * CPR + part]);
        __builtin_nontemporal_store(bt.v[u], &vout[dst * CPR + part]);
        if (part == 0) {
          pos_out[dst] = bt.pos[u];
          if (kept_out) kept_out[dst] = bt.src[u];
        }
      }
    }
  };
  Batch b0, b1, b2, b3;
  load(b0, 0);
  load(b1, STEP);
  for (int r0 = 0; r0 < cnt; r0 += 4 * STEP) {
    load(b2, r0 + 2 * STEP);
    store(b0, r0);
    load(b3, r0 + 3 * STEP);
    store(b1, r0 + STEP);
    if (r0 + 2 * STEP >= cnt) break;
    load(b0, r0 + 4 * STEP);
    store(b2, r0 + 2 * STEP);
    load(b1, r0 + 5 * STEP);
    store(b3, r0 + 3 * STEP);
  }
}

// Threshold of a top-kc selection: find the kc-th largest order key T among the
// candidate keys of the work-group (MSB-first radix select over LDS histograms
// of at most 8-bit digits) and kk, the number of candidates equal to T that
// are kept.  visit(f) calls f(key) once for every candidate key this thread
// holds; every thread must visit the same keys on each call.  The caller may
// pass the number of leading bits `known` (0..32) that every candidate shares
// with `prefix` (e.g. the common prefix of the candidates' minimum and
// maximum); the digits then start below them.  kc == 0 gives T = 0xFFFFFFFF,
// kk = 0.  When the digit that holds the kc-th key is kept whole (its count is
// exactly what is still needed), the passes stop there with T one below the
// digit's smallest possible key and kk = 0: the same kept set (every key
// above T), usually one digit pass sooner.  hist: 256 uints of LDS; sh: 2 uints of LDS.  When the candidates
// are spread over several work-groups, merge(hist) replaces each digit pass's
// local histogram by the sum over all of them (every work-group then takes the
// same digits) and returns false if they could not meet, which ends the
// selection with false.
struct LocalHist {
  __device__ bool operator()(uint32_t*) const { return true; }
};
template <int BLOCK, typename Visit, typename Merge = LocalHist>
__device__ __forceinline__ bool radix_threshold_v(const Visit& visit, int kc, uint32_t* hist, uint32_t* sh,
                                                  uint32_t& T, uint32_t& kk_out, uint32_t prefix = 0,
                                                  int known = 0, const Merge& merge = Merge()) {
  const int tid = threadIdx.x;
  uint32_t mask = known == 0 ? 0u : ~0u << (32 - known);
  prefix &= mask;
  uint32_t kk = uint32_t(kc);
  if (kc == 0) {
    T = 0xFFFFFFFFu;
    kk_out = 0;
    return true;
  }
  for (int hi = 32 - known; hi > 0;) {
    const int shift = hi > 8 ? hi - 8 : 0;
    const uint32_t wmask = (1u << (hi - shift)) - 1u;
    for (int d = tid; d < 256; d += BLOCK) hist[d] = 0;
    __syncthreads();
    visit([&](uint32_t key) {
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & wmask], 1u);
    });
    __syncthreads();
    if (!merge(hist)) return false;
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t h[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * tid - i];
        loc += h[i];
      }
      const uint32_t incl = wave_inclusive_sum(loc);   // over lanes, high digits first
      const uint32_t excl = incl - loc;
      const uint64_t hit = __ballot(incl >= kk);
      const int first = __ffsll((unsigned long long)hit) - 1;
      if (tid == first) {
        uint32_t cum = excl;
        int digit = 0;
        uint32_t above = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + h[i] >= kk) {
            digit = 255 - 4 * tid - i;
            above = cum;
            break;
          }
          cum += h[i];
        }
        const uint32_t pick = prefix | (uint32_t(digit) << shift);
        if (shift > 0 && pick != 0u && hist[digit] == kk - above) {
          // every candidate with this digit is kept: T just below them, no ties
          sh[0] = pick - 1u;
          sh[1] = 0u;
        } else {
          sh[0] = pick;
          sh[1] = kk - above;
        }
      }
    }
    __syncthreads();
    prefix = sh[0];
    kk = sh[1];
    mask |= wmask << shift;
    hi = shift;
    __syncthreads();
    if (kk == 0u) break;
  }
  T = prefix;
  kk_out = kk;
  return true;
}

// Protected form over one segment: candidates are the slots j in [P, n-R),
// key_at(j) returns slot j's order key.
template <int BLOCK, typename KeyAt>
__device__ __forceinline__ void radix_threshold(const KeyAt& key_at, int P, int n, int R, int kc, uint32_t* hist,
                                                uint32_t* sh, uint32_t& T, uint32_t& kk_out) {
  radix_threshold_v<BLOCK>(
      [&](const auto& f) {
        for (int j = P + int(threadIdx.x); j < n - R; j += BLOCK) f(key_at(j));
      },
      kc, hist, sh, T, kk_out);
}

}  // namespace kve
