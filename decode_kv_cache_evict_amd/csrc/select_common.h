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
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) wtot[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int q = 0; q < BLOCK / kWave; ++q) t += wtot[q];
  __syncthreads();
  return t;
}

// Threshold of a top-kc selection: find the kc-th largest order key T among the
// candidate keys of the work-group (MSB-first radix select over LDS histograms
// of at most 8-bit digits) and kk, the number of candidates equal to T that
// are kept.  visit(f) calls f(key) once for every candidate key this thread
// holds; every thread must visit the same keys on each call.  The caller may
// pass the number of leading bits `known` (0..32) that every candidate shares
// with `prefix` (e.g. the common prefix of the candidates' minimum and
// maximum); the digits then start below them.  kc == 0 gives T = 0xFFFFFFFF,
// kk = 0.  hist: 256 uints of LDS; sh: 2 uints of LDS.
template <int BLOCK, typename Visit>
__device__ __forceinline__ void radix_threshold_v(const Visit& visit, int kc, uint32_t* hist, uint32_t* sh,
                                                  uint32_t& T, uint32_t& kk_out, uint32_t prefix = 0,
                                                  int known = 0) {
  const int tid = threadIdx.x;
  uint32_t mask = known == 0 ? 0u : ~0u << (32 - known);
  prefix &= mask;
  uint32_t kk = uint32_t(kc);
  if (kc == 0) {
    T = 0xFFFFFFFFu;
    kk_out = 0;
    return;
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
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t h[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[255 - 4 * tid - i];
        loc += h[i];
      }
      uint32_t incl = loc;                  // inclusive scan over lanes, high digits first
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += v;
      }
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
        sh[0] = prefix | (uint32_t(digit) << shift);
        sh[1] = kk - above;
      }
    }
    __syncthreads();
    prefix = sh[0];
    kk = sh[1];
    mask |= wmask << shift;
    hi = shift;
    __syncthreads();
  }
  T = prefix;
  kk_out = kk;
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
