// Device helpers shared by the eviction-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "kvevict.h"

namespace kve {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

// double -> bf16 rounded once, to nearest even.  The float conversion is exact
// enough unless it lands on a bf16 midpoint, where the double decides.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float r = float(x);
  uint32_t b = __float_as_uint(r);
  if ((b & 0xFFFFu) == 0x8000u) {
    double ax = fabs(x), ar = fabs(double(r));
    if (ax > ar) return uint16_t((b + 0x8000u) >> 16);  // away from zero
    if (ax < ar) return uint16_t(b >> 16);              // toward zero
  }
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ uint16_t from_f64(double x) { return f64_to_bf16(x); }
  static __device__ __forceinline__ float widen(uint16_t v) { return bf16_to_f32(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f64(double x) { return float(x); }
  static __device__ __forceinline__ float widen(float v) { return v; }
};

// ---------------------------------------------------------------- RoPE
// Rotate the pair (a, b) of frequency index i (of head_dim d) to position p:
// (a cos - b sin, b cos + a sin), angle p * theta^(-2i/d) in double.  The
// inverse frequencies theta^(-2i/d), i < d/2, are formed once on the host
// (double-precision pow) and passed to the kernels by value.
struct InvFreq {
  double v[64];
};
inline InvFreq inv_freq(double theta, int d) {
  InvFreq f{};
  for (int i = 0; i < d / 2 && i < 64; ++i) f.v[i] = std::pow(theta, -2.0 * double(i) / double(d));
  return f;
}
struct RotPair { double a, b; };
__device__ __forceinline__ RotPair rotate_pair(double a, double b, double c, double s) {
#pragma clang fp contract(off)
  RotPair r;
  r.a = a * c - b * s;
  r.b = b * c + a * s;
  return r;
}
__device__ __forceinline__ RotPair rope_pair(double a, double b, double inv, int p) {
  const double ang = double(p) * inv;
  double s, c;
  sincos(ang, &s, &c);
  return rotate_pair(a, b, c, s);
}

// ---------------------------------------------------------------- wave reductions
// Combine v over lanes l and l ^ 16 (lanes16_*) or l ^ 32 (lanes32_*) with the
// gfx950 row-swap instructions: v_permlane16_swap with both operands v leaves
// each lane holding {v[l], v[l ^ 16]} across its two results (v_permlane32_swap
// likewise for l ^ 32), so the pair's max or sum needs no LDS round trip.
// Every lane of the wave must be active.
__device__ __forceinline__ float lanes16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float lanes32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float lanes16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float lanes32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// dpp<CTRL, ROW_MASK>(v, fill): the value of v in the lane that the DPP
// (data-parallel primitive) control CTRL names for this lane, read by the
// VALU with no LDS traffic and no per-lane address register; lanes whose
// source is outside their row, or whose row ROW_MASK leaves out, get `fill`.
// The controls used here (rows are 16 lanes):
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane l ^ 1
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane l ^ 2
constexpr int kDppRor4 = 0x124;      // row_ror:4: lane (l - 4) mod 16 of the row
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane 7 - l inside each group of 8
constexpr int kDppRor8 = 0x128;      // row_ror:8: lane l ^ 8
constexpr int kDppShr1 = 0x111;      // row_shr:n (0x110 + n): lane l - n of the row
constexpr int kDppBcast15 = 0x142;   // row_bcast:15: lane 15 of the previous row
constexpr int kDppBcast31 = 0x143;   // row_bcast:31: lane 31
template <int CTRL, int ROW_MASK = 0xF, typename T>
__device__ __forceinline__ T dpp(T v, T fill = T{}) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             CTRL, ROW_MASK, 0xF, false));
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, v), f = __builtin_bit_cast(uint64_t, fill);
    const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(int(uint32_t(f)), int(uint32_t(b)), CTRL, ROW_MASK, 0xF, false));
    const uint32_t hi =
        uint32_t(__builtin_amdgcn_update_dpp(int(uint32_t(f >> 32)), int(uint32_t(b >> 32)), CTRL, ROW_MASK, 0xF, false));
    return __builtin_bit_cast(T, (uint64_t(hi) << 32) | lo);
  }
}
// op(v[l], v[l ^ 16]) (ROW = 16) or op(v[l], v[l ^ 32]) (ROW = 32) with the
// row-swap instructions; both lanes of a pair combine the same two operands.
template <int ROW, typename T, typename Op>
__device__ __forceinline__ T swap_combine(T v, Op op) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
  auto swp = [](uint32_t x) {
    return ROW == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                     : __builtin_amdgcn_permlane32_swap(x, x, false, false);
  };
  if constexpr (sizeof(T) == 4) {
    const auto p = swp(__builtin_bit_cast(uint32_t, v));
    return op(__builtin_bit_cast(T, uint32_t(p[0])), __builtin_bit_cast(T, uint32_t(p[1])));
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const auto lo = swp(uint32_t(b)), hi = swp(uint32_t(b >> 32));
    return op(__builtin_bit_cast(T, (uint64_t(uint32_t(hi[0])) << 32) | uint32_t(lo[0])),
              __builtin_bit_cast(T, (uint64_t(uint32_t(hi[1])) << 32) | uint32_t(lo[1])));
  }
}

// op over the 64 lanes, the same value in every lane, combined in the order
// of the xor butterfly: lane l with l ^ 32, then l ^ 16, 8, 4, 2, 1.  After the
// l ^ 8 step the lanes l and l ^ 8 hold equal values, so row_ror:4 reads the
// value of lane l ^ 4.  op must be commutative (both lanes of a pair then
// get the same result).  Every lane of the wave must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = swap_combine<32>(v, op);
  v = swap_combine<16>(v, op);
  v = op(v, dpp<kDppRor8>(v));
  v = op(v, dpp<kDppRor4>(v));
  v = op(v, dpp<kDppXor2>(v));
  return op(v, dpp<kDppXor1>(v));
}
// op over each row of 16 lanes in the order l ^ 1, 2, 4, 8 (once the l ^ 1
// and l ^ 2 steps have made every quad uniform, the half-row mirror reads a
// lane of quad l ^ 4's, with the same value as lane l ^ 4).  op commutative;
// every lane active.
template <typename T, typename Op>
__device__ __forceinline__ T row16_reduce(T v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  return op(v, dpp<kDppRor8>(v));
}
// Inclusive prefix sum over the 64 lanes in lane order (integer T): a
// Hillis-Steele scan inside each row (row_shr 1, 2, 4, 8), then row 0's total
// into row 1 and row 2's into row 3, then rows 0-1's total into rows 2 and 3.
// Every lane active.
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T v) {
  v += dpp<kDppShr1>(v);
  v += dpp<kDppShr1 + 1>(v);
  v += dpp<kDppShr1 + 3>(v);
  v += dpp<kDppShr1 + 7>(v);
  v += dpp<kDppBcast15, 0xA>(v);
  v += dpp<kDppBcast31, 0xC>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  return wave_reduce(v, [](double x, double y) { return x + y; });
}

// Order-preserving map of fp32 values to uint32 (larger float -> larger key;
// -0.0 and +0.0 compare equal, as IEEE values do).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------- debug build bounds checks
// Built with -DKVE_DEBUG, KVE_CHECK(cond, bit) guards a global-memory access
// whose index comes from device-resident metadata (segment offsets, lengths,
// kept slots): a failed check sets `bit` in this source file's flag word and
// the caller skips the access (nothing traps).  kve_debug_flags() on the host
// reads and clears the words.  In the regular build the checks compile away.
#ifdef KVE_DEBUG
static __device__ unsigned int kve_debug_word;
__device__ __forceinline__ bool kve_debug_check(bool ok, unsigned int bit) {
  if (!ok) atomicOr(&kve_debug_word, 1u << bit);
  return ok;
}
#define KVE_CHECK(cond, bit) ::kve::kve_debug_check((cond), (bit))
#else
#define KVE_CHECK(cond, bit) true
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

}  // namespace kve
