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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
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
