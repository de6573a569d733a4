// Device helpers shared by the gfx950 kernels: bf16 rounding, RoPE angles,
// mask / slot arithmetic, MFMA vector types and LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hattn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kHeadDim = 256;
constexpr int kGroup = 4;             // query heads per KV head (both model shapes)
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 by the hardware conversion (v_cvt_pk_bf16_f32): round to
// nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// fp64 -> bf16 with a single rounding (nearest, ties to even). x is first
// rounded to fp32 with round-to-odd (truncate, then set the last bit when
// anything was cut), then to bf16 by the hardware's round-to-nearest-even:
// with 24 >= 8 + 2 significant bits in between, the two roundings give the
// correctly rounded result (the round-to-odd lemma). Branch-free; NaN stays
// NaN, infinities and overflow go to infinity.
__device__ __forceinline__ uint16_t double_to_bf16_bits(double x) {
  const float f = (float)x;  // nearest even
  const double back = (double)f;
  uint32_t u = __float_as_uint(f);
  u -= (fabs(back) > fabs(x)) ? 1u : 0u;  // rounded away from zero: step back
  u |= (back != x) ? 1u : 0u;             // inexact: odd
  return float_to_bf16_bits(__uint_as_float(u));
}

// ---------------------------------------------------------------- RoPE
// cos and sin of the fp64 angle p * inv_freq. The angle is reduced by 2*pi
// with a three-part Cody-Waite split (24 + 24 + 53 bits; exact for the
// quotients |k| < 2^28 that positions below 2^30 produce), then evaluated in
// fp64 on [-pi, pi]. inv_freq_i = theta^(-2i/r) is computed on the host.
constexpr double kTwoPiHi = 0x1.921fb6p+2;
constexpr double kTwoPiMid = -0x1.777a5cp-23;
constexpr double kTwoPiLo = -0x1.ee59d9cceba40p-48;
constexpr double kInvTwoPi = 0x1.45f306dc9c883p-3;

__device__ __forceinline__ void rope_sincos(int pos, double inv_freq, double* s, double* c) {
  const double ang = (double)pos * inv_freq;
  const double k = rint(ang * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, ang);
  r = fma(-k, kTwoPiMid, r);
  r = fma(-k, kTwoPiLo, r);
  sincos(r, s, c);
}

// ---------------------------------------------------------------- masks
// Visibility of key position pk from query position pq; window <= 0 means
// unbounded (full causal). Negative pk marks an empty slot.
__device__ __forceinline__ bool key_visible(int pq, int pk, int window) {
  return pk >= 0 && pk <= pq && (window <= 0 || pq - pk < window);
}

// Slot that position p is written to.
__device__ __forceinline__ int cache_slot(int p, int ring, int cap) {
  return ring ? (p % cap) : p;
}

// Position held by `slot` once positions 0..last have been written.
__device__ __forceinline__ int slot_position(int slot, int last, int ring, int cap) {
  if (ring) {
    int d = (last - slot) % cap;
    if (d < 0) d += cap;
    int p = last - d;
    return p >= 0 ? p : -1;
  }
  return slot <= last ? slot : -1;
}

// Contiguous slot range [lo, hi) whose keys a decode query at position p
// sees (the cache holding positions 0..p).
__device__ __forceinline__ void decode_key_range(int p, int ring, int cap, int window,
                                                 int* lo, int* hi) {
  if (ring) {
    *lo = 0;
    *hi = p + 1 < cap ? p + 1 : cap;
  } else {
    int l = (window > 0) ? p - window + 1 : 0;
    *lo = l > 0 ? l : 0;
    *hi = p + 1;
  }
}

// ---------------------------------------------------------------- gate
// The per-head output gate factor in fp32: sigmoid(g) (act 0), or
// silu(g) = g * sigmoid(g) (act 1).
__device__ __forceinline__ float gate_factor(float g, int act) {
  const float s = 1.0f / (1.0f + expf(-g));
  return act ? g * s : s;
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace hattn
