// Device-side rules of per-row symmetric int8 quantisation (Quasar, Sec. 3.3 "Online
// Activation Smoothing and Quantization"), shared by every kernel that quantises a row so
// that all of them produce the same codes bit for bit:
//   x'   = f32(x) * inv_smooth[k]      (if a multiplier vector is given)
//   a    = max_k |x'|,  s = a / 127    (IEEE fp32 division)
//   code = a == 0 ? 0 : clamp(rint(x' / s), -127, 127)   (correctly rounded division, RNE)
// The codes are bit-identical to rint(x' / s) with an IEEE correctly rounded division (the
// library is built with -fhip-fp32-correctly-rounded-divide-sqrt), but most elements avoid
// the division: with r the correctly rounded 1/s (one division per row), t = x' * r differs
// from the exact quotient by at most |x'/s| * 2^-23 <= 1.6e-5, and the correctly rounded
// quotient is within 2^-18 of it, so when t is farther than 2^-14 from a half-integer both
// round to the same integer.  Elements inside that band (true ties included) take the
// division.
#pragma once

#include "qv_internal.h"

namespace qv {
namespace {

// Element j of eight 16-bit values as fp32: fp16 (activations) or bf16 (offline weights).
template <bool kBf16>
__device__ __forceinline__ float elem(u32x4 raw, int j) {
  if (kBf16) {
    const uint32_t d = raw[j >> 1];
    return __builtin_bit_cast(float, (j & 1) ? (d & 0xFFFF0000u) : (d << 16));
  }
  return (float)__builtin_bit_cast(f16x8, raw)[j];
}

// rint(x / s) with the division correctly rounded; r = correctly rounded 1 / s.
__device__ __forceinline__ float code_of(float f, float s, float r) {
  const float t = f * r;
  const float fr = t - __builtin_floorf(t);
  float q;
  if (__builtin_fabsf(fr - 0.5f) > 0x1p-14f) {  // false for NaN/Inf too
    q = __builtin_rintf(t);
  } else {
    q = __builtin_rintf(f / s);
  }
  return fminf(fmaxf(q, -127.0f), 127.0f);
}

// 8 codes of one 16-byte vector of the row (k = 8v .. 8v+7), packed little-endian.
template <bool kSmooth, bool kBf16>
__device__ __forceinline__ u32x2 quantise8(u32x4 raw, const float* __restrict__ inv_smooth,
                                           int v, float amax, float s, float rs) {
  uint32_t packed[2] = {0u, 0u};
  if (amax != 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f = elem<kBf16>(raw, j);
      if (kSmooth) f = f * inv_smooth[v * 8 + j];
      const float t = code_of(f, s, rs);
      packed[j >> 2] |= ((uint32_t)(int)t & 0xFFu) << (8 * (j & 3));
    }
  }
  return u32x2{packed[0], packed[1]};
}

template <bool kSmooth, bool kBf16>
__device__ __forceinline__ float vec_absmax(u32x4 raw, const float* __restrict__ inv_smooth, int v,
                                            float amax) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float f = elem<kBf16>(raw, j);
    if (kSmooth) f = f * inv_smooth[v * 8 + j];
    amax = fmaxf(amax, fabsf(f));
  }
  return amax;
}

}  // namespace
}  // namespace qv
