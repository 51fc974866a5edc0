// Per-block power-of-two scales for E4M3 codes (device code only).
//
// A block of 32 elements along the contraction of a product shares one scale
// 2^X: X is the smallest integer with amax * 2^-X <= 448 (E4M3's largest
// finite value), so no element of the block saturates.  From amax's binary
// exponent E and mantissa M in [1, 2): X = E - 8 while M * 2^8 <= 448, i.e.
// M <= 1.75, else E - 7; X = -127 when amax is zero or an fp32 subnormal;
// clamped to [-127, 127].  The E8M0 code of the scale is X + 127, the form the
// gfx950 scaled MFMA takes per 32-element block.  (The pages' GB10 builds
// quantise with per-block scales calibrated on the activations: h3-spark
// model card, "What this config does".)
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace h3a {

__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int e = int((b >> 23) & 0xffu);
  if (e == 0) return -127;
  const int X = e - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// 2^-X exactly, for X in [-127, 127] (2^-127 is an fp32 subnormal).
__device__ __forceinline__ float mx_inv_scale(int X) {
  return X >= 127 ? __uint_as_float(0x00400000u) : __uint_as_float(uint32_t(127 - X) << 23);
}

// Saturate to +-448 before the E4M3 conversion (the hardware conversion turns
// values past 464 into NaN); NaN passes through unchanged (fminf/fmaxf alone
// would turn it into -448).
__device__ __forceinline__ float e4m3_sat(float x) { return x != x ? x : fminf(fmaxf(x, -448.0f), 448.0f); }

// Largest magnitude, NaN ignored (fmaxf returns the other operand).
__device__ __forceinline__ float abs_max(float m, float x) { return fmaxf(m, fabsf(x)); }

}  // namespace h3a
