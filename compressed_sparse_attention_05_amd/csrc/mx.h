// MXFP4 quantisation on the device (OCP Microscaling Formats v1.0: e2m1 elements, one e8m0 shared
// scale per 32 consecutive elements), the storage of indexer keys and queries ("Anatomy of a Frontier
// Model", sections "The KV cache, recomputed" and "Precision: FP8 everywhere, FP4 experts").
//
// A block's shared exponent is X = floor(log2(max |x|)) - 2 (2: the largest e2m1 exponent), clamped to
// [-127, 127] and stored as X + 127; each element x * 2^-X (exact: a power of two) goes to the nearest
// e2m1 value, ties to the even code, magnitudes past 6 to 6; the sign bit is x's sign bit.
#pragma once

#include "common.h"

namespace csa {

// X of a block whose largest magnitude is amax (finite, >= 0): floor(log2 amax) is the unbiased
// exponent field of a normal float; zero and subnormal maxima fall below -125 and clamp to -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int X = e - 127 - 2;
  return X < -127 ? -127 : X;
}

// 2^-X as a float (X in [-127, 125]: the result is a normal float)
__device__ __forceinline__ float mx_inv_scale(int X) { return __uint_as_float((uint32_t)(127 - X) << 23); }

// e2m1 code of a scaled element s: the magnitude code counts the rounding midpoints s passes. At a
// midpoint the count goes to the even code (0.25 -> 0, 0.75 -> 2, 1.25 -> 2, 1.75 -> 4, 2.5 -> 4,
// 3.5 -> 6, 5 -> 6), so the comparisons are strict below odd codes and inclusive below even ones.
__device__ __forceinline__ uint32_t e2m1_code(float s) {
  const float a = fabsf(s);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(s) >> 28) & 8u);
}

// Quantises V consecutive elements per lane; the 32 / V lanes of one block are consecutive and aligned
// and all of them take part (the block maximum is a butterfly over them). Returns the lane's V / 2
// code bytes packed little-endian (element 2i in the low nibble of byte i); *x_out = the block's
// shared exponent X.
template <int V>
__device__ __forceinline__ uint32_t mxfp4_quant_lanes(const float (&v)[V], int& x_out) {
  static_assert(V == 4 || V == 8, "4 or 8 elements per lane");
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 32 / V; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const int X = mx_block_exp(amax);
  const float inv = mx_inv_scale(X);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) packed |= e2m1_code(v[i] * inv) << (4 * i);
  x_out = X;
  return packed;
}

// Stores what mxfp4_quant_lanes<V> returned for the lane holding elements j0 .. j0 + V - 1 of a row
// whose codes start at `codes` and scales at `scales`.
template <int V>
__device__ __forceinline__ void mxfp4_store_lanes(uint8_t* codes, uint8_t* scales, int j0, uint32_t packed, int X) {
  if constexpr (V == 8) *reinterpret_cast<uint32_t*>(codes + j0 / 2) = packed;
  else *reinterpret_cast<uint16_t*>(codes + j0 / 2) = (uint16_t)packed;
  if ((j0 & 31) == 0) scales[j0 / 32] = (uint8_t)(X + 127);
}

}  // namespace csa
