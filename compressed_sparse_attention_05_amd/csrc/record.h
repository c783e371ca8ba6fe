// The 584-byte compressed-entry record ("Anatomy of a Frontier Model", section "The KV cache,
// recomputed": 448 dims in FP8 with seven one-byte UE8M0 scales, the 64 RoPE dims in BF16, a pad
// byte; bullet "QK-norm and partial RoPE": the position-free dims are the FP8 ones).
//
// Record bytes: e4m3 codes of dims 0..447 | bf16 of dims 448..511 (little-endian) | scale exponents
// E_0..E_6 | 0. Group g = dims 64g..64g+63 has scale 2^(E_g - 127), the smallest power of two s with
// max|x| / s <= 448 (no element saturates); an all-zero group takes E = 127. Codes are OCP E4M3
// (bias 7, subnormals 2^-6 m/8, largest finite 448), rounded to nearest with ties to the even code,
// the sign bit taken from the value's sign bit.
#pragma once

#include "common.h"

namespace csa {

// e4m3 code of y (|y| <= 448 for a group scaled as above; larger magnitudes saturate to 448)
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                 // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)rintf(a * 512.f);        // exact scaling; rintf rounds half to even; 8 -> 0x08
  } else {
    const uint32_t bits = __float_as_uint(a);
    int ex = (int)(bits >> 23) - 127;         // -6 .. 8
    uint32_t keep = (bits >> 20) & 7u;
    const uint32_t rem = bits & 0xFFFFFu, half = 0x80000u;
    if (rem > half || (rem == half && (keep & 1u))) ++keep;
    if (keep == 8u) {
      keep = 0;
      ++ex;
    }
    code = ((uint32_t)(ex + 7) << 3) | keep;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// One wave packs one entry: lane l holds dims 8l..8l+7 in v (lanes 8g..8g+7 hold FP8 group g, g < 7;
// lanes 56..63 the bf16 dims); a group's maximum comes from a three-step lane butterfly. rec is the
// record's first byte (8-byte aligned). Every lane of the wave must call it.
__device__ __forceinline__ void pack_record_wave(const float (&v)[8], uint8_t* rec) {
  const int lane = lane_id();
  if (lane >= 56) {  // RoPE dims: bf16 (the value itself for bf16 input, RNE otherwise)
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f2bf(v[2 * j]) | ((uint32_t)f2bf(v[2 * j + 1]) << 16);
    uint2* dst = reinterpret_cast<uint2*>(rec + 448 + 16 * (lane - 56));
    dst[0] = make_uint2(w[0], w[1]);
    dst[1] = make_uint2(w[2], w[3]);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  // E = 127 + ceil(log2(amax / 448)); with amax = f 2^e (0.5 <= f < 1), amax / 448 = (f / 0.875)
  // 2^(e-9), so ceil(log2) is e - 9 when f <= 0.875 and e - 8 above
  int E = 127;
  if (amax > 0.f) {
    int e;
    const float f = frexpf(amax, &e);
    E = 127 + e - 9 + (f > 0.875f ? 1 : 0);
    E = E < 1 ? 1 : (E > 254 ? 254 : E);
  }
  if (lane < 56) {
    const float inv = __uint_as_float((uint32_t)(254 - E) << 23);  // 2^(127 - E)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= e4m3_code(v[j] * inv) << (8 * j);
      hi |= e4m3_code(v[j + 4] * inv) << (8 * j);
    }
    *reinterpret_cast<uint2*>(rec + 8 * lane) = make_uint2(lo, hi);
  }
  // scales and pad: lane 0 gathers E of the seven groups (lanes 0, 8, ..., 48)
  uint32_t s_lo = 0, s_hi = 0;
#pragma unroll
  for (int g = 0; g < 7; ++g) {
    const uint32_t Eg = (uint32_t)__shfl(E, 8 * g, 64);
    if (g < 4) s_lo |= Eg << (8 * g);
    else s_hi |= Eg << (8 * (g - 4));
  }
  if (lane == 0) *reinterpret_cast<uint2*>(rec + 576) = make_uint2(s_lo, s_hi);
}

}  // namespace csa
