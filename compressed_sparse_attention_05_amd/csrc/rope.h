// RoPE angles ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE": the last dims of
// queries and entries turn by their position). Pair i of the rotated slice turns by
// pos * theta^(-2i/rope_dims); lt = log2(theta).
#pragma once

#include "common.h"

namespace csa {

// cos and sin of pos * theta^(-2i/rope_dims): the angle is formed and reduced to [-pi, pi] in fp64,
// then its sine and cosine are taken in fp32 (the reduced angle is exact to ~1e-7 rad)
__device__ __forceinline__ void rope_cos_sin(double pos, int i, int rope_dims, double lt, bool inverse, float& c,
                                             float& s) {
  const double ang = pos * exp2(-(2.0 * i / rope_dims) * lt);
  const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
  const float red = (float)fma(-k, 6.283185307179586, ang);
  sincosf(red, &s, &c);
  if (inverse) s = -s;
}

}  // namespace csa
