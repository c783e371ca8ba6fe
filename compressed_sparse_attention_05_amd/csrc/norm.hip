// QK-norm and partial RoPE ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE"):
// queries and compressed entries are RMS-normalised per head, RoPE turns only the last rope_dims
// dims, and the attention output is turned back by the query's own position.
//
// One wave per head vector: lane l holds dims l, l + 64, ... (coalesced across the wave for any
// D). The norm is y = x / sqrt(mean(x^2) + eps) * gamma (fp32, the sum of squares by a wave
// reduction). The rotated slice is taken in adjacent pairs (2i, 2i+1), which sit in lanes 2j and
// 2j+1, so the partner value comes by one lane swap; pair i turns by pos * theta^(-2i/rope_dims).
// The angle is formed and its sine and cosine taken in fp64: at positions near 2^20 an fp32 angle
// would be off by up to ~0.06 rad.
#include "kernels.h"

namespace csa {

namespace {

constexpr int kNormWaves = 4;
constexpr int kNormMaxPer = 64;  // D <= 4096

// PER: dims per lane, a compile-time bound (D <= 64 * PER) so that v[] stays in registers
template <int DT, int PER>
__global__ void __launch_bounds__(kNormWaves * 64) norm_rope_kernel(NormRopeArgs a) {
  const int lane = lane_id();
  const int64_t vec = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);  // (b, r, h)
  if (vec >= (int64_t)a.B * a.R * a.H) return;
  const int h = (int)(vec % a.H);
  const int64_t br = vec / a.H;
  const int64_t r = br % a.R, b = br / a.R;
  const int64_t xo = b * a.x_seq_stride + r * a.x_ld + (int64_t)h * a.D;
  const int64_t yo = b * a.y_seq_stride + r * a.y_ld + (int64_t)h * a.D;
  // in place without the norm (the output's back-rotation) only the rotated slice is read and written
  const bool inplace = a.x == a.y && a.x_ld == a.y_ld && a.x_seq_stride == a.y_seq_stride;
  const int jlo = (a.gamma || !inplace) ? 0 : (a.D - a.rope_dims) / 64;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = lane + 64 * j;
    v[j] = (j >= jlo && d < a.D) ? load_elem<DT>(a.x, xo + d) : 0.f;
  }
  if (a.gamma) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) ss = fmaf(v[j], v[j], ss);
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)a.D + a.eps);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      if (d < a.D) v[j] = v[j] * inv * a.gamma[d];
    }
  }
  if (a.rope_dims > 0) {
    const int rs = a.D - a.rope_dims;
    const double pos = (double)(a.pos0 + r * a.pos_step);
    const double lt = log2(a.theta);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (64 * j + 63 < rs) continue;  // uniform: the whole wave takes part in the swap
      const int d = lane + 64 * j;
      const float other = __shfl_xor(v[j], 1, 64);
      if (d >= rs && d < a.D) {
        const int i = (d - rs) >> 1;
        const double ang = pos * exp2(-(2.0 * i / a.rope_dims) * lt);
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float c = (float)cd, s = a.inverse ? -(float)sd : (float)sd;
        // even dim: a' = a c - b s; odd dim: b' = a s + b c (a = even member, b = odd member)
        v[j] = ((d - rs) & 1) == 0 ? v[j] * c - other * s : other * s + v[j] * c;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = lane + 64 * j;
    if (j >= jlo && d < a.D) store_elem<DT>(a.y, yo + d, v[j]);
  }
}

}  // namespace

int norm_rope_max_dim() { return 64 * kNormMaxPer; }

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.R * a.H;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, kNormWaves));
  const int per = (a.D + 63) / 64;
  const bool bf = a.dtype == CSA_BF16;
#define CSA_NORM_LAUNCH(P)                                                                              \
  if (bf) hipLaunchKernelGGL((norm_rope_kernel<CSA_BF16, P>), grid, dim3(kNormWaves * 64), 0, s, a);    \
  else hipLaunchKernelGGL((norm_rope_kernel<CSA_F32, P>), grid, dim3(kNormWaves * 64), 0, s, a);
  if (per <= 1) { CSA_NORM_LAUNCH(1) }
  else if (per <= 2) { CSA_NORM_LAUNCH(2) }
  else if (per <= 4) { CSA_NORM_LAUNCH(4) }
  else if (per <= 8) { CSA_NORM_LAUNCH(8) }
  else if (per <= 16) { CSA_NORM_LAUNCH(16) }
  else { CSA_NORM_LAUNCH(kNormMaxPer) }
#undef CSA_NORM_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
