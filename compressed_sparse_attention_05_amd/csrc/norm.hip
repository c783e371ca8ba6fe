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
#include "rope.h"

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
    const double pos = (double)(pos_at(a.pos, b) + a.pos_off + r * a.pos_step);
    const double lt = log2(a.theta);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (64 * j + 63 < rs) continue;  // uniform: the whole wave takes part in the swap
      const int d = lane + 64 * j;
      const float other = __shfl_xor(v[j], 1, 64);
      if (d >= rs && d < a.D) {
        float c, s;
        rope_cos_sin(pos, (d - rs) >> 1, a.rope_dims, lt, a.inverse != 0, c, s);
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

// Contiguous layout (D = 64 * PER, PER a multiple of the 16-byte vector, 16-byte aligned rows): lane
// l holds dims PER*l .. PER*l + PER - 1, loaded and stored as whole vectors, so every rotated pair
// sits in one lane. A wave takes up to kHeadsPerWave head vectors of one row, which share the
// row's position: the cosines and sines are formed once per wave.
constexpr int kHeadsPerWave = 8;

template <int DT, int PER>
__global__ void __launch_bounds__(kNormWaves * 64) norm_rope_contig(NormRopeArgs a, int hpw) {
  constexpr int VE = DT == CSA_BF16 ? 8 : 4;  // elements per 16-byte vector
  static_assert(PER % VE == 0, "whole vectors per lane");
  const int lane = lane_id();
  const int hg_per_row = (a.H + hpw - 1) / hpw;
  const int64_t wv = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);  // (b, r, head group)
  if (wv >= (int64_t)a.B * a.R * hg_per_row) return;
  const int hg = (int)(wv % hg_per_row);
  const int64_t br = wv / hg_per_row;
  const int64_t r = br % a.R, b = br / a.R;
  const int d0 = PER * lane;
  const int rs = a.D - a.rope_dims;
  const bool rot = a.rope_dims > 0 && d0 + PER > rs;  // this lane holds rotated dims
  const bool inplace = a.x == a.y && a.x_ld == a.y_ld && a.x_seq_stride == a.y_seq_stride;
  // in place without the norm (the output's back-rotation) only lanes holding rotated dims work
  const bool mine = a.gamma || !inplace || rot;
  float cs[PER / 2], sn[PER / 2];
  if (rot) {
    const double pos = (double)(pos_at(a.pos, b) + a.pos_off + r * a.pos_step);
    const double lt = log2(a.theta);
#pragma unroll
    for (int t = 0; t < PER / 2; ++t) {
      cs[t] = 1.f;
      sn[t] = 0.f;
      if (d0 + 2 * t >= rs) rope_cos_sin(pos, (d0 + 2 * t - rs) >> 1, a.rope_dims, lt, a.inverse != 0, cs[t], sn[t]);
    }
  }
  float g[PER];
  if (a.gamma) {
#pragma unroll
    for (int j = 0; j < PER; ++j) g[j] = a.gamma[d0 + j];
  }
  for (int hh = 0; hh < hpw; ++hh) {
    const int h = hg * hpw + hh;
    if (h >= a.H) break;  // wave-uniform
    const int64_t xo = b * a.x_seq_stride + r * a.x_ld + (int64_t)h * a.D + d0;
    const int64_t yo = b * a.y_seq_stride + r * a.y_ld + (int64_t)h * a.D + d0;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = 0.f;
    if (mine) {
#pragma unroll
      for (int j = 0; j < PER; j += VE) {
        if (DT == CSA_BF16) {
          const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + xo + j);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[j + 2 * t] = __uint_as_float(w[t] << 16);
            v[j + 2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
          }
        } else {
          const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + xo + j);
          v[j] = f.x;
          v[j + 1] = f.y;
          v[j + 2] = f.z;
          v[j + 3] = f.w;
        }
      }
    }
    if (a.gamma) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) ss = fmaf(v[j], v[j], ss);
      ss = wave_sum(ss);
      const float inv = 1.f / sqrtf(ss / (float)a.D + a.eps);
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] = v[j] * inv * g[j];
    }
    if (rot) {
#pragma unroll
      for (int t = 0; t < PER / 2; ++t) {
        const float x0 = v[2 * t], x1 = v[2 * t + 1];
        v[2 * t] = x0 * cs[t] - x1 * sn[t];
        v[2 * t + 1] = x0 * sn[t] + x1 * cs[t];
      }
    }
    if (mine) {
#pragma unroll
      for (int j = 0; j < PER; j += VE) {
        if (DT == CSA_BF16) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = (uint32_t)f2bf(v[j + 2 * t]) | ((uint32_t)f2bf(v[j + 2 * t + 1]) << 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + yo + j) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.y) + yo + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
        }
      }
    }
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
  // contiguous layout: whole 16-byte vectors per lane (bf16: D = 512 or 1024; fp32: D = 256, 512, 1024)
  const int64_t ve = bf ? 8 : 4;
  const int cper = a.D / 64;
  const bool contig = a.D % 64 == 0 && cper % ve == 0 && cper <= 16 && (uintptr_t)a.x % 16 == 0 &&
                      (uintptr_t)a.y % 16 == 0 && a.x_ld % ve == 0 && a.y_ld % ve == 0 && a.x_seq_stride % ve == 0 &&
                      a.y_seq_stride % ve == 0;
  if (contig) {
    const int hpw = a.H < kHeadsPerWave ? a.H : kHeadsPerWave;
    const int64_t waves = (int64_t)a.B * a.R * ((a.H + hpw - 1) / hpw);
    const dim3 g2((unsigned)ceil_div(waves, kNormWaves)), blk(kNormWaves * 64);
    if (cper == 4) hipLaunchKernelGGL((norm_rope_contig<CSA_F32, 4>), g2, blk, 0, s, a, hpw);
    else if (cper == 8 && bf) hipLaunchKernelGGL((norm_rope_contig<CSA_BF16, 8>), g2, blk, 0, s, a, hpw);
    else if (cper == 8) hipLaunchKernelGGL((norm_rope_contig<CSA_F32, 8>), g2, blk, 0, s, a, hpw);
    else if (bf) hipLaunchKernelGGL((norm_rope_contig<CSA_BF16, 16>), g2, blk, 0, s, a, hpw);
    else hipLaunchKernelGGL((norm_rope_contig<CSA_F32, 16>), g2, blk, 0, s, a, hpw);
    return hipGetLastError();
  }
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
