// Helpers of the compressors ("The Exchange Rates of a Million Tokens", section 3; "Anatomy of a
// Frontier Model", bullet "Compressed Sparse Attention (CSA)"): 16-byte channel vectors and the
// per-channel softmax pooling over a block's logits, accumulated online in row order.
#pragma once

#include "common.h"

namespace csa {

template <int DT>
struct Vec;
template <>
struct Vec<CSA_BF16> {
  static constexpr int N = 8;
  __device__ static void load(const void* p, int64_t off, float* v) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  __device__ static void store(void* p, int64_t off, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f2bf(v[2 * j]) | ((uint32_t)f2bf(v[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<CSA_F32> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, int64_t off, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(void* p, int64_t off, const float* v) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Scalar fallback for channel counts or strides that are not vector aligned.
template <int DT>
struct Scalar {
  static constexpr int N = 1;
  __device__ static void load(const void* p, int64_t off, float* v) { v[0] = load_elem<DT>(p, off); }
  __device__ static void store(void* p, int64_t off, const float* v) { store_elem<DT>(p, off, v[0]); }
};

// Softmax-weighted sum accumulated online per channel: running maximum mx, denominator den and
// numerator num; each logit rescales the running sums when it raises the maximum.
template <int V>
__device__ __forceinline__ void accumulate(const float* z, const float* bias, const float* c,
                                           float* mx, float* den, float* num) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float l = z[v] + bias[v];
    const float nm = fmaxf(mx[v], l);
    const float sc = expf(mx[v] - nm);
    const float p = expf(l - nm);
    den[v] = fmaf(den[v], sc, p);
    num[v] = fmaf(num[v], sc, p * c[v]);
    mx[v] = nm;
  }
}

// Merges the online-softmax state of another thread's rows: both maxima are brought to the larger
// one. Symmetric in its two operands, so every lane of a butterfly ends with the same bits.
template <int V>
__device__ __forceinline__ void merge(float* mx, float* den, float* num, const float* mx2, const float* den2,
                                      const float* num2) {
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float nm = fmaxf(mx[v], mx2[v]);
    const float s1 = expf(mx[v] - nm), s2 = expf(mx2[v] - nm);
    den[v] = den[v] * s1 + den2[v] * s2;
    num[v] = num[v] * s1 + num2[v] * s2;
    mx[v] = nm;
  }
}

}  // namespace csa
