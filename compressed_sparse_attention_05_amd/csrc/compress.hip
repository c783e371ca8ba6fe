// Step 1: the CSA compressor.
//
// One entry per complete block of m tokens, per channel a softmax over the 2m logits of the
// entry's own block (series a) and the previous block (series b), then the weighted sum of the
// matching values ("The Exchange Rates of a Million Tokens", section 3; "Anatomy of a Frontier
// Model", bullet "Compressed Sparse Attention (CSA)"). The HCA compressor ("Anatomy of a Frontier
// Model", bullet "Heavily Compressed Attention (HCA)": blocks of 128 tokens, no overlap) is the
// same pooling over the own block only (overlap = false).
//
// The step is HBM-bound and reads every input element exactly once: entry i reads block i of
// series a and block i-1 of series b, so no row is shared between entries and no LDS staging is
// needed. A thread owns VEC consecutive channels of one entry and issues 16-byte loads along the
// channel axis (coalesced across the threads of a row).
#include "kernels.h"

namespace csa {

namespace {

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

constexpr int kMaxM = 128;

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

// G consecutive threads share one (entry, channel vector): thread `sub` takes rows sub, sub + G, ...
// of each block, and the G partial softmax states meet through a shuffle butterfly. G = 1 for short
// blocks (CSA, m = 4); long blocks (HCA, m = 128) use G = 16 so that a chunk has enough threads.
template <class VI, class VO>
__global__ void __launch_bounds__(256) compress_kernel(CompressArgs a) {
  constexpr int V = VI::N;
  const int G = a.group;
  const int cv = a.c / V;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  const int64_t slot = gid / G;
  const int sub = (int)(gid % G);
  if (slot >= (int64_t)a.n_new * cv) return;  // whole groups only: G divides the block size
  const int e = (int)(slot / cv);
  const int j0 = (int)(slot % cv) * V;
  const int m = a.m;
  const int64_t i = a.first_entry + e;
  const int64_t sbase = (int64_t)b * a.seq_stride;

  float mx[V], den[V], num[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    mx[v] = -INFINITY;
    den[v] = 0.f;
    num[v] = 0.f;
  }
  // This thread's rows of a block are taken kRows at a time, all loads of a group issued before any
  // is used (one memory latency per group, not per row); the logits enter the online softmax in
  // row order.
  constexpr int kRows = 8;
  // own block, series a
  for (int r0 = sub; r0 < m; r0 += kRows * G) {
    float z[kRows][V], c[kRows][V];
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      if (r0 + q * G >= m) break;
      const int64_t row = sbase + (int64_t)(e * m + r0 + q * G) * a.ld + j0;
      VI::load(a.za, row, z[q]);
      VI::load(a.ca, row, c[q]);
    }
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      if (r0 + q * G >= m) break;
      float bias[V];
#pragma unroll
      for (int v = 0; v < V; ++v) bias[v] = a.bias_a[(r0 + q * G) * a.c + j0 + v];
      accumulate<V>(z[q], bias, c[q], mx, den, num);
    }
  }
  // previous block, series b (entry 0 has none; HCA pools its own block only)
  if (a.overlap && i >= 1) {
    const void* cb = e >= 1 ? a.cb : a.halo_cb;
    const void* zb = e >= 1 ? a.zb : a.halo_zb;
    for (int r0 = sub; r0 < m; r0 += kRows * G) {
      float z[kRows][V], c[kRows][V];
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        if (r0 + q * G >= m) break;
        const int r = r0 + q * G;
        const int64_t row = e >= 1 ? sbase + (int64_t)((e - 1) * m + r) * a.ld + j0
                                   : (int64_t)b * a.halo_seq_stride + (int64_t)r * a.halo_ld + j0;
        VI::load(zb, row, z[q]);
        VI::load(cb, row, c[q]);
      }
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        if (r0 + q * G >= m) break;
        float bias[V];
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = a.bias_b[(r0 + q * G) * a.c + j0 + v];
        accumulate<V>(z[q], bias, c[q], mx, den, num);
      }
    }
  }
  for (int off = G >> 1; off > 0; off >>= 1) {
    float mx2[V], den2[V], num2[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      mx2[v] = __shfl_xor(mx[v], off, 64);
      den2[v] = __shfl_xor(den[v], off, 64);
      num2[v] = __shfl_xor(num[v], off, 64);
    }
    merge<V>(mx, den, num, mx2, den2, num2);
  }
  if (sub != 0) return;
  float out[V];
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = num[v] / den[v];
  const int64_t orow = (a.out_first >= 0 ? a.out_first : a.first_entry) + e;
  VO::store(a.entries, (int64_t)b * a.entries_seq_stride + orow * a.c + j0, out);
}

template <int DI, int DO>
hipError_t launch_typed(const CompressArgs& a, hipStream_t s) {
  const bool vec_ok = (a.c % Vec<DI>::N == 0) && (a.ld % Vec<DI>::N == 0) &&
                      (a.seq_stride % Vec<DI>::N == 0) && (a.halo_ld % Vec<DI>::N == 0) &&
                      (a.halo_seq_stride % Vec<DI>::N == 0) && (a.entries_seq_stride % Vec<DI>::N == 0) &&
                      Vec<DI>::N == Vec<DO>::N && a.aligned16;
  const int V = vec_ok ? Vec<DI>::N : 1;
  const int64_t threads = (int64_t)a.n_new * (a.c / V) * a.group;
  dim3 grid((unsigned)ceil_div(threads, 256), (unsigned)a.B);
  if (vec_ok) {
    hipLaunchKernelGGL((compress_kernel<Vec<DI>, Vec<DO>>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((compress_kernel<Scalar<DI>, Scalar<DO>>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a0, hipStream_t s) {
  if (a0.n_new <= 0 || a0.B <= 0) return hipSuccess;
  CompressArgs a = a0;
  a.group = a.m >= 64 ? 16 : 1;  // threads per (entry, channel vector); every thread has >= 4 rows
  if (a.in_dtype == CSA_BF16 && a.out_dtype == CSA_BF16) return launch_typed<CSA_BF16, CSA_BF16>(a, s);
  if (a.in_dtype == CSA_F32 && a.out_dtype == CSA_F32) return launch_typed<CSA_F32, CSA_F32>(a, s);
  if (a.in_dtype == CSA_BF16 && a.out_dtype == CSA_F32) {
    CompressArgs b = a;
    b.aligned16 = false;
    return launch_typed<CSA_BF16, CSA_F32>(b, s);
  }
  CompressArgs b = a;
  b.aligned16 = false;
  return launch_typed<CSA_F32, CSA_BF16>(b, s);
}

int compress_max_m() { return kMaxM; }

}  // namespace csa
