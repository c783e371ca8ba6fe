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
#include "mx.h"
#include "pool.h"
#include "record.h"
#include "rope.h"

namespace csa {

namespace {

constexpr int kMaxM = 128;

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
  const int64_t first = pos_at(a.pos0, b) / m;  // entry of the chunk's first block
  const int64_t i = first + e;
  // the entry's row: rows past the capacity are not written (and their inputs not read)
  const int64_t orow = (a.out_first >= 0 ? a.out_first : first) + e;
  if (a.out_first < 0 && orow >= a.n_cap) return;
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
  if (a.epilogue) {
    // The cv = c / V threads of one entry are consecutive lanes of one wave (G = 1, cv a power of two
    // <= 64). The entry is rounded to its storage type, RMS-normalised (gain gamma) and turned by RoPE
    // at its block's last token, (i + 1) m - 1, as a separate pass over the stored entry would; then
    // stored, packed into its 584-byte record (cv = 64: lane l holds dims 8l .. 8l + 7), or (indexer
    // keys) quantised to MXFP4.
    const bool bf = a.out_dtype == CSA_BF16;
    if (bf) {
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = bf2f(f2bf(out[v]));
    }
    if (a.gamma) {
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) ss = fmaf(out[v], out[v], ss);
      for (int o = cv >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = 1.f / sqrtf(ss / (float)a.c + a.eps);
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = out[v] * inv * a.gamma[j0 + v];
    }
    if (a.rope_dims > 0) {
      const int rs = a.c - a.rope_dims;
      const double pos = (double)((i + 1) * m - 1), lt = log2(a.theta);
      if (V >= 2) {  // pairs (2t, 2t + 1) inside the vector (j0 is even)
#pragma unroll
        for (int v = 0; v + 1 < V; v += 2) {
          if (j0 + v < rs) continue;
          float cs, sn;
          rope_cos_sin(pos, (j0 + v - rs) >> 1, a.rope_dims, lt, false, cs, sn);
          const float x0 = out[v], x1 = out[v + 1];
          out[v] = x0 * cs - x1 * sn;
          out[v + 1] = x0 * sn + x1 * cs;
        }
      } else {  // one channel per lane: the partner is the neighbouring lane
        const float other = __shfl_xor(out[0], 1, 64);
        if (j0 >= rs) {
          float cs, sn;
          rope_cos_sin(pos, (j0 - rs) >> 1, a.rope_dims, lt, false, cs, sn);
          out[0] = ((j0 - rs) & 1) == 0 ? out[0] * cs - other * sn : other * sn + out[0] * cs;
        }
      }
    }
    if (bf) {  // stored values: what the record is packed from
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = bf2f(f2bf(out[v]));
    }
    if (a.fp4_codes) {  // MXFP4 key: the 32 / V lanes of each block meet for its maximum
      if constexpr (V == 4 || V == 8) {
        int X;
        const uint32_t pk = mxfp4_quant_lanes<V>(out, X);
        const int64_t r = (int64_t)b * a.n_cap + orow;
        mxfp4_store_lanes<V>(a.fp4_codes + r * (a.c / 2), a.fp4_scales + r * (a.c / 32), j0, pk, X);
      }
      return;
    }
    if (a.records) {
      if constexpr (V == 8) {
        pack_record_wave(out, static_cast<uint8_t*>(a.entries) + (int64_t)b * a.entries_seq_stride +
                                  orow * kEntryRecordBytes);
      }
      return;
    }
  }
  VO::store(a.entries, (int64_t)b * a.entries_seq_stride + orow * a.c + j0, out);
}

template <int DI, int DO>
hipError_t launch_typed(const CompressArgs& a, hipStream_t s) {
  const bool vec_ok = (a.c % Vec<DI>::N == 0) && (a.ld % Vec<DI>::N == 0) &&
                      (a.seq_stride % Vec<DI>::N == 0) && (a.halo_ld % Vec<DI>::N == 0) &&
                      (a.halo_seq_stride % Vec<DI>::N == 0) && (a.entries_seq_stride % Vec<DI>::N == 0) &&
                      Vec<DI>::N == Vec<DO>::N && a.aligned16;
  const int V = vec_ok ? Vec<DI>::N : 1;
  const int cv = a.c / V;
  // the epilogue's reductions need an entry's threads inside one wave
  if (a.epilogue && (cv > 64 || (cv & (cv - 1)) || (a.records && V != 8))) return hipErrorInvalidValue;
  if (a.fp4_codes && (!a.epilogue || (V != 4 && V != 8) || a.c % 32)) return hipErrorInvalidValue;
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

bool compress_epilogue_ok(const CompressArgs& a) {
  // one entry's channel vectors on consecutive lanes of one wave; records need one wave of 8 dims
  const int V = a.in_dtype == CSA_BF16 && a.out_dtype == CSA_BF16 ? 8 : (a.in_dtype == CSA_F32 && a.out_dtype == CSA_F32 ? 4 : 1);
  const int cv = a.c / V;
  if (a.m >= 64 || a.c % V || cv > 64 || (cv & (cv - 1))) return false;
  if (a.records && (a.c != 512 || V != 8 || a.out_dtype != CSA_BF16)) return false;
  if (a.fp4_codes && (a.c % 32 || V == 1 || a.records)) return false;
  return true;
}

hipError_t launch_compress(const CompressArgs& a0, hipStream_t s) {
  if (a0.n_new <= 0 || a0.B <= 0) return hipSuccess;
  CompressArgs a = a0;
  a.group = a.m >= 64 ? 16 : 1;  // threads per (entry, channel vector); every thread has >= 4 rows
  if (a.epilogue && (!compress_epilogue_ok(a) || a.group != 1)) return hipErrorInvalidValue;
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
