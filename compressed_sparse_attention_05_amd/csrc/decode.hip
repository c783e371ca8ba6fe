// The decode state's append ("Anatomy of a Frontier Model", section "The attention: compress, then
// select", run token by token): each sequence's new token joins its state at the sequence's own
// position p, and when the token completes its block the entry (and, for CSA, its indexer key) is
// pooled at once, so a query on a block's last token sees that entry.
//
// One launch does the whole append for every sequence of the batch, whatever their positions:
//  * workgroup (0, b), the state of sequence b:
//      - the token's compressor inputs go to the block rows: CSA keeps two blocks, block i in rows
//        (i % 2) * m .. (i % 2) * m + m - 1, so the previous block stays in place and nothing is
//        shifted; HCA keeps the current block only (rows 0 .. m - 1);
//      - the raw KV goes to window ring row p % W, RMS-normalised and rotated at p when the layer
//        has QK-norm / RoPE ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE");
//      - when (p + 1) % m == 0, entry i = (p + 1) / m - 1 is pooled per channel (CSA: softmax over
//        the own block's logits with bias_a and the previous block's with bias_b, "The Exchange
//        Rates of a Million Tokens", section 3; HCA: the own block only), rounded to the storage
//        type, normalised and rotated at p (its block's last token) when on, and stored as a row
//        or packed into a 584-byte record; the CSA indexer key is pooled the same way;
//  * workgroups (1 .., b), when the query is normalised or rotated: four query heads each, one per
//    wave, normalised and rotated at p into the caller's buffer;
//  * with an MXFP4 indexer, the pooled key is quantised (mx.h) into the key cache, and the last
//    workgroups of each sequence quantise its indexer query, 2048 values each.
// The pooling takes the rows in the order of the prefill compressor (compress.hip), so an entry
// pooled here has the bits the chunked prefill gives it.
#include "kernels.h"
#include "mx.h"
#include "pool.h"
#include "record.h"
#include "rope.h"

namespace csa {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kMaxPer = 16;  // dims per lane of a head vector (D <= 1024)

// v[j] = element lane + 64 j of a head vector of D dims (zero past D)
template <int DT>
__device__ __forceinline__ void load_strided(const void* p, int64_t off, int D, float (&v)[kMaxPer]) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int d = lane + 64 * j;
    v[j] = d < D ? load_elem<DT>(p, off + d) : 0.f;
  }
}

// RMS norm with gain (gamma != nullptr) and rotation of the last rope_dims dims at position pos,
// on a head vector held as v[j] = dim lane + 64 j; the value is then rounded to the storage type
// (bf16: RNE) as a store would leave it.
template <int DT>
__device__ __forceinline__ void norm_rope_strided(float (&v)[kMaxPer], int D, const float* gamma, float eps,
                                                  int rope_dims, double lt, int64_t pos) {
  const int lane = lane_id();
  if (gamma) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) ss = fmaf(v[j], v[j], ss);
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int d = lane + 64 * j;
      if (d < D) v[j] = v[j] * inv * gamma[d];
    }
  }
  if (rope_dims > 0) {
    // only the 64-dim chunks that hold rotated dims, in a loop that is not unrolled (one copy of the
    // angle code); chunk j's value is picked from and put back into v by selects on the uniform j
    const int rs = D - rope_dims;
#pragma unroll 1
    for (int j = rs / 64; j < (D + 63) / 64; ++j) {
      float x = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxPer; ++t) x = t == j ? v[t] : x;
      const int d = lane + 64 * j;
      const float other = __shfl_xor(x, 1, 64);
      if (d >= rs && d < D) {
        float c, s;
        rope_cos_sin((double)pos, (d - rs) >> 1, rope_dims, lt, false, c, s);
        x = ((d - rs) & 1) == 0 ? x * c - other * s : other * s + x * c;
      }
#pragma unroll
      for (int t = 0; t < kMaxPer; ++t) v[t] = t == j ? x : v[t];
    }
  }
  if (DT == CSA_BF16) {
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) v[j] = bf2f(f2bf(v[j]));
  }
}

template <int DT>
__device__ __forceinline__ void store_strided(void* p, int64_t off, int D, const float (&v)[kMaxPer]) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int d = lane + 64 * j;
    if (d < D) store_elem<DT>(p, off + d, v[j]);
  }
}

// Pools channel vector j0 .. j0 + V - 1 of one entry: the own block's rows (series a: values at
// column ca, logits at column za, biases bias_a) and, when prev is given, the previous block's rows
// (series b: cb, zb, bias_b); rows are `ld` elements apart. G threads share the vector (thread sub
// takes rows sub, sub + G, ...) and meet through a butterfly, as in the prefill compressor.
template <class VI>
__device__ __forceinline__ void pool_entry(const void* own, const void* prev, int64_t ld, int m, int c,
                                           int64_t col_ca, int64_t col_za, int64_t col_cb, int64_t col_zb,
                                           const float* bias_a, const float* bias_b, int j0, int sub, int G,
                                           float* out) {
  constexpr int V = VI::N;
  constexpr int kRows = 8;
  float mx[V], den[V], num[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    mx[v] = -INFINITY;
    den[v] = 0.f;
    num[v] = 0.f;
  }
  for (int series = 0; series < (prev ? 2 : 1); ++series) {
    const void* base = series == 0 ? own : prev;
    const int64_t cc = series == 0 ? col_ca : col_cb, cz = series == 0 ? col_za : col_zb;
    const float* bias = series == 0 ? bias_a : bias_b;
    for (int r0 = sub; r0 < m; r0 += kRows * G) {
      float z[kRows][V], cv[kRows][V];
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        if (r0 + q * G >= m) break;
        const int64_t row = (int64_t)(r0 + q * G) * ld + j0;
        VI::load(base, row + cz, z[q]);
        VI::load(base, row + cc, cv[q]);
      }
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        if (r0 + q * G >= m) break;
        float bs[V];
#pragma unroll
        for (int v = 0; v < V; ++v) bs[v] = bias[(r0 + q * G) * c + j0 + v];
        accumulate<V>(z[q], bs, cv[q], mx, den, num);
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
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = num[v] / den[v];
}

__device__ __forceinline__ const void* elem_ptr(const void* p, int64_t off, int es) {
  return static_cast<const uint8_t*>(p) + off * es;
}

template <int DT, class VI>
__global__ void __launch_bounds__(kAppendThreads) append_kernel(AppendArgs a) {
  constexpr int es = DT == CSA_F32 ? 4 : 2;
  const int b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int64_t p = pos_at(a.pos, b);
  const int m = a.m, D = a.D, DI = a.D_I;
  const double lt = a.rope_dims > 0 ? log2(a.theta) : 0.0;

  const int nq = a.qn ? (a.H + kAppendThreads / 64 - 1) / (kAppendThreads / 64) : 0;
  if ((int)blockIdx.x > nq) {  // the indexer query to MXFP4: 8 values per thread, 4 lanes per block
    const int64_t n = (int64_t)a.H_I * DI;
    const int64_t j0 = ((int64_t)(blockIdx.x - 1 - nq) * kAppendThreads + tid) * 8;
    if (j0 >= n) return;  // whole blocks of 32: n is a multiple of 32
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i += VI::N) VI::load(a.q_idx, b * n + j0 + i, v + i);
    int X;
    const uint32_t pk = mxfp4_quant_lanes<8>(v, X);
    mxfp4_store_lanes<8>(a.qi_codes + b * (n / 2), a.qi_scales + b * (n / 32), (int)j0, pk, X);
    return;
  }
  if (blockIdx.x > 0) {  // query heads, normalised and rotated at p
    const int h = (blockIdx.x - 1) * (kAppendThreads / 64) + wave;
    if (h >= a.H) return;
    const int64_t off = ((int64_t)b * a.H + h) * D;
    float v[kMaxPer];
    load_strided<DT>(a.q, off, D, v);
    norm_rope_strided<DT>(v, D, a.gamma_q, a.eps, a.rope_dims, lt, p);
    store_strided<DT>(a.qn, off, D, v);
    return;
  }

  __shared__ float ent[1024];  // the pooled entry (D <= 1024)
  __shared__ float kent[1024];  // the pooled indexer key when it is quantised (D_I <= 1024)
  const int64_t blk = p / m;
  const int r = (int)(p % m);
  const int64_t nc = a.hca ? 2LL * D : 4LL * D + 4LL * DI;
  uint8_t* block = static_cast<uint8_t*>(a.block) + (int64_t)b * (a.hca ? m : 2 * m) * nc * es;
  const int64_t own_row0 = a.hca ? 0 : (blk & 1) * m;
  // the token's compressor inputs (16 bytes per thread and step when rows are 16-byte multiples)
  {
    const uint8_t* src = static_cast<const uint8_t*>(a.comp) + (int64_t)b * nc * es;
    uint8_t* dst = block + (own_row0 + r) * nc * es;
    const int64_t nbytes = nc * es;
    if (nbytes % 16 == 0 && a.aligned16) {
      for (int64_t i = tid; i < nbytes / 16; i += kAppendThreads)
        reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
      for (int64_t i = tid; i < nbytes; i += kAppendThreads) dst[i] = src[i];
    }
  }
  // the raw KV into its ring row
  if (wave == 1) {
    float v[kMaxPer];
    load_strided<DT>(a.kv, (int64_t)b * D, D, v);
    if (a.gamma_kv || a.rope_dims > 0) norm_rope_strided<DT>(v, D, a.gamma_kv, a.eps, a.rope_dims, lt, p);
    store_strided<DT>(a.win, ((int64_t)b * a.W + p % a.W) * D, D, v);
  }
  if ((p + 1) % m != 0 || blk >= a.n_cap) return;  // uniform over the workgroup
  __syncthreads();  // the block's rows, this token's included, are in place

  // pool the entry (and the indexer key): thread slots over the channel vectors
  constexpr int V = VI::N;
  const int G = (a.hca && m >= 64) ? 16 : 1;  // threads per vector, as in the prefill compressor
  const int nve = D / V, nvk = a.hca ? 0 : DI / V;
  const void* own = block + own_row0 * nc * es;
  const void* prev = (!a.hca && blk >= 1) ? block + (int64_t)((blk + 1) & 1) * m * nc * es : nullptr;
  const bool finish = a.entry_fmt != 0 || a.gamma_kv || a.rope_dims > 0;  // the entry passes through LDS
  const bool kfp4 = !a.hca && a.key_fmt != 0;                              // so does an MXFP4 key
  for (int slot = tid / G; slot < nve + nvk; slot += kAppendThreads / G) {
    const int sub = tid % G;
    float out[V];
    if (slot < nve) {
      const int j0 = slot * V;
      if (a.hca)
        pool_entry<VI>(own, nullptr, nc, m, D, 0, D, 0, 0, a.bias_a, nullptr, j0, sub, G, out);
      else
        pool_entry<VI>(own, prev, nc, m, D, 0, D, 2LL * D, 3LL * D, a.bias_a, a.bias_b, j0, sub, G, out);
      if (sub == 0) {
        if (finish) {
#pragma unroll
          for (int v = 0; v < V; ++v) ent[j0 + v] = DT == CSA_BF16 ? bf2f(f2bf(out[v])) : out[v];
        } else {
          VI::store(a.entries, ((int64_t)b * a.n_cap + blk) * D + j0, out);
        }
      }
    } else {
      const int j0 = (slot - nve) * V;
      const int64_t c0 = 4LL * D;
      pool_entry<VI>(own, prev, nc, m, DI, c0, c0 + DI, c0 + 2LL * DI, c0 + 3LL * DI, a.ibias_a, a.ibias_b, j0, sub,
                     G, out);
      if (sub == 0) {
        if (kfp4) {
#pragma unroll
          for (int v = 0; v < V; ++v) kent[j0 + v] = DT == CSA_BF16 ? bf2f(f2bf(out[v])) : out[v];
        } else {
          VI::store(a.keys, ((int64_t)b * a.n_cap + blk) * DI + j0, out);
        }
      }
    }
  }
  if (!finish && !kfp4) return;
  __syncthreads();
  if (kfp4 && wave == 1) {  // the stored key to MXFP4: 4 dims per lane, 8 lanes per block of 32
    const int64_t row = (int64_t)b * a.n_cap + blk;
    for (int base = 0; base < DI; base += 256) {
      const int j0 = base + 4 * lane;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = j0 + i < DI ? kent[j0 + i] : 0.f;
      int X;
      const uint32_t pk = mxfp4_quant_lanes<4>(v, X);
      if (j0 < DI)
        mxfp4_store_lanes<4>(static_cast<uint8_t*>(a.keys) + row * (DI / 2), a.key_scales + row * (DI / 32), j0, pk, X);
    }
  }
  if (!finish || wave != 0) return;
  // wave 0: normalise and rotate the entry at p (its block's last token), then store or pack it
  float v[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int d = lane + 64 * j;
    v[j] = d < D ? ent[d] : 0.f;
  }
  if (a.gamma_kv || a.rope_dims > 0) norm_rope_strided<DT>(v, D, a.gamma_kv, a.eps, a.rope_dims, lt, p);
  if (a.entry_fmt == 0) {
    store_strided<DT>(a.entries, ((int64_t)b * a.n_cap + blk) * D, D, v);
    return;
  }
  // records (D = 512): regroup so that lane l holds dims 8l .. 8l + 7
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int d = lane + 64 * j;
    if (d < D) ent[d] = v[j];
  }
  wave_sync();
  float w8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w8[j] = ent[8 * lane + j];
  pack_record_wave(w8, static_cast<uint8_t*>(a.entries) + ((int64_t)b * a.n_cap + blk) * kEntryRecordBytes);
}

template <int DT>
hipError_t launch_typed(const AppendArgs& a, hipStream_t s) {
  const int nq = a.qn ? (int)ceil_div(a.H, kAppendThreads / 64) : 0;
  const int nqi = a.qi_codes ? (int)ceil_div((int64_t)a.H_I * a.D_I, kAppendThreads * 8) : 0;
  if ((a.key_fmt != 0 && (a.hca || a.D_I % 32)) || (a.qi_codes && (a.H_I * a.D_I) % 32)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(1 + nq + nqi), (unsigned)a.B), block(kAppendThreads);
  constexpr int V = Vec<DT>::N;
  const bool vec = a.aligned16 && a.D % V == 0 && (a.hca || a.D_I % V == 0);
  if (vec) hipLaunchKernelGGL((append_kernel<DT, Vec<DT>>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((append_kernel<DT, Scalar<DT>>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  return a.dtype == CSA_BF16 ? launch_typed<CSA_BF16>(a, s) : launch_typed<CSA_F32>(a, s);
}

int append_max_dim() { return 64 * kMaxPer; }

}  // namespace csa
