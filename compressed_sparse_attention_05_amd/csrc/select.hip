// Exact top-k over materialised score rows with many workgroups per row (see select_radix.h).
#include "kernels.h"
#include "select_radix.h"

namespace csa {

namespace {

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ void __launch_bounds__(256) sel_zero(uint32_t* hist, uint32_t* cnt, int R) {
  const int64_t n = (int64_t)R * kSelBins;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) hist[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 4LL * R; i += stride) cnt[i] = 0u;
}

__device__ __forceinline__ int64_t row_valid(const int32_t* n_valid, int64_t row, int64_t ld) {
  int64_t nv = n_valid[row];
  return nv < 0 ? 0 : (nv > ld ? ld : nv);
}

// Pass A on caller scores: histogram of the top 12 key bits per row.
__global__ void __launch_bounds__(kSelThreads) sel_hist(const float* scores, int64_t ld, const int32_t* n_valid,
                                                        uint32_t* hist) {
  __shared__ uint32_t lh[kSelBins];
  const int64_t row = blockIdx.y;
  const int64_t nv = row_valid(n_valid, row, ld);
  const int64_t base = (int64_t)blockIdx.x * kSelChunk;
  if (base >= nv) return;
  sel_zero_lds_hist(lh);
  __syncthreads();
  const int64_t end = base + kSelChunk < nv ? base + kSelChunk : nv;
  const float* s = scores + row * ld;
  constexpr int kPer = kSelChunk / kSelThreads;
  uint32_t dg[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {  // all loads first, then the LDS atomics
    const int64_t i = base + (int64_t)j * kSelThreads + threadIdx.x;
    dg[j] = i < end ? score_to_key(s[i]) >> kSelShift : kSelBins;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (dg[j] < (uint32_t)kSelBins) atomicAdd(&lh[dg[j]], 1u);
  __syncthreads();
  sel_flush_hist(lh, hist + row * kSelBins);
}

// Pass B: boundary digit of the row, then classify this workgroup's chunk.
__global__ void __launch_bounds__(kSelThreads) sel_collect(const float* scores, int64_t ld, const int32_t* n_valid,
                                                           int k, SelWork w) {
  __shared__ uint32_t scan4[4];
  __shared__ uint32_t sh_d;
  const int64_t row = blockIdx.y;
  const int64_t nv = row_valid(n_valid, row, ld);
  const int64_t base = (int64_t)blockIdx.x * kSelChunk;
  if (base >= nv) return;
  const int tid = threadIdx.x;
  const bool all = nv <= k;
  uint32_t d = 0;
  if (!all) {
    const uint32_t* h = w.hist + row * kSelBins;
    constexpr int per = kSelBins / kSelThreads;  // 16 bins per thread, scanned from the top digit down
    uint32_t c[per];
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      c[j] = h[kSelBins - 1 - per * tid - j];
      local += c[j];
    }
    const uint32_t incl = block_incl_scan(local, scan4);
    const uint32_t excl = incl - local;
    if (excl < (uint32_t)k && (uint32_t)k <= incl) {
      uint32_t run = excl;
      for (int j = 0; j < per; ++j) {
        if (run + c[j] >= (uint32_t)k) {
          sh_d = kSelBins - 1 - per * tid - j;
          break;
        }
        run += c[j];
      }
    }
    __syncthreads();
    d = sh_d;
  }
  const float* s = scores + row * ld;
  uint32_t* cnt = w.cnt + row * 4;
  uint64_t* above = w.above + row * k;
  uint64_t* bnd = w.bnd + row * ld;
  // classify this thread's scores, count per wave, then one atomic per list per workgroup
  constexpr int kPer = kSelChunk / kSelThreads;
  uint64_t keyv[kPer];
  uint32_t cls = 0;  // bit 2j: above, bit 2j+1: boundary
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = base + (int64_t)j * kSelThreads + tid;
    const bool valid = i < nv;
    const float v = valid ? s[i] : 0.f;
    const uint32_t key = score_to_key(v);
    const uint32_t dig = key >> kSelShift;
    const bool isA = valid && (all || dig > d);
    const bool isB = valid && !all && dig == d;
    keyv[j] = ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)i);
    cls |= (isA ? 1u : 0u) << (2 * j);
    cls |= (isB ? 1u : 0u) << (2 * j + 1);
  }
  uint32_t nA = 0, nB = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    nA += (cls >> (2 * j)) & 1u;
    nB += (cls >> (2 * j + 1)) & 1u;
  }
  // block-exclusive offsets of this thread's A and B candidates
  const uint32_t packed = nA | (nB << 16);  // at most 16 each per thread, 4096 per block: fits 16 bits
  const uint32_t incl = block_incl_scan(packed, scan4);
  __shared__ uint32_t base_ab[2];
  if (tid == kSelThreads - 1) {
    const uint32_t totA = incl & 0xFFFFu, totB = incl >> 16;
    base_ab[0] = totA ? atomicAdd(&cnt[0], totA) : 0u;
    base_ab[1] = totB ? atomicAdd(&cnt[1], totB) : 0u;
  }
  __syncthreads();
  uint32_t offA = base_ab[0] + ((incl - packed) & 0xFFFFu);
  uint32_t offB = base_ab[1] + ((incl - packed) >> 16);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((cls >> (2 * j)) & 1u) above[offA++] = keyv[j];
    if ((cls >> (2 * j + 1)) & 1u) bnd[offB++] = keyv[j];
  }
}

// Pass C: exact selection among the boundary candidates, then the selected entries in index order.
// The boundary list is staged in LDS when it fits. Ordering: rows of up to kBitmapMax entries mark
// the selected indices in an LDS bitmap, and each entry's output slot is the number of marked
// indices below it (word prefix counts + popcount), so no sort is needed; longer rows fall back to
// a bitonic sort.
constexpr int kBndCache = 4096;        // boundary keys staged in LDS
constexpr int kBitmapMax = 262144;     // entries per row ordered through the bitmap

struct FinalSmem {
  uint64_t bc[kBndCache];              // boundary keys
  uint32_t bm[kBitmapMax / 32];        // selected-index bitmap
  uint16_t wc[kBitmapMax / 32];        // exclusive popcount per bitmap word
  uint32_t hist[256];
  uint32_t scan4[4];
  uint32_t sh[3];
  uint32_t nsel;
};

__global__ void __launch_bounds__(kSelThreads) sel_final(const int32_t* n_valid, int64_t ld, int k, SelWork w,
                                                         int32_t* out_idx, float* out_score) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  FinalSmem& sm = *reinterpret_cast<FinalSmem*>(smem_raw);
  uint64_t* sel = reinterpret_cast<uint64_t*>(smem_raw + sizeof(FinalSmem));  // next_pow2(k) keys
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t nv = row_valid(n_valid, row, ld);
  const int ntake = (int)(nv < k ? nv : k);
  const uint32_t na = w.cnt[row * 4], nb = w.cnt[row * 4 + 1];
  const int krem = ntake - (int)na;
  const uint64_t* A = w.above + row * k;
  const uint64_t* Bg = w.bnd + row * ld;
  for (uint32_t i = tid; i < na; i += kSelThreads) sel[i] = A[i];
  const bool cached = nb <= (uint32_t)kBndCache;
  if (krem > 0 && cached)
    for (uint32_t i = tid; i < nb; i += kSelThreads) sm.bc[i] = Bg[i];
  __syncthreads();
  const uint64_t* Bl = cached ? sm.bc : Bg;
  uint64_t T = 0;
  if (krem > 0 && (uint32_t)krem < nb) {
    // every boundary key shares the top 12 bits (the boundary digit): start below them
    const uint64_t known = ~0ull << (32 + kSelShift);
    uint64_t prefix = Bl[0] & known, pmask = known;
    uint32_t kr = (uint32_t)krem;
    for (int shift = 32 + kSelShift - 8; shift >= 0; shift = shift >= 8 ? shift - 8 : (shift > 0 ? 0 : -1)) {
      sm.hist[tid] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < nb; i += kSelThreads) {
        const uint64_t key = Bl[i];
        if ((key & pmask) == prefix) atomicAdd(&sm.hist[(uint32_t)(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t c = sm.hist[255 - tid];
      const uint32_t incl = block_incl_scan(c, sm.scan4);
      const uint32_t excl = incl - c;
      if (excl < kr && kr <= incl) {
        sm.sh[0] = 255 - tid;
        sm.sh[1] = excl;
        sm.sh[2] = c;
      }
      __syncthreads();
      const uint32_t digit = sm.sh[0], ab = sm.sh[1], inbin = sm.sh[2];
      __syncthreads();
      prefix |= (uint64_t)digit << shift;
      pmask |= 255ull << shift;
      kr -= ab;
      if (inbin == kr) break;
    }
    T = prefix;
  }
  if (tid == 0) sm.nsel = na;
  __syncthreads();
  if (krem > 0) {
    for (uint32_t i = tid; i < nb; i += kSelThreads) {
      const uint64_t key = Bl[i];
      if (key >= T) sel[atomicAdd(&sm.nsel, 1u)] = key;
    }
  }
  __syncthreads();
  const int have = (int)sm.nsel;  // == ntake
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;
  for (int j = have + tid; j < k; j += kSelThreads) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
  if (nv <= kBitmapMax) {
    const int nw = (int)((nv + 31) / 32);
    for (int i = tid; i < nw; i += kSelThreads) sm.bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < have; i += kSelThreads) {
      const uint32_t idx = ~(uint32_t)sel[i];
      atomicOr(&sm.bm[idx >> 5], 1u << (idx & 31));
    }
    __syncthreads();
    const int wpt = (nw + kSelThreads - 1) / kSelThreads;
    const int w0 = tid * wpt, w1 = w0 + wpt < nw ? w0 + wpt : nw;
    uint32_t local = 0;
    for (int i = w0; i < w1; ++i) local += __popc(sm.bm[i]);
    uint32_t run = block_incl_scan(local, sm.scan4) - local;
    for (int i = w0; i < w1; ++i) {
      sm.wc[i] = (uint16_t)run;
      run += __popc(sm.bm[i]);
    }
    __syncthreads();
    for (int i = tid; i < have; i += kSelThreads) {
      const uint64_t key = sel[i];
      const uint32_t idx = ~(uint32_t)key;
      const uint32_t wd = idx >> 5;
      const int rank = sm.wc[wd] + __popc(sm.bm[wd] & ((1u << (idx & 31)) - 1u));
      oi[rank] = (int32_t)idx;
      if (os) os[rank] = key_to_score((uint32_t)(key >> 32));
    }
    return;
  }
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = tid; i < P; i += kSelThreads) {
    uint64_t v = ~0ull;
    if (i < have) {
      const uint64_t key = sel[i];
      v = ((uint64_t)(~(uint32_t)key) << 32) | (key >> 32);
    }
    sel[i] = v;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (P >> 1); t += kSelThreads) {
        const int i = (t / stride) * stride * 2 + (t % stride);
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t a = sel[i], b = sel[j];
        if ((a > b) == up) {
          sel[i] = b;
          sel[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < have; j += kSelThreads) {
    const uint64_t v = sel[j];
    oi[j] = (int32_t)(uint32_t)(v >> 32);
    if (os) os[j] = key_to_score((uint32_t)v);
  }
}

SelWork carve(void* ws, int R, int64_t ld, int k) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  SelWork w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += a256((size_t)R * kSelBins * 4);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += a256((size_t)R * 4 * 4);
  w.above = reinterpret_cast<uint64_t*>(p);
  p += a256((size_t)R * k * 8);
  w.bnd = reinterpret_cast<uint64_t*>(p);
  return w;
}

}  // namespace

size_t select_workspace(int R, int64_t ld, int k) {
  return a256((size_t)R * kSelBins * 4) + a256((size_t)R * 4 * 4) + a256((size_t)R * k * 8) + a256((size_t)R * ld * 8);
}

uint32_t* select_hist(void* ws) { return static_cast<uint32_t*>(ws); }

int64_t select_zero_words(int R) { return (int64_t)((a256((size_t)R * kSelBins * 4) + (size_t)R * 4 * 4) / 4); }

hipError_t launch_select_zero(void* ws, int R, int64_t ld, int k, hipStream_t s) {
  SelWork w = carve(ws, R, ld, k);
  const int64_t n = (int64_t)R * kSelBins;
  unsigned g = (unsigned)ceil_div(n, 256);
  if (g > 1024) g = 1024;
  hipLaunchKernelGGL(sel_zero, dim3(g), dim3(256), 0, s, w.hist, w.cnt, R);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k, int32_t* out_idx,
                         float* out_score, void* ws, bool zeroed, hipStream_t s) {
  SelWork w = carve(ws, R, ld, k);
  hipError_t e;
  const unsigned nchunks = (unsigned)(ceil_div(ld, kSelChunk) > 0 ? ceil_div(ld, kSelChunk) : 1);
  if (!zeroed && (e = launch_select_zero(ws, R, ld, k, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_hist, dim3(nchunks, (unsigned)R), dim3(kSelThreads), 0, s, scores, ld, n_valid, w.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_collect, dim3(nchunks, (unsigned)R), dim3(kSelThreads), 0, s, scores, ld, n_valid, k, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int P = 1;
  while (P < k) P <<= 1;
  const int lds = (int)sizeof(FinalSmem) + P * 8;
  if ((e = allow_lds((const void*)sel_final, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_final, dim3((unsigned)R), dim3(kSelThreads), lds, s, n_valid, ld, k, w, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace csa
