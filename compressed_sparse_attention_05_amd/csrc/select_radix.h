// Multi-workgroup exact top-k over materialised score rows (the decode shape: few rows, up to
// millions of candidates per row).
//
// Keys are the same 64-bit keys as the streaming selection (topk_wave.h): order-preserving score
// bits in the high half, ~index in the low half, so the k largest keys are the layer's top-k.
//   pass A  (sel_hist, many workgroups per row): a 4096-bin histogram of the top 12 bits of every
//           row's score keys, built in LDS per workgroup and added to the row's global histogram
//           (integer atomics: the totals are exact and order-independent);
//   pass B  (sel_collect, many workgroups per row): every workgroup finds the row's boundary digit
//           d (the 12-bit bin holding the k-th key) from the histogram, then appends its
//           candidates with digit > d to the row's "above" list (fewer than k of them) and those
//           with digit == d to the row's "boundary" list;
//   pass C  (sel_final, one workgroup per row): a block radix select over the boundary list picks
//           the k - |above| largest, and the union is written in entry-index order.
// List order depends on atomic slot assignment, but the selected set does not, and the output is
// sorted: results are deterministic.
#pragma once

#include "topk_wave.h"

namespace csa {

constexpr int kSelBins = 4096;     // 12-bit first digit
constexpr int kSelShift = 20;      // key32 >> 20
constexpr int kSelChunk = 4096;    // scores per workgroup in pass B
constexpr int kSelThreads = 256;

struct SelWork {
  uint32_t* hist;      // [R, kSelBins]
  uint32_t* cnt;       // [R, 4]: above count, boundary count (two words unused)
  uint64_t* above;     // [R, k]
  uint64_t* bnd;       // [R, n]
};

// Adds a workgroup-local histogram (LDS, kSelBins counters) to the row's global histogram.
__device__ __forceinline__ void sel_flush_hist(const uint32_t* lh, uint32_t* gh) {
  for (int b = threadIdx.x; b < kSelBins; b += blockDim.x) {
    const uint32_t c = lh[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

__device__ __forceinline__ void sel_zero_lds_hist(uint32_t* lh) {
  for (int b = threadIdx.x; b < kSelBins; b += blockDim.x) lh[b] = 0u;
}

// Block-wide inclusive scan of one value per thread (blockDim.x == kSelThreads).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* scratch4) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  uint32_t incl = wave_incl_scan(v);
  if (lane == 63) scratch4[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += scratch4[w];
  __syncthreads();
  return incl + off;
}

}  // namespace csa
