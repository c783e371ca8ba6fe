// Wave-level streaming top-k selection in LDS.
//
// Each candidate (score s, entry i) is packed into one 64-bit key that orders candidates exactly as
// the layer's selection does: larger score first, equal scores toward the smaller entry index.
//   high 32 bits: order-preserving map of the float32 score (-0 mapped to +0)
//   low  32 bits: ~i
// All keys of one query are distinct, so "the k largest keys" is a unique set and a threshold on
// the key selects it exactly.
//
// One wave owns one query's candidate buffer (capacity `cap` >= k + 64). Candidates above the
// running threshold are appended (ballot + prefix popcount, no atomics). When a batch would
// overflow the buffer, a radix select (8-bit digits, most significant first, histogram in LDS)
// finds a key at or below the k-th largest that keeps at most cap - 64 keys, the buffer is
// compacted to the keys at or above it, and the smallest kept key becomes the new threshold. The
// final selection resolves the exact k-th largest key. Candidates are offered in ascending entry
// order and every step keeps the buffer's order, so the kept entries come out in index order,
// padded with -1.
//
// Every function must be called by all 64 lanes of the wave with uniform arguments.
#pragma once

#include "common.h"

namespace csa {

__device__ __forceinline__ uint32_t score_to_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_cand(float s, uint32_t idx) {
  return ((uint64_t)score_to_key(s) << 32) | (uint32_t)(~idx);
}

struct WaveTopK {
  uint64_t* buf;   // LDS, cap entries
  uint32_t* hist;  // LDS, 256 counters
  int cap;
  int k;
  int cnt;         // wave-uniform
  uint64_t thr;    // wave-uniform: a candidate enters iff key > thr

  __device__ void init(uint64_t* b, uint32_t* h, int capacity, int kk) {
    buf = b;
    hist = h;
    cap = capacity;
    k = kk;
    cnt = 0;
    thr = 0;
  }

  // A threshold T such that the keys >= T among buf[0, cnt) are at least k and at most `limit`
  // (limit >= k; limit == k gives the exact k-th largest key). Requires cnt >= k >= 1.
  //
  // Radix select over 8-bit digits, most significant first, starting at the highest bit in which
  // the buffered keys differ (the bits above it are common to all of them). After each digit the
  // bin holding the k-th key is known; if keeping that whole bin stays within `limit`, its lower
  // bound is returned without resolving the remaining bits.
  __device__ uint64_t kth_threshold(int limit) {
    const int lane = lane_id();
    uint64_t mn = ~0ull, mx = 0ull;
    for (int i = lane; i < cnt; i += 64) {
      const uint64_t key = buf[i];
      mn = key < mn ? key : mn;
      mx = key > mx ? key : mx;
    }
    mn = wave_min_u64(mn);
    mx = wave_max_u64(mx);
    const uint64_t diff = mn ^ mx;
    if (diff == 0) return mx;  // a single key
    int top = 63 - __clzll((long long)diff);
    uint64_t pmask = top == 63 ? 0ull : ~((2ull << top) - 1ull);
    uint64_t prefix = mx & pmask;
    uint32_t krem = (uint32_t)k;       // keys still needed from those matching the prefix
    uint32_t kept_above = 0;           // keys above the prefix range
    while (true) {
      const int shift = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (uint32_t)((2ull << (top - shift)) - 1ull);
      for (int b = lane; b < 256; b += 64) hist[b] = 0;
      wave_sync();
      for (int base = 0; base < cnt; base += 256) {
        uint64_t kk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = base + j * 64 + lane;
          kk[j] = i < cnt ? buf[i] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = base + j * 64 + lane;
          if (i < cnt && (kk[j] & pmask) == prefix) atomicAdd(&hist[(uint32_t)(kk[j] >> shift) & dmask], 1u);
        }
      }
      wave_sync();
      // lane l owns digits 255-4l .. 252-4l, scanned from the top digit down
      uint32_t c[4];
      uint32_t local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        local += c[j];
      }
      const uint32_t incl = wave_incl_scan(local);
      const uint32_t excl = incl - local;
      const bool mine = (excl < krem) && (krem <= incl);
      const uint64_t who = __ballot(mine);
      const int src = __ffsll((unsigned long long)who) - 1;
      uint32_t digit = 0, above = excl, inbin = 0;
      if (mine) {
        uint32_t run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run + c[j] >= krem) {
            digit = 255u - 4u * lane - j;
            above = run;
            inbin = c[j];
            break;
          }
          run += c[j];
        }
      }
      digit = __shfl(digit, src, 64);
      above = __shfl(above, src, 64);
      inbin = __shfl(inbin, src, 64);
      wave_sync();
      prefix |= (uint64_t)digit << shift;
      pmask |= (uint64_t)dmask << shift;
      // keys >= prefix (its low bits zero): those above the range, above the bin, and the whole bin
      if (inbin == krem - above || kept_above + above + inbin <= (uint32_t)limit || shift == 0) return prefix;
      kept_above += above;
      krem -= above;
      top = shift - 1;
    }
  }

  // Keep the keys >= T at the front; the smallest kept becomes thr.
  __device__ void compact_to(uint64_t T) {
    const int lane = lane_id();
    int out = 0;
    uint64_t mn = ~0ull;
    for (int base = 0; base < cnt; base += 256) {
      uint64_t kk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j * 64 + lane;
        kk[j] = i < cnt ? buf[i] : 0ull;
      }
      wave_sync();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j * 64 + lane;
        const bool keep = (i < cnt) && (kk[j] >= T);
        const uint64_t bm = __ballot(keep);
        if (keep) {
          buf[out + __popcll(bm & lanemask_lt())] = kk[j];
          mn = kk[j] < mn ? kk[j] : mn;
        }
        out += __popcll(bm);
      }
      wave_sync();
    }
    cnt = out;
    thr = wave_min_u64(mn);
  }

  // Frees room while streaming: keeps at least k and at most cap - 64 keys.
  __device__ void shrink() { compact_to(kth_threshold(cap - 64)); }

  // Offer one candidate per lane (valid lanes only).
  __device__ void offer(uint64_t key, bool valid) {
    bool pass = valid && key > thr;
    uint64_t bm = __ballot(pass);
    int n = __popcll(bm);
    if (n == 0) return;
    if (cnt + n > cap) {
      shrink();
      pass = valid && key > thr;
      bm = __ballot(pass);
      n = __popcll(bm);
    }
    if (pass) buf[cnt + __popcll(bm & lanemask_lt())] = key;
    cnt += n;
    wave_sync();
  }

  // Final top-k, in entry index order; out_idx[j] (and out_score[j]) for j < k, -1 padded.
  // Every caller offers its candidates in ascending entry order, appends keep the lane (= entry)
  // order, and compaction is stable, so the buffer is always sorted by entry index: the exact
  // k-th-key compaction leaves the answer in order and nothing is sorted.
  __device__ void finish(int32_t* out_idx, float* out_score) {
    const int lane = lane_id();
    if (cnt > k) compact_to(kth_threshold(k));
    for (int j = lane; j < k; j += 64) {
      const bool have = j < cnt;
      const uint64_t v = have ? buf[j] : 0ull;
      out_idx[j] = have ? (int32_t)(~(uint32_t)v) : -1;
      if (out_score) out_score[j] = have ? key_to_score((uint32_t)(v >> 32)) : -INFINITY;
    }
    wave_sync();
  }
};

// LDS bytes one wave needs for a k-selection with capacity cap.
__host__ __device__ inline int topk_cap_for(int k, int slack) {
  int P = 1;
  while (P < k) P <<= 1;
  int cap = k + slack;
  if (cap < k + 64) cap = k + 64;
  if (cap < P) cap = P;
  return (cap + 63) & ~63;
}

}  // namespace csa
