// Exact top-k of long materialised score rows (decode: few rows, up to millions of entries each;
// "Anatomy of a Frontier Model", bullet "Compressed Sparse Attention (CSA)": each query keeps the
// 1,024 entries the indexer ranks highest).
//
// Keys are the 64-bit keys of the streaming selection (topk_wave.h): order-preserving score bits in
// the high half, ~index in the low half, so the k largest keys are the layer's top-k (ties toward the
// smaller index) and all keys of a row are distinct.
//
// A lower bound first: split the row into G groups of gs consecutive entries. If G >= k, the k-th
// largest group maximum T0 is at most the k-th largest score (k distinct groups each hold an entry
// >= T0), so every entry of the top-k has a score >= T0. With G ~ 2k groups few entries clear T0
// (about 1.4 k for independent scores), so the exact selection runs over a short list.
//   sel_gmax     (csa_topk_from_scores only: the decode indexer writes the maxima with its scores)
//                the maxima of every g0 consecutive entries (g0 = min(gs, 64): one wave's lanes)
//   sel_collect  (many workgroups per row) T0 from the row's group maxima (the lower bound of the
//                bin, in one histogram pass over their range, that holds the k-th largest), then
//                every entry of its piece with a score key >= T0 is appended to the row's candidate
//                list (one atomic per workgroup; the list order varies, the set does not)
//   sel_final    (one workgroup per row) the exact k-th largest key of the candidates (12-bit
//                histogram passes over the range that holds it, from LDS when the candidates fit,
//                else from the global list), then the k selected entries in index order (ranks from
//                a bitmap of the selected indices; a bitonic sort for rows beyond the bitmap).
//   sel_row      (rows of up to 32K scores, which need no group maxima: one workgroup per row, one
//                launch) the row held in registers, radix passes over its key range.
// Rows with at most k valid entries keep them all.
#include "kernels.h"
#include "topk_wave.h"

namespace csa {

namespace {

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kCollectThreads = 256;
constexpr int kCollectPer = 16;                                  // scores per thread
constexpr int kCollectPiece = kCollectThreads * kCollectPer;     // scores per workgroup
constexpr int kFinalThreads = 1024;
constexpr int kFinalCap = 8192;                                  // candidates held in LDS

__device__ __forceinline__ int64_t row_valid(const int32_t* n_valid, int64_t row, int64_t ld) {
  int64_t nv = n_valid[row];
  return nv < 0 ? 0 : (nv > ld ? ld : nv);
}

// Block-wide exclusive scan of one value per thread; wsum holds one word per wave.
template <int BT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum) {
  constexpr int NW = BT / 64;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) off += w < wave ? wsum[w] : 0u;
  __syncthreads();
  return off + incl - v;
}

// Four consecutive scores of a row from i on, loaded without a branch so that a thread's loads all go
// out together: indices are clamped into the row (ld entries; entries past the valid count are masked
// by the caller). vec: rows of a multiple of 4 floats at a 16-byte aligned base.
__device__ __forceinline__ void load4(const float* srow, int64_t ld, int64_t i, bool vec, float* v) {
  if (vec) {
    const int64_t ic = i + 4 <= ld ? i : ld - 4;
    const float4 f = *reinterpret_cast<const float4*>(srow + ic);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = srow[i + e < ld ? i + e : ld - 1];
  }
}

constexpr int kBins = 4096;  // 12-bit digits of the radix passes

// Block-wide minimum and maximum of keys (KT = uint32_t or uint64_t); red: 2 * (BT / 64) words.
template <int BT, class KT>
__device__ __forceinline__ void block_minmax(KT& mn, KT& mx, KT* red) {
  constexpr int NW = BT / 64;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  for (int o = 32; o > 0; o >>= 1) {
    KT a, b;
    if constexpr (sizeof(KT) == 8) {
      a = shfl_u64(mn, lane ^ o);
      b = shfl_u64(mx, lane ^ o);
    } else {
      a = (KT)__shfl_xor((uint32_t)mn, o, 64);
      b = (KT)__shfl_xor((uint32_t)mx, o, 64);
    }
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) {
    red[wave] = mn;
    red[NW + wave] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    mn = red[w] < mn ? red[w] : mn;
    mx = red[NW + w] > mx ? red[NW + w] : mx;
  }
  __syncthreads();
}

// One histogram pass over the keys in [lo, lo + span] (key_at(i), i < n): kBins bins of width 2^sh,
// sh = max(0, bits(span) - 12), so keys that share their high bits still spread over the bins. Finds
// the bin holding the krem-th largest of those keys: returns its index d; above = keys in higher
// bins, inbin = keys in it. sh: the shift used. hist: kBins words, wsum: BT / 64 words, out: 3 words.
template <int BT, class KT, class KeyAt>
__device__ uint32_t range_pass(int64_t n, KeyAt key_at, KT lo, KT span, uint32_t krem, int& sh, uint32_t& above,
                               uint32_t& inbin, uint32_t* hist, uint32_t* wsum, uint32_t* out) {
  constexpr int KB = 8 * (int)sizeof(KT);
  constexpr int PER = kBins / BT;  // bins per thread, scanned from the top down
  const int tid = threadIdx.x;
  const int bits = span == 0 ? 0 : KB - (sizeof(KT) == 8 ? __clzll((long long)span) : __clz((int)span));
  sh = bits > 12 ? bits - 12 : 0;
  for (int b = tid; b < kBins; b += BT) hist[b] = 0u;
  __syncthreads();
  for (int64_t i = tid; i < n; i += BT) {
    const KT v = key_at(i);
    const KT u = v - lo;
    if (v >= lo && u <= span) atomicAdd(&hist[(uint32_t)(u >> sh)], 1u);
  }
  __syncthreads();
  uint32_t cnt[PER], local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cnt[j] = hist[kBins - 1 - PER * tid - j];
    local += cnt[j];
  }
  const uint32_t excl = block_excl_scan<BT>(local, wsum);
  if (excl < krem && krem <= excl + local) {
    uint32_t run = excl;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (run < krem && krem <= run + cnt[j]) {
        out[0] = (uint32_t)(kBins - 1 - PER * tid - j);
        out[1] = run;
        out[2] = cnt[j];
      }
      run += cnt[j];
    }
  }
  __syncthreads();
  const uint32_t d = out[0];
  above = out[1];
  inbin = out[2];
  __syncthreads();
  return d;
}

// The g0-maxima of rows of scores (csa_topk_from_scores); zeroes the candidate counters.
__global__ void __launch_bounds__(256) sel_gmax(const float* scores, int64_t ld, const int32_t* n_valid, int g0,
                                               int64_t gstride, float* gmax, uint32_t* cnt) {
  const int64_t row = blockIdx.y;
  if (blockIdx.x == 0 && threadIdx.x == 0) cnt[row] = 0u;
  const int64_t nv = row_valid(n_valid, row, ld);
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64; base < nv; base += waves * 64) {
    const int64_t i = base + lane;
    float v = i < nv ? scores[row * ld + i] : -INFINITY;
    for (int o = 1; o < g0; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if ((lane & (g0 - 1)) == 0 && i < nv) gmax[row * gstride + i / g0] = v;
  }
}

// Scratch of the selection between its kernels.
struct SelBufs {
  uint32_t* cnt;   // [R] candidates appended per row (zero before sel_collect)
  float* gmax;     // [R, gstride] maxima of g0 consecutive scores
  uint64_t* cand;  // [R, ld] candidate keys
};

__global__ void __launch_bounds__(kCollectThreads) sel_collect(const float* scores, int64_t ld,
                                                                const int32_t* n_valid, int k, SelPlan pl,
                                                                SelBufs w) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[2 * (kCollectThreads / 64)];
  __shared__ uint32_t sh3[kCollectThreads / 64 + 4];
  const int64_t row = blockIdx.y;
  const int64_t nv = row_valid(n_valid, row, ld);
  const int64_t p0 = (int64_t)blockIdx.x * kCollectPiece;
  if (nv <= k || p0 >= nv) return;  // uniform
  const int tid = threadIdx.x;
  // the row's score loads of this piece go out first; the threshold is formed while they fly
  float s[kCollectPer];
  const float* srow = scores + row * ld;
  const bool vec = (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
#pragma unroll
  for (int j = 0; j < kCollectPer / 4; ++j) load4(srow, ld, p0 + (int64_t)(j * kCollectThreads + tid) * 4, vec, s + 4 * j);
  // T0: the lower bound of the bin (one histogram pass over the range of the keys) that holds the
  // k-th largest maximum of the row's groups of gs entries; at most that maximum, so at most the
  // k-th largest score
  const int r = pl.gs / pl.g0;  // stored maxima per group
  const int64_t G = (nv + pl.gs - 1) / pl.gs;
  const int64_t G0 = (nv + pl.g0 - 1) / pl.g0;
  const float* gm = w.gmax + row * pl.gstride;
  auto group_key = [&](int64_t g) -> uint32_t {
    float v = -INFINITY;
    for (int j = 0; j < r; ++j) {
      const int64_t q = g * r + j;
      if (q < G0) v = fmaxf(v, gm[q]);
    }
    return score_to_key(v);
  };
  uint32_t T0 = 0;
  if (G >= k) {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int64_t g = tid; g < G; g += kCollectThreads) {
      const uint32_t v = group_key(g);
      mn = v < mn ? v : mn;
      mx = v > mx ? v : mx;
    }
    block_minmax<kCollectThreads, uint32_t>(mn, mx, red);
    int shv;
    uint32_t above, inbin;
    const uint32_t d = range_pass<kCollectThreads, uint32_t>(G, group_key, mn, mx - mn, (uint32_t)k, shv, above,
                                                             inbin, hist, sh3, sh3 + kCollectThreads / 64);
    T0 = mn + (d << shv);
  }
  // append this piece's entries with a key >= T0: the workgroup's count is added to the row's
  // counter by one atomic, and each thread writes its entries after those of the threads before it
  uint32_t take = 0;
#pragma unroll
  for (int j = 0; j < kCollectPer; ++j) {
    const int64_t i = p0 + (int64_t)((j >> 2) * kCollectThreads + tid) * 4 + (j & 3);
    take |= (i < nv && score_to_key(s[j]) >= T0 ? 1u : 0u) << j;
  }
  const uint32_t mine = (uint32_t)__popc(take);
  uint32_t off = block_excl_scan<kCollectThreads>(mine, sh3);
  if (tid == kCollectThreads - 1) hist[0] = off + mine ? atomicAdd(w.cnt + row, off + mine) : 0u;
  __syncthreads();
  off += hist[0];
  uint64_t* cand = w.cand + row * ld;
#pragma unroll
  for (int j = 0; j < kCollectPer; ++j) {
    if ((take >> j) & 1u) {
      const uint32_t i = (uint32_t)(p0 + (int64_t)((j >> 2) * kCollectThreads + tid) * 4 + (j & 3));
      cand[off++] = ((uint64_t)score_to_key(s[j]) << 32) | (uint32_t)(~i);
    }
  }
}

// LDS of sel_final: candidate keys | bins | (bitmap of selected indices and per-word ranks, or the
// selected keys for the bitonic sort of rows longer than the bitmap) | small scratch
constexpr int kBitmapMax = 262144;  // row length ordered through the bitmap
struct FinalSmem {
  uint64_t keys[kFinalCap];
  uint32_t hist[kBins];
  union {
    struct {
      uint32_t bm[kBitmapMax / 32];
      uint16_t wc[kBitmapMax / 32];
    } b;
    uint64_t sel[kMaxTopK];
  } u;
  uint64_t red[2 * (kFinalThreads / 64)];
  uint32_t sh[kFinalThreads / 64 + 4];
  uint32_t nsel;
};

// The exact top-k among c candidate keys (all distinct; c >= k) given by key_at, written to
// oi / os in index order; entries of a row of nv. mn, mx: the smallest and largest candidate key.
template <class KeyAt>
__device__ void select_candidates(uint32_t c, KeyAt key_at, uint64_t mn, uint64_t mx, int64_t nv, int k,
                                  FinalSmem& sm, int32_t* oi, float* os) {
  const int tid = threadIdx.x;
  // the exact k-th largest key: passes over the range that holds it
  uint64_t lo = mn, span = mx - mn;
  uint32_t krem = (uint32_t)k;
  uint64_t T1;
  while (true) {
    int shv;
    uint32_t above, inbin;
    const uint32_t d = range_pass<kFinalThreads, uint64_t>((int64_t)c, key_at, lo, span, krem, shv, above, inbin,
                                                           sm.hist, sm.sh, sm.sh + kFinalThreads / 64);
    krem -= above;
    lo += (uint64_t)d << shv;
    // keys >= lo are the ones above the range, above the bin, and the whole bin
    if (inbin == krem || shv == 0) {
      T1 = lo;
      break;
    }
    const uint64_t wdt = ((uint64_t)1 << shv) - 1;
    span = span - ((uint64_t)d << shv) < wdt ? span - ((uint64_t)d << shv) : wdt;
  }
  if (nv <= kBitmapMax) {
    // ranks in index order from a bitmap of the selected indices
    const int nw = (int)((nv + 31) / 32);
    for (int i = tid; i < nw; i += kFinalThreads) sm.u.b.bm[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < c; i += kFinalThreads) {
      const uint64_t v = key_at(i);
      if (v >= T1) {
        const uint32_t idx = ~(uint32_t)v;
        atomicOr(&sm.u.b.bm[idx >> 5], 1u << (idx & 31));
      }
    }
    __syncthreads();
    const int wpt = (nw + kFinalThreads - 1) / kFinalThreads;
    const int w0 = tid * wpt, w1 = w0 + wpt < nw ? w0 + wpt : nw;
    uint32_t local_cnt = 0;
    for (int i = w0; i < w1; ++i) local_cnt += __popc(sm.u.b.bm[i]);
    uint32_t run = block_excl_scan<kFinalThreads>(local_cnt, sm.sh);
    for (int i = w0; i < w1; ++i) {
      sm.u.b.wc[i] = (uint16_t)run;
      run += __popc(sm.u.b.bm[i]);
    }
    __syncthreads();
    for (uint32_t i = tid; i < c; i += kFinalThreads) {
      const uint64_t v = key_at(i);
      if (v >= T1) {
        const uint32_t idx = ~(uint32_t)v;
        const uint32_t wd = idx >> 5;
        const uint32_t rank = sm.u.b.wc[wd] + __popc(sm.u.b.bm[wd] & ((1u << (idx & 31)) - 1u));
        if (rank < (uint32_t)k) {
          oi[rank] = (int32_t)idx;
          if (os) os[rank] = key_to_score((uint32_t)(v >> 32));
        }
      }
    }
    return;
  }
  // longer rows: the k selected keys re-keyed as (index, score key) and sorted by a bitonic network
  if (tid == 0) sm.nsel = 0;
  __syncthreads();
  for (uint32_t i = tid; i < c; i += kFinalThreads) {
    const uint64_t v = key_at(i);
    if (v >= T1) {
      const uint32_t slot = atomicAdd(&sm.nsel, 1u);
      if (slot < (uint32_t)k) sm.u.sel[slot] = ((uint64_t)(~(uint32_t)v) << 32) | (v >> 32);
    }
  }
  int P = 1;
  while (P < k) P <<= 1;
  __syncthreads();
  for (int i = k + tid; i < P; i += kFinalThreads) sm.u.sel[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (P >> 1); t += kFinalThreads) {
        const int i = (t / stride) * stride * 2 + (t % stride);
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t a = sm.u.sel[i], b = sm.u.sel[j];
        if ((a > b) == up) {
          sm.u.sel[i] = b;
          sm.u.sel[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < k; j += kFinalThreads) {
    const uint64_t v = sm.u.sel[j];
    oi[j] = (int32_t)(uint32_t)(v >> 32);
    if (os) os[j] = key_to_score((uint32_t)v);
  }
}

// Rows with at most k valid entries keep them all, in order (returns true then).
__device__ __forceinline__ bool keep_all(const float* scores, int64_t ld, int64_t row, int64_t nv, int k,
                                         int32_t* oi, float* os) {
  if (nv > k) return false;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    oi[j] = j < nv ? j : -1;
    if (os) os[j] = j < nv ? key_to_score(score_to_key(scores[row * ld + j])) : -INFINITY;
  }
  return true;
}

__global__ void __launch_bounds__(kFinalThreads) sel_final(const float* scores, int64_t ld, const int32_t* n_valid,
                                                            int k, SelBufs w, int32_t* out_idx, float* out_score) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  FinalSmem& sm = *reinterpret_cast<FinalSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t nv = row_valid(n_valid, row, ld);
  int32_t* oi = out_idx + row * k;
  float* os = out_score ? out_score + row * k : nullptr;
  if (keep_all(scores, ld, row, nv, k, oi, os)) return;
  const uint32_t c = w.cnt[row];  // >= k: at least k entries clear T0
  const uint64_t* gc = w.cand + row * ld;
  const bool local = c <= (uint32_t)kFinalCap;
  uint64_t mn = ~0ull, mx = 0ull;
  for (uint32_t i = tid; i < c; i += kFinalThreads) {
    const uint64_t v = gc[i];
    if (local) sm.keys[i] = v;
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
  }
  block_minmax<kFinalThreads, uint64_t>(mn, mx, sm.red);  // its barrier also publishes the keys
  if (local)
    select_candidates(c, [&](int64_t i) { return sm.keys[i]; }, mn, mx, nv, k, sm, oi, os);
  else
    select_candidates(c, [&](int64_t i) { return gc[i]; }, mn, mx, nv, k, sm, oi, os);
}

// Rows of up to kRowMax scores: one workgroup per row does the whole selection with the row held in
// registers, so nothing is staged in global memory and there is one launch instead of three.
// Thread t holds the four consecutive scores 4(q*kRowThreads + t) .. +3 for q < P/4 (one 16-byte load
// per q, coalesced across the workgroup). The k-th largest 32-bit key is found by radix passes over an
// LDS histogram (12 bits per pass) of the candidate range [lo, lo + span]. The first pass bins only
// the keys at or above a lower bound of the k-th largest: the smallest of the per-thread maxima when
// every thread holds a score and k <= kRowThreads (then kRowThreads distinct scores are at least that
// large), else the row minimum; this keeps most of the row out of the LDS atomics. Selected are the
// keys above the k-th largest plus the lowest-indexed keys equal to it (ties toward the smaller
// index). Ranks in index order come from per-wave ballots and one scan of per-chunk counts, a chunk
// being the 256 consecutive scores one wave holds for one q.
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowMax = 32 * kRowThreads;
constexpr int kRowBins = 4096;
constexpr int kRowChunks = kRowMax / 256;
constexpr int kFillRows = 256;  // one-workgroup selections that fill the chip (one per compute unit)

struct RowSmem {
  uint32_t hist[kRowBins];
  uint32_t chunk[kRowChunks];
  uint32_t wsum[kRowWaves];
  uint32_t wred[3][kRowWaves];
  uint32_t sh[3];
};

// Block-wide exclusive scan of one value per thread over kRowThreads threads.
__device__ __forceinline__ uint32_t row_excl_scan(uint32_t v, uint32_t* wsum) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) off += w < wave ? wsum[w] : 0u;
  __syncthreads();
  return off + incl - v;
}

// Ranks in index order among the row's flagged elements (bit 4q+e of `mask` flags score
// 4(q*kRowThreads + t) + e): base[q] is the rank of this thread's first flagged element of group q,
// and an element's rank adds the flagged bits below it in its group.
template <int P>
__device__ __forceinline__ void row_ranks(uint32_t mask, RowSmem& sm, uint32_t* base) {
  constexpr int NQ = P / 4, NC = NQ * kRowWaves;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    uint32_t tot = 0, mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t b = __ballot((mask >> (4 * q + e)) & 1u);
      tot += (uint32_t)__popcll(b);
      mine += (uint32_t)__popcll(b & lt);
    }
    base[q] = mine;
    if (lane == 0) sm.chunk[q * kRowWaves + wave] = tot;
  }
  __syncthreads();
  if (wave == 0) {  // chunks 2l, 2l+1 per lane: exclusive scan over the NC chunk counts
    const uint32_t c0 = 2 * lane < NC ? sm.chunk[2 * lane] : 0u;
    const uint32_t c1 = 2 * lane + 1 < NC ? sm.chunk[2 * lane + 1] : 0u;
    const uint32_t ex = wave_incl_scan(c0 + c1) - c0 - c1;
    if (2 * lane < NC) sm.chunk[2 * lane] = ex;
    if (2 * lane + 1 < NC) sm.chunk[2 * lane + 1] = ex + c0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NQ; ++q) base[q] += sm.chunk[q * kRowWaves + wave];
  __syncthreads();
}

// A workgroup selects within one piece of a row: piece c of row r is scores r*ld + c*chunk .. (at most
// chunk of them), and its k results go to slots (r*nchunk + c)*k of the outputs. remap (optional)
// turns a position p of the row into the index remap[r*ld + p]; row_nv (optional) is the row's own
// count of valid entries when the scores are candidates of another selection: with at most k of
// them, every entry 0 .. row_nv-1 is selected.
struct RowSel {
  const float* scores;
  int64_t ld, chunk;
  int nchunk;
  const int32_t* n_valid;  // nullable: every score of the row is valid
  int k;
  int32_t* out_idx;
  float* out_score;        // nullable
  const int32_t* remap;    // nullable
  const int32_t* row_nv;   // nullable
  bool cand_pads;          // pad slots get the smallest key (score bits 0xFFFFFFFF), below any score's
};

template <int P, bool VEC>
__global__ void __launch_bounds__(kRowThreads) sel_row(RowSel a) {
  static_assert(P % 4 == 0 && 4 * P <= kRowChunks && P <= 32, "row layout");
  constexpr int NQ = P / 4;
  __shared__ RowSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int k = a.k;
  const int64_t row = blockIdx.x / a.nchunk;
  const int64_t base = (int64_t)(blockIdx.x % a.nchunk) * a.chunk;
  const int64_t nv_row = a.n_valid ? row_valid(a.n_valid, row, a.ld) : a.ld;
  const int64_t piece = a.ld - base < a.chunk ? a.ld - base : a.chunk;
  const int64_t nv = nv_row - base <= 0 ? 0 : (nv_row - base < piece ? nv_row - base : piece);
  const float* s = a.scores + row * a.ld + base;
  int32_t* oi = a.out_idx + (int64_t)blockIdx.x * k;
  float* os = a.out_score ? a.out_score + (int64_t)blockIdx.x * k : nullptr;
  auto index_of = [&](int64_t p) -> int32_t { return a.remap ? a.remap[row * a.ld + p] : (int32_t)p; };
  if (a.row_nv) {
    // candidates of a row with at most k valid entries: all of them, in order. They all lie in the
    // first piece (valid entries are a prefix of the row), whose candidates lead the list with
    // positions equal to their indices.
    const int64_t t = a.row_nv[row] < 0 ? 0 : a.row_nv[row];
    if (t <= k) {
      for (int j = tid; j < k; j += kRowThreads) {
        oi[j] = j < t ? j : -1;
        if (os) os[j] = j < t ? a.scores[row * a.ld + j] : -INFINITY;
      }
      return;
    }
  }
  if (nv <= k) {  // every valid entry is selected
    for (int j = tid; j < k; j += kRowThreads) {
      oi[j] = j < nv ? index_of(base + j) : -1;
      if (os) os[j] = j < nv ? key_to_score(score_to_key(s[j])) : (a.cand_pads ? __uint_as_float(0xFFFFFFFFu) : -INFINITY);
    }
    return;
  }
  const int64_t ld = piece;  // bound of this piece's loads
  uint32_t key[P];
  uint32_t valid = 0;  // bit j: key[j] is a score of the row (index < nv)
  uint32_t tmin = 0xFFFFFFFFu, tmax = 0u;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i = 4 * ((int64_t)q * kRowThreads + tid);
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
      if (i + 4 <= ld) {
        const float4 x = *reinterpret_cast<const float4*>(s + i);
        v[0] = x.x;
        v[1] = x.y;
        v[2] = x.z;
        v[3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < nv) v[e] = s[i + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = i + e < nv;
      const uint32_t kk = score_to_key(v[e]);
      key[4 * q + e] = kk;
      valid |= (ok ? 1u : 0u) << (4 * q + e);
      tmin = ok && kk < tmin ? kk : tmin;
      tmax = ok && kk > tmax ? kk : tmax;
    }
  }
  // block reductions: smallest per-thread maximum (threads holding a score), row maximum, row minimum
  uint32_t r0 = valid ? tmax : 0xFFFFFFFFu, r1 = tmax, r2 = tmin;
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = __shfl_xor(r0, o, 64), b = __shfl_xor(r1, o, 64), c = __shfl_xor(r2, o, 64);
    r0 = a < r0 ? a : r0;
    r1 = b > r1 ? b : r1;
    r2 = c < r2 ? c : r2;
  }
  if (lane == 0) {
    sm.wred[0][wave] = r0;
    sm.wred[1][wave] = r1;
    sm.wred[2][wave] = r2;
  }
  __syncthreads();
  uint32_t bound = 0xFFFFFFFFu, hi = 0u, rmin = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    bound = sm.wred[0][w] < bound ? sm.wred[0][w] : bound;
    hi = sm.wred[1][w] > hi ? sm.wred[1][w] : hi;
    rmin = sm.wred[2][w] < rmin ? sm.wred[2][w] : rmin;
  }
  const bool every_thread = nv > 4 * (int64_t)(kRowThreads - 1);
  uint32_t lo = (every_thread && k <= kRowThreads) ? bound : rmin;
  uint32_t span = hi - lo;
  uint32_t need = (uint32_t)k;
  bool whole;  // true: select every key >= lo; false: keys > lo plus the first `need` keys equal to lo
  for (;;) {
    const int bits = span == 0u ? 0 : 32 - __clz(span);
    const int sh = bits > 12 ? bits - 12 : 0;
#pragma unroll
    for (int b = tid; b < kRowBins; b += kRowThreads) sm.hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const uint32_t u = key[j] - lo;
      if (((valid >> j) & 1u) && key[j] >= lo && u <= span) atomicAdd(&sm.hist[u >> sh], 1u);
    }
    __syncthreads();
    // thread t scans bins 4095-4t .. 4092-4t, i.e. from the top digit down
    constexpr int per = kRowBins / kRowThreads;
    uint32_t c[per], local = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      c[j] = sm.hist[kRowBins - 1 - per * tid - j];
      local += c[j];
    }
    const uint32_t excl = row_excl_scan(local, sm.wsum);
    if (excl < need && need <= excl + local) {
      uint32_t run = excl;
#pragma unroll
      for (int j = 0; j < per; ++j) {
        if (run < need && need <= run + c[j]) {
          sm.sh[0] = (uint32_t)(kRowBins - 1 - per * tid - j);
          sm.sh[1] = run;
          sm.sh[2] = c[j];
        }
        run += c[j];
      }
    }
    __syncthreads();
    const uint32_t d = sm.sh[0], above = sm.sh[1], inbin = sm.sh[2];
    __syncthreads();
    need -= above;
    lo += d << sh;
    if (inbin == need) {
      whole = true;
      break;
    }
    if (sh == 0) {  // the bin is the single key value lo
      whole = false;
      break;
    }
    const uint32_t w = (1u << sh) - 1u;
    span = span - (d << sh) < w ? span - (d << sh) : w;
  }
  uint32_t sel = 0;
  if (whole) {
#pragma unroll
    for (int j = 0; j < P; ++j) sel |= (((valid >> j) & 1u) && key[j] >= lo ? 1u : 0u) << j;
  } else {
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      sel |= (((valid >> j) & 1u) && key[j] > lo ? 1u : 0u) << j;
      eq |= (((valid >> j) & 1u) && key[j] == lo ? 1u : 0u) << j;
    }
    uint32_t rb[NQ];
    row_ranks<P>(eq, sm, rb);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const uint32_t r = rb[j / 4] + (uint32_t)__popc(eq & (((1u << (j % 4)) - 1u) << (j & ~3)));
      sel |= (((eq >> j) & 1u) && r < need ? 1u : 0u) << j;
    }
  }
  uint32_t pb[NQ];
  row_ranks<P>(sel, sm, pb);
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const uint32_t pos = pb[j / 4] + (uint32_t)__popc(sel & (((1u << (j % 4)) - 1u) << (j & ~3)));
    if (((sel >> j) & 1u) && pos < (uint32_t)k) {  // exactly k are selected; the test only bounds the writes
      oi[pos] = index_of(base + 4 * ((int64_t)(j / 4) * kRowThreads + tid) + (j % 4));
      if (os) os[pos] = key_to_score(key[j]);
    }
  }
}

template <int P>
void launch_row_p(const RowSel& a, int R, hipStream_t s) {
  const bool vec = (a.ld % 4 == 0) && (a.chunk % 4 == 0) && (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0);
  const dim3 grid((unsigned)(R * a.nchunk));
  if (vec) hipLaunchKernelGGL((sel_row<P, true>), grid, dim3(kRowThreads), 0, s, a);
  else hipLaunchKernelGGL((sel_row<P, false>), grid, dim3(kRowThreads), 0, s, a);
}
// pieces of at most kRowMax scores
void launch_row(const RowSel& a, int R, hipStream_t s) {
  const int64_t n = a.chunk;
  if (n <= 4 * kRowThreads) launch_row_p<4>(a, R, s);
  else if (n <= 8 * kRowThreads) launch_row_p<8>(a, R, s);
  else if (n <= 16 * kRowThreads) launch_row_p<16>(a, R, s);
  else launch_row_p<32>(a, R, s);
}

SelBufs carve(void* ws, int R, int64_t ld, int k) {
  const SelPlan pl = select_plan(ld, k);
  uint8_t* p = static_cast<uint8_t*>(ws);
  SelBufs w;
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += a256((size_t)R * 4);
  w.gmax = reinterpret_cast<float*>(p);
  p += a256((size_t)R * pl.gstride * 4);
  w.cand = reinterpret_cast<uint64_t*>(p);
  return w;
}

}  // namespace

// Rows of up to 4 x 32K scores whose pieces' candidates fit one workgroup go in two passes of the
// one-workgroup kernel; longer rows take the group-maximum path.
bool select_two_pass(int64_t ld, int k) {
  return ld <= kRowMax || (ld <= 4 * (int64_t)kRowMax && ceil_div(ld, kRowMax) * k <= kRowMax);
}

bool select_needs_gmax(int64_t ld, int k) { return !select_two_pass(ld, k); }

SelPlan select_plan(int64_t ld, int k) {
  // gs: the largest power of two with ld / gs >= 2k groups (at least 16 entries per group)
  SelPlan pl{};
  int64_t gs = 16;
  while (gs * 2 * 2 * (int64_t)k <= ld) gs *= 2;
  pl.gs = (int)gs;
  pl.g0 = gs < 64 ? (int)gs : 64;
  pl.gstride = (ld + pl.g0 - 1) / pl.g0;
  return pl;
}

size_t select_workspace(int R, int64_t ld, int k) {
  const SelPlan pl = select_plan(ld, k);
  return a256((size_t)R * 4) + a256((size_t)R * pl.gstride * 4) + a256((size_t)R * ld * 8);
}

uint32_t* select_counters(void* ws) { return static_cast<uint32_t*>(ws); }

float* select_gmax(void* ws, int R) { return reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + a256((size_t)R * 4)); }

hipError_t launch_select(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k, int32_t* out_idx,
                         float* out_score, void* ws, bool have_gmax, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const SelPlan pl = select_plan(ld, k);
  const SelBufs w = carve(ws, R, ld, k);
  hipError_t e;
  const int lds = (int)sizeof(FinalSmem);
  if (select_two_pass(ld, k)) {  // one workgroup per row (or per piece of a row), the scores in registers
    RowSel rs{};
    rs.scores = scores;
    rs.ld = ld;
    rs.chunk = ld;
    rs.nchunk = 1;
    rs.n_valid = n_valid;
    rs.k = k;
    rs.out_idx = out_idx;
    rs.out_score = out_score;
    // Rows longer than one workgroup holds, or too few rows to fill the chip: the k best of each of
    // several pieces of a row (at most 32K and, by choice, at least 2k scores each), then the k best
    // of those candidates with positions mapped back to indices. The row's k best are among its
    // pieces' k best, every list is in index order and both passes use the same key order, so the
    // result is the one-pass selection's.
    int64_t pieces = ceil_div(ld, kRowMax);
    if (R < kFillRows) {
      // a launch's cost grows with the scores a workgroup holds, on top of a fixed part, so about
      // sqrt(ld / k) pieces balance the two passes
      const int64_t want = ceil_div(kFillRows, R), most = ld / (2 * (int64_t)k);
      const int64_t bal = (int64_t)ceil(sqrt((double)ld / k));
      int64_t p = want < most ? want : most;
      p = p < bal ? p : bal;
      p = p < kRowMax / k ? p : kRowMax / k;  // the candidates fit one workgroup
      pieces = p > pieces ? p : pieces;
    }
    const int64_t chunk = pieces > 1 ? ceil_div(ceil_div(ld, pieces), 1024) * 1024 : ld;
    const int64_t nchunk = ceil_div(ld, chunk);
    if (nchunk <= 1) {
      launch_row(rs, R, s);
      return hipGetLastError();
    }
    int32_t* cand_idx = reinterpret_cast<int32_t*>(w.cand);
    float* cand_score = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(w.cand) + a256((size_t)R * nchunk * k * 4));
    rs.chunk = chunk;
    rs.nchunk = (int)nchunk;
    rs.out_idx = cand_idx;
    rs.out_score = cand_score;
    rs.cand_pads = true;  // a piece with fewer than k entries pads below every real candidate
    launch_row(rs, R, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    RowSel r2{};
    r2.scores = cand_score;
    r2.ld = nchunk * k;
    r2.chunk = nchunk * k;
    r2.nchunk = 1;
    r2.k = k;
    r2.out_idx = out_idx;
    r2.out_score = out_score;
    r2.remap = cand_idx;
    r2.row_nv = n_valid;
    launch_row(r2, R, s);
    return hipGetLastError();
  }
  if (!have_gmax) {
    int64_t gx = ceil_div(ld, 256 * 4);
    if (gx > 1024) gx = 1024;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(sel_gmax, dim3((unsigned)gx, (unsigned)R), dim3(256), 0, s, scores, ld, n_valid, pl.g0,
                       pl.gstride, w.gmax, w.cnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned pieces = (unsigned)(ceil_div(ld, kCollectPiece) > 0 ? ceil_div(ld, kCollectPiece) : 1);
  hipLaunchKernelGGL(sel_collect, dim3(pieces, (unsigned)R), dim3(kCollectThreads), 0, s, scores, ld, n_valid, k, pl,
                     w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = allow_lds((const void*)sel_final, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_final, dim3((unsigned)R), dim3(kFinalThreads), lds, s, scores, ld, n_valid, k, w, out_idx,
                     out_score);
  return hipGetLastError();
}

}  // namespace csa
