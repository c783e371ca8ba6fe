// Exact top-k over materialised score rows: one workgroup per row for rows that fit its registers
// (sel_row), many workgroups per row for longer rows (see select_radix.h).
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
      if (os) os[j] = j < nv ? key_to_score(score_to_key(s[j])) : -INFINITY;
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
                         float* out_score, void* ws, bool zeroed, hipStream_t s, int64_t max_valid) {
  RowSel rs{};
  rs.k = k;
  // the part of a row that can hold valid scores (n_valid never exceeds max_valid when it is given)
  const int64_t span = max_valid >= 0 && max_valid < ld ? max_valid : ld;
  if (span <= kRowMax) {
    rs.scores = scores;
    rs.ld = ld;
    rs.chunk = span;
    rs.nchunk = 1;
    rs.n_valid = n_valid;
    rs.out_idx = out_idx;
    rs.out_score = out_score;
    launch_row(rs, R, s);
    return hipGetLastError();
  }
  // Longer rows, while the candidates fit one workgroup: the k best of every piece
  // (the row's k best are among them; each piece's list is in index order, so the concatenation
  // is too), then the k best of those candidates with positions mapped back to indices. Both
  // passes use the same key order, so the result is the direct selection's.
  // pieces of 16K scores when their candidates fit (more workgroups, shorter ones: measured faster
  // than 32K or 8K pieces for 1M-token rows), else 32K
  const int64_t piece = ceil_div(span, kRowMax / 2) * k <= kRowMax ? kRowMax / 2 : kRowMax;
  const int64_t nchunk = ceil_div(span, piece);
  if (nchunk * k <= kRowMax && (size_t)R * nchunk * k * 8 + 256 <= select_workspace(R, ld, k)) {
    int32_t* cand_idx = static_cast<int32_t*>(ws);
    float* cand_score = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + a256((size_t)R * nchunk * k * 4));
    rs.scores = scores;
    rs.ld = ld;
    rs.chunk = piece;
    rs.nchunk = (int)nchunk;
    rs.n_valid = n_valid;
    rs.out_idx = cand_idx;
    rs.out_score = cand_score;
    launch_row(rs, R, s);
    hipError_t e;
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
