// Step 4: sparse single-KV-head attention over the selected entries plus the raw-token window,
// one softmax over both ("Anatomy of a Frontier Model", "The skeleton, and what's kept": one KV
// head for every query head, the entry is key and value; bullet "A sliding window in every
// layer"; bullet "An attention sink": an extra exp(sink_h) in the denominator).
//
// Paths:
//  * attn_mfma (bf16, D = 512, 64-head groups): one workgroup per (query row, 64-head group); the
//    four waves split the 512 dims into quarters. For each tile of 32 gathered keys a wave loads its
//    quarter of every key straight from HBM/L2 into MFMA B-fragments, computes the partial logits of
//    all 64 heads (QK^T over its 128 dims, q resident in VGPRs), and stores the partials plus a
//    transposed copy of its key quarter (the V operand) in LDS. After a barrier each wave finishes
//    the online softmax of 16 heads (sum of the four partials, running max and sum, P in bf16);
//    after a second barrier each wave accumulates O[64 heads x its 128 dims] += P V with MFMA.
//    Key bytes cross the L2->CU path once per head group; the entry is both K and V.
//  * attn_generic (any H, D, fp32 or bf16): one wave per (row, head), lanes over dims, one key at
//    a time with a wave reduction; used for fp32 layers and odd shapes.
#include "kernels.h"

namespace csa {

namespace {

__device__ __forceinline__ int64_t window_lo(const AttnArgs& a, int64_t p) {
  int64_t lo = p - a.W + 1;
  if (lo < 0) lo = 0;
  if (lo < a.raw_pos0) lo = a.raw_pos0;
  return lo;
}
__device__ __forceinline__ int64_t window_hi(const AttnArgs& a, int64_t p) {
  int64_t hi = p;
  if (hi > a.raw_pos0 + a.raw_len - 1) hi = a.raw_pos0 + a.raw_len - 1;
  return hi;
}

// ---------------------------------------------------------------- generic

constexpr int kGenWaves = 4;

template <int DT, int OT>
__global__ void __launch_bounds__(kGenWaves * 64) attn_generic(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const int64_t p = a.q_pos0 + t;
  const int64_t wlo = window_lo(a, p), whi = window_hi(a, p);
  const int32_t* idx = a.idx + row * a.k;
  constexpr int kMaxPer = 16;  // dims per lane (D <= 1024)
  const int per = (a.D + 63) / 64;
  for (int h = wave; h < a.H; h += kGenWaves) {
    const int64_t qoff = (int64_t)b * a.q_seq_stride + (int64_t)t * a.q_ld + (int64_t)h * a.D;
    float qv[kMaxPer], ov[kMaxPer];
    for (int j = 0; j < kMaxPer; ++j) {
      const int d = lane + 64 * j;
      qv[j] = (j < per && d < a.D) ? load_elem<DT>(a.q, qoff + d) * a.scale : 0.f;
      ov[j] = 0.f;
    }
    float mx = -INFINITY, den = 0.f;
    if (a.sink) {
      mx = a.sink[h];
      den = 1.f;
    }
    const int64_t nsel = a.k;
    const int64_t nwin = whi >= wlo ? whi - wlo + 1 : 0;
    for (int64_t j = 0; j < nsel + nwin; ++j) {
      int64_t off;
      const void* src;
      if (j < nsel) {
        const int32_t e = idx[j];
        if (e < 0 || e >= a.n_cap) continue;
        src = a.entries;
        off = (int64_t)b * a.entries_seq_stride + (int64_t)e * a.D;
      } else {
        src = a.raw;
        off = (int64_t)b * a.raw_seq_stride + (wlo + (j - nsel) - a.raw_pos0) * a.raw_ld;
      }
      float kv[kMaxPer];
      float part = 0.f;
      for (int jj = 0; jj < kMaxPer; ++jj) {
        const int d = lane + 64 * jj;
        kv[jj] = (jj < per && d < a.D) ? load_elem<DT>(src, off + d) : 0.f;
        part = fmaf(qv[jj], kv[jj], part);
      }
      const float l = wave_sum(part);
      const float nm = fmaxf(mx, l);
      const float sc = expf(mx - nm);
      const float pe = expf(l - nm);
      den = den * sc + pe;
      for (int jj = 0; jj < kMaxPer; ++jj) ov[jj] = fmaf(ov[jj], sc, pe * kv[jj]);
      mx = nm;
    }
    const float inv = 1.f / den;
    const int64_t ooff = (row * a.H + h) * (int64_t)a.D;
    for (int j = 0; j < kMaxPer; ++j) {
      const int d = lane + 64 * j;
      if (j < per && d < a.D) store_elem<OT>(a.out, ooff + d, ov[j] * inv);
    }
  }
}

// ---------------------------------------------------------------- MFMA (bf16, D = 512)

constexpr int kHG = 64;                // heads per workgroup
constexpr int kNW = 8;                 // waves per workgroup; each owns 512/kNW dims
constexpr int kDW = 512 / kNW;         // dims per wave (64)
constexpr int kNK = 32;                // keys per tile
constexpr int kVT = 40;                // LDS row stride (bf16) of the transposed key slice and of P
constexpr int kHW = kHG / kNW;         // heads whose softmax a wave finishes (8)
constexpr float kRescaleLog2 = 8.f;    // reference-max slack before O is rescaled
constexpr int kSR = 40;                // row stride (floats) of the partial logits: the two lane halves,
                                       // which write rows 4 apart, land on opposite bank halves

struct AttnSmem {
  float sred[kNW][kHG][kSR];       // partial logits per wave          80 KiB
  uint16_t vt[kNW][kDW][kVT];      // key slices, dim-major            40 KiB
  uint16_t pl[kHG][kVT];           // probabilities, bf16              5 KiB
  float alpha[kHG];                // per-head rescale of O this tile
  float lsum[kHG];                 // per-head running denominators
  float mrun[kHG];                 // per-head running maxima (log2 units)
  int32_t rescale[2];              // some head rescaled O in this tile (by tile parity)
  int32_t keys[1];                 // gathered key list (entry ids >= 0, window rows as -(r+1))
};

// Split-KV bookkeeping: in the decode regime (fewer than 8 query rows per sequence) the key list
// of a row is cut into fixed ranges of split_keys keys, one workgroup each; every workgroup leaves
// (running max in log2 units, running sum, O / sum in bf16) and attn_combine merges the splits in a
// fixed order. The plan depends only on T, k and the window, never on the batch size, so a row's
// result is the same alone or inside any batch.
struct AttnSplit {
  int n_splits, split_keys;
  uint16_t* part_o;  // [R*G*S, 64, 512] bf16, each split's output normalised by its own sum
  float* part_ml;    // [R*G*S, 64, 2]: running max (log2 units), running sum
};

// This wave's slice of one gathered key as B-fragments: key kj, dims wave*64 + s*16 + (lane/32)*8.
__device__ __forceinline__ void load_slice(uint4 (&ku)[kDW / 16], const int32_t* keys, int kj, int kend,
                                           const uint16_t* ent, const uint16_t* raw, int64_t raw_ld, int wave,
                                           int lane) {
  const bool kok = kj < kend;
  const uint16_t* krow = nullptr;
  if (kok) {
    const int32_t id = keys[kj];
    krow = id >= 0 ? ent + (int64_t)id * 512 : raw + (int64_t)(-id - 1) * raw_ld;
  }
#pragma unroll
  for (int s = 0; s < kDW / 16; ++s)
    ku[s] = kok ? *reinterpret_cast<const uint4*>(krow + wave * kDW + s * 16 + (lane >> 5) * 8) : make_uint4(0, 0, 0, 0);
}

template <int OT>
__global__ void __launch_bounds__(kNW * 64) attn_mfma(AttnArgs a, int n_groups, AttnSplit sp) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int split = (int)(blockIdx.x % sp.n_splits);
  const int64_t rg = blockIdx.x / sp.n_splits;
  const int64_t row = rg / n_groups;
  const int hg = (int)(rg % n_groups);
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const int64_t p = a.q_pos0 + t;
  const int64_t wlo = window_lo(a, p), whi = window_hi(a, p);

  // ---- key list: valid selected entries, then the window rows
  if (wave == 0) {
    int nsel = 0;
    const int32_t* idx = a.idx + row * a.k;
    for (int base = 0; base < a.k; base += 64) {
      const int j = base + lane;
      const int32_t e = j < a.k ? idx[j] : -1;
      const bool ok = e >= 0 && e < a.n_cap;
      const uint64_t bm = __ballot(ok);
      if (ok) sm.keys[nsel + __popcll(bm & lanemask_lt())] = e;
      nsel += __popcll(bm);
    }
    const int nwin = whi >= wlo ? (int)(whi - wlo + 1) : 0;
    for (int j = lane; j < nwin; j += 64) sm.keys[nsel + j] = -(int32_t)(wlo - a.raw_pos0 + j) - 1;
    if (lane == 0) {
      sm.keys[a.k + a.W] = nsel + nwin;
      sm.rescale[0] = 0;
    }
  }
  __syncthreads();
  const int nkeys = sm.keys[a.k + a.W];
  const int kbeg = split * sp.split_keys;
  const int kend = kbeg + sp.split_keys < nkeys ? kbeg + sp.split_keys : nkeys;

  // ---- q slice as A-fragments: head hg*64 + mt*32 + lane%32, dims wave*64 + s*16 + (lane/32)*8
  const float scale = a.scale * 1.4426950408889634f;  // logits in log2 units
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)t * a.q_ld +
                         (int64_t)hg * kHG * 512 + wave * kDW;
  bf16x8 qf[2][kDW / 16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < kDW / 16; ++s)
      qf[mt][s] = *reinterpret_cast<const bf16x8*>(qrow + (int64_t)(mt * 32 + (lane & 31)) * 512 + s * 16 + (lane >> 5) * 8);

  f32x16 o[2][kDW / 32];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < kDW / 32; ++nt) o[mt][nt] = f32x16{};

  // softmax ownership: wave w finishes heads w*8 + lane/8, keys (lane%8)*4 .. +3
  const int sh = wave * kHW + (lane >> 3);
  const int sk0 = (lane & 7) * 4;
  float m_run = -INFINITY, l_run = 0.f;
  if (a.sink && sp.n_splits == 1) {
    m_run = a.sink[hg * kHG + sh] * 1.4426950408889634f;
    l_run = 1.f;
  }

  const uint16_t* ent = static_cast<const uint16_t*>(a.entries) + (int64_t)b * a.entries_seq_stride;
  const uint16_t* raw = static_cast<const uint16_t*>(a.raw) + (int64_t)b * a.raw_seq_stride;
  const int ntiles = kend > kbeg ? (kend - kbeg + kNK - 1) / kNK : 0;
  // Gathered key slices cycle through three register sets: the loads of tile i+3 are issued as soon
  // as tile i has been consumed, so three tiles of HBM/L2 latency are in flight behind the math.
  uint4 kbuf[3][kDW / 16];
  auto tile_step = [&](uint4 (&ku)[kDW / 16], const int tile) {
    const int k0 = kbeg + tile * kNK;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < kDW / 16; ++s) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, ku[s]);
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], kf, sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], kf, sacc[1], 0, 0, 0);
    }
    // partial logits -> LDS: head mt*32 + (r/4)*8 + (lane/32)*4 + r%4, key lane%32
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sm.sred[wave][mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)][lane & 31] = sacc[mt][r];
    // key slice, transposed: vt[dim][key]
#pragma unroll
    for (int s = 0; s < kDW / 16; ++s) {
      const uint32_t w4[4] = {ku[s].x, ku[s].y, ku[s].z, ku[s].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sm.vt[wave][s * 16 + (lane >> 5) * 8 + j][lane & 31] = (uint16_t)(w4[j >> 1] >> ((j & 1) * 16));
    }
    // this register set is free again: start gathering the tile three ahead into it
    if (tile + 3 < ntiles) load_slice(ku, sm.keys, k0 + 3 * kNK + (lane & 31), kend, ent, raw, a.raw_ld, wave, lane);
    __syncthreads();

    // ---- online softmax of kHW heads x 32 keys per wave
    {
      float sv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = sk0 + j;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) v += sm.sred[w][sh][key];
        v = (k0 + key < kend) ? v * scale : -INFINITY;
        sv[j] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4, 64));
      // lazy rescaling: the reference max moves only when a logit exceeds it by more than 2^8, so
      // weights stay below 256 and O is rescaled in few tiles
      const float m_new = tmax > m_run + kRescaleLog2 ? tmax : m_run;
      const float al = m_new == m_run ? 1.f : exp2f(m_run - m_new);
      float psum = 0.f;
      uint16_t pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t h16 = f2bf(exp2f(sv[j] - m_new));
        pb[j] = h16;
        psum += bf2f(h16);  // the denominator sums the same rounded weights P V uses
      }
      psum += __shfl_xor(psum, 1, 64);
      psum += __shfl_xor(psum, 2, 64);
      psum += __shfl_xor(psum, 4, 64);
      l_run = l_run * al + psum;
      m_run = m_new;
      *reinterpret_cast<uint2*>(&sm.pl[sh][sk0]) =
          make_uint2(pb[0] | ((uint32_t)pb[1] << 16), pb[2] | ((uint32_t)pb[3] << 16));
      if ((lane & 7) == 0) {
        sm.alpha[sh] = al;
        sm.lsum[sh] = l_run;
        sm.mrun[sh] = m_run;
      }
      // the flag of this tile's parity was cleared a tile ago; clear the other one for the next tile
      if (al != 1.f) sm.rescale[tile & 1] = 1;
      if (threadIdx.x == 0) sm.rescale[(tile + 1) & 1] = 0;
    }
    __syncthreads();

    // ---- O = alpha * O + P V over this wave's dims
    if (sm.rescale[tile & 1]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float al = sm.alpha[mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)];
#pragma unroll
          for (int nt = 0; nt < kDW / 32; ++nt) o[mt][nt][r] *= al;
        }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pf[ks] = *reinterpret_cast<const bf16x8*>(&sm.pl[mt * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int nt = 0; nt < kDW / 32; ++nt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sm.vt[wave][nt * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
          o[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[ks], vf, o[mt][nt], 0, 0, 0);
        }
      }
    }
    };
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < ntiles) load_slice(kbuf[j], sm.keys, kbeg + j * kNK + (lane & 31), kend, ent, raw, a.raw_ld, wave, lane);
  for (int tile = 0; tile < ntiles; tile += 3) {
    tile_step(kbuf[0], tile);
    if (tile + 1 < ntiles) tile_step(kbuf[1], tile + 1);
    if (tile + 2 < ntiles) tile_step(kbuf[2], tile + 2);
  }
  if (ntiles == 0 && (lane & 7) == 0) {
    sm.lsum[sh] = l_run;
    sm.mrun[sh] = m_run;
  }
  __syncthreads();
  if (sp.n_splits == 1) {
    // ---- normalise and store: head hg*64 + row index, dim wave*64 + nt*32 + lane%32
    const int64_t obase = (row * a.H + (int64_t)hg * kHG) * 512 + wave * kDW;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const float inv = 1.f / sm.lsum[h];
#pragma unroll
        for (int nt = 0; nt < kDW / 32; ++nt)
          store_elem<OT>(a.out, obase + (int64_t)h * 512 + nt * 32 + (lane & 31), o[mt][nt][r] * inv);
      }
  } else {
    // ---- this split's partial for attn_combine: O / l in bf16, (m, l) in fp32
    const int64_t pidx = rg * sp.n_splits + split;
    uint16_t* po = sp.part_o + pidx * (kHG * 512) + wave * kDW;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const float l = sm.lsum[h];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int nt = 0; nt < kDW / 32; ++nt) po[h * 512 + nt * 32 + (lane & 31)] = f2bf(o[mt][nt][r] * inv);
      }
    if (threadIdx.x < kHG) {
      sp.part_ml[(pidx * kHG + threadIdx.x) * 2] = sm.mrun[threadIdx.x];
      sp.part_ml[(pidx * kHG + threadIdx.x) * 2 + 1] = sm.lsum[threadIdx.x];
    }
  }
}

// Merges the n_splits partials of every (row, head): M = max m_s, L = sum l_s 2^(m_s - M) (plus the
// sink), O = sum l_s 2^(m_s - M) (O_s / l_s) / L, splits taken in order. One workgroup per
// (row, 4 heads).
template <int OT>
__global__ void __launch_bounds__(256) attn_combine(AttnArgs a, int n_groups, AttnSplit sp) {
  const int64_t R = (int64_t)a.B * a.T;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head)
  if (gid >= R * a.H) return;
  const int64_t row = gid / a.H;
  const int h = (int)(gid % a.H);
  const int hg = h / kHG, hl = h % kHG;
  const int64_t rg = row * n_groups + hg;
  const int lane = lane_id();
  float M = -INFINITY;
  for (int s = 0; s < sp.n_splits; ++s) {
    const float* ml = sp.part_ml + ((rg * sp.n_splits + s) * kHG + hl) * 2;
    if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
  }
  float sink2 = -INFINITY;
  if (a.sink) {
    sink2 = a.sink[h] * 1.4426950408889634f;
    M = fmaxf(M, sink2);
  }
  float L = a.sink ? exp2f(sink2 - M) : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < sp.n_splits; ++s) {
    const int64_t pidx = rg * sp.n_splits + s;
    const float* ml = sp.part_ml + (pidx * kHG + hl) * 2;
    if (!(ml[1] > 0.f)) continue;
    const float wgt = ml[1] * exp2f(ml[0] - M);
    L += wgt;
    const uint4 u = *reinterpret_cast<const uint4*>(sp.part_o + pidx * (kHG * 512) + hl * 512 + lane * 8);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(__uint_as_float((w4[j >> 1] >> ((j & 1) * 16)) << 16), wgt, acc[j]);
  }
  const float inv = 1.f / L;
  const int64_t ob = (row * a.H + h) * 512 + lane * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) store_elem<OT>(a.out, ob + j, acc[j] * inv);
}

int attn_mfma_lds(const AttnArgs& a) { return (int)(sizeof(AttnSmem) + (size_t)(a.k + a.W + 1) * 4); }

bool use_attn_mfma(const AttnArgs& a) {
  return a.in_dtype == CSA_BF16 && a.D == 512 && a.H % kHG == 0 && a.raw_ld % 8 == 0 && a.q_ld % 8 == 0 &&
         a.q_seq_stride % 8 == 0 && a.entries_seq_stride % 8 == 0 && a.raw_seq_stride % 8 == 0;
}


constexpr int kDecodeRows = 8;     // fewer query rows per sequence than this: decode regime
constexpr int kSplitKeys = 256;    // keys per split in the decode regime

AttnSplit plan_split(const AttnArgs& a) {
  AttnSplit sp{1, a.k + a.W, nullptr, nullptr};
  if (!use_attn_mfma(a) || a.T >= kDecodeRows) return sp;
  const int maxkeys = a.k + a.W;
  const int S = (int)ceil_div(maxkeys, kSplitKeys);
  if (S <= 1) return sp;
  sp.n_splits = S;
  sp.split_keys = kSplitKeys;
  return sp;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t attn_workspace(const AttnArgs& a) {
  const AttnSplit sp = plan_split(a);
  if (sp.n_splits <= 1) return 0;
  const int64_t parts = (int64_t)a.B * a.T * (a.H / kHG) * sp.n_splits;
  return align256((size_t)parts * kHG * 512 * 2) + align256((size_t)parts * kHG * 2 * 4);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.T;
  if (R == 0) return hipSuccess;
  hipError_t e;
  if (use_attn_mfma(a)) {
    const int ng = a.H / kHG;
    const int lds = attn_mfma_lds(a);
    AttnSplit sp = plan_split(a);
    if (sp.n_splits > 1) {
      if (ws == nullptr || ws_bytes < attn_workspace(a)) return hipErrorInvalidValue;
      const int64_t parts = R * ng * sp.n_splits;
      sp.part_o = static_cast<uint16_t*>(ws);
      sp.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256((size_t)parts * kHG * 512 * 2));
    }
    const dim3 grid((unsigned)(R * ng * sp.n_splits));
    if (a.out_dtype == CSA_BF16) {
      if ((e = allow_lds((const void*)attn_mfma<CSA_BF16>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(attn_mfma<CSA_BF16>, grid, dim3(kNW * 64), lds, s, a, ng, sp);
    } else {
      if ((e = allow_lds((const void*)attn_mfma<CSA_F32>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(attn_mfma<CSA_F32>, grid, dim3(kNW * 64), lds, s, a, ng, sp);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (sp.n_splits > 1) {
      const dim3 cg((unsigned)ceil_div(R * a.H, 4));
      if (a.out_dtype == CSA_BF16)
        hipLaunchKernelGGL(attn_combine<CSA_BF16>, cg, dim3(256), 0, s, a, ng, sp);
      else
        hipLaunchKernelGGL(attn_combine<CSA_F32>, cg, dim3(256), 0, s, a, ng, sp);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  const dim3 grid((unsigned)R), block(kGenWaves * 64);
  if (a.in_dtype == CSA_F32 && a.out_dtype == CSA_F32)
    hipLaunchKernelGGL((attn_generic<CSA_F32, CSA_F32>), grid, block, 0, s, a);
  else if (a.in_dtype == CSA_F32)
    hipLaunchKernelGGL((attn_generic<CSA_F32, CSA_BF16>), grid, block, 0, s, a);
  else if (a.out_dtype == CSA_F32)
    hipLaunchKernelGGL((attn_generic<CSA_BF16, CSA_F32>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn_generic<CSA_BF16, CSA_BF16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
