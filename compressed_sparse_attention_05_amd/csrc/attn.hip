// Step 4: sparse single-KV-head attention over the selected entries plus the raw-token window,
// one softmax over both ("Anatomy of a Frontier Model", "The skeleton, and what's kept": one KV
// head for every query head, the entry is key and value; bullet "A sliding window in every
// layer"; bullet "An attention sink": an extra exp(sink_h) in the denominator).
//
// Paths:
//  * attn_pairs (bf16, D = 512, 128 heads, 8 waves): one workgroup per (query row, key split);
//    wave pairs own 32 heads and split the 512 dims in halves, meet through LDS for the logits, and
//    run as two groups half a tile apart so that softmax and MFMA work of a SIMD overlap.
//  * attn_mfma (bf16, D = 512, 64-head groups of 4 waves): each wave owns 16 heads whole; used for
//    64-head layers.
//  * attn_generic (any H, D, fp32 or bf16): one wave per (row, head), lanes over dims, one key at
//    a time with a wave reduction; used for fp32 layers and odd shapes.
// With fewer than 8 query rows per sequence the key list is cut into fixed splits and
// attn_combine merges the partial results.
#include "kernels.h"
#include "rope.h"

namespace csa {

namespace {

// The window [max(0, p - W + 1), p], cut to the raw rows the caller holds: positions rp .. rp +
// raw_len - 1 (rp = raw_pos[b]); for a ring only the last raw_ring positions up to p.
__device__ __forceinline__ int64_t window_lo(const AttnArgs& a, int64_t p, int64_t rp) {
  int64_t lo = p - a.W + 1;
  if (lo < 0) lo = 0;
  if (lo < rp) lo = rp;
  if (a.raw_ring > 0 && lo < p - a.raw_ring + 1) lo = p - a.raw_ring + 1;
  return lo;
}
__device__ __forceinline__ int64_t window_hi(const AttnArgs& a, int64_t p, int64_t rp) {
  int64_t hi = p;
  if (hi > rp + a.raw_len - 1) hi = rp + a.raw_len - 1;
  return hi;
}
// row of kv_raw holding raw position u: u - rp, or u mod raw_ring for a ring buffer
__device__ __forceinline__ int64_t raw_row(const AttnArgs& a, int64_t u, int64_t rp) {
  return a.raw_ring > 0 ? u % a.raw_ring : u - rp;
}
// dense mode: the entries visible to position p, min(floor((p+1)/m), n_cap)
__host__ __device__ __forceinline__ int64_t dense_visible(const AttnArgs& a, int64_t p) {
  const int64_t n = (p + 1) / a.m;
  return n < a.n_cap ? n : a.n_cap;
}

// ---------------------------------------------------------------- generic

constexpr int kEntryBytes = 584;  // FP8 entry record: 448 e4m3 codes | 64 bf16 | 7 UE8M0 scales | pad

// Element d of a 584-byte entry record: dims < 448 are e4m3 codes (OCP E4M3: bias 7, subnormals
// 2^-6 m/8) times 2^(E-127) of their 64-dim group; dims 448..511 are stored bf16.
__device__ __forceinline__ float record_elem(const uint8_t* rec, int d) {
  if (d >= 448) {
    const uint16_t h = *reinterpret_cast<const uint16_t*>(rec + 448 + 2 * (d - 448));
    return __uint_as_float((uint32_t)h << 16);
  }
  const uint32_t c = rec[d], e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  const float v = ldexpf(mag, (int)rec[576 + (d >> 6)] - 127);
  return (c & 0x80u) ? -v : v;
}

constexpr int kGenWaves = 4;

template <int DT, int OT>
__global__ void __launch_bounds__(kGenWaves * 64) attn_generic(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const int64_t p = pos_at(a.q_pos, b) + t, rp = raw_at(a.raw_pos, b) + a.raw_off;
  const int64_t wlo = window_lo(a, p, rp), whi = window_hi(a, p, rp);
  const int32_t* idx = a.dense ? nullptr : a.idx + row * a.k;
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
    const int64_t nsel = a.dense ? dense_visible(a, p) : a.k;
    const int64_t nwin = whi >= wlo ? whi - wlo + 1 : 0;
    for (int64_t j = 0; j < nsel + nwin; ++j) {
      int64_t off;
      const void* src;
      bool record = false;
      if (j < nsel) {
        const int32_t e = a.dense ? (int32_t)j : idx[j];
        if (e < 0 || e >= a.n_cap) continue;
        src = a.entries;
        record = a.entry_fmt != 0;
        off = (int64_t)b * a.entries_seq_stride + (int64_t)e * (record ? kEntryBytes : a.D);
      } else {
        src = a.raw;
        off = (int64_t)b * a.raw_seq_stride + raw_row(a, wlo + (j - nsel), rp) * a.raw_ld;
      }
      float kv[kMaxPer];
      float part = 0.f;
      for (int jj = 0; jj < kMaxPer; ++jj) {
        const int d = lane + 64 * jj;
        if (record)
          kv[jj] = (jj < per && d < a.D) ? record_elem(static_cast<const uint8_t*>(src) + off, d) : 0.f;
        else
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

constexpr int kHPW = 16;              // query heads per wave
constexpr int kNK = 32;               // keys per tile
constexpr int kKNS = 536;             // LDS row stride (bf16) of a key row, 1072 B: 16 consecutive
                                      // rows start in 16 distinct 16-byte bank groups, and 4
                                      // consecutive rows keep 32-byte reads apart
constexpr float kRescaleLog2 = 8.f;   // reference-max slack before O is rescaled

// output staging row of the 16-head kernel: 512 bf16 plus 16 bytes, so that the 16 rows of a
// wave start on different banks
constexpr int kOutStageRowM = 1040;

// RING key tiles in LDS: the one read and RING - 1 being loaded
template <int RING>
struct AttnSmem {
  uint16_t kn[RING][kNK][kKNS];     // RING x 34304 B
  int32_t wcnt[16];                 // per-wave counts while the key list is compacted
  int32_t keys[1];                  // gathered key list (entry ids >= 0, window rows as -(r+1))
};

// Split-KV bookkeeping: with fewer than 8 query rows per sequence the key list of a row is cut into
// fixed ranges of split_keys keys, one workgroup each; every workgroup leaves (running max in log2
// units, running sum, O / sum in bf16) and attn_combine merges the splits in a fixed order. The plan
// depends only on T, k and the window, never on the batch size, so a row's result is the same alone
// or inside any batch.
struct AttnSplit {
  int n_splits, split_keys;
  uint16_t* part_o;  // [R*S, H, 512] bf16, each split's output normalised by its own sum
  float* part_ml;    // [R*S, H, 2]: running max (log2 units), running sum
};

// Cross-lane reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap permutes, which stay on the VALU.
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One workgroup per (query row, split, group of 16 * NW heads); each wave owns 16 heads whole, so
// logits, softmax and O of a head never leave its wave:
//   S^T[32 keys x 16 heads] = K[32 x 512] Q_w^T   (v_mfma_f32_16x16x32_bf16, K rows from LDS, Q in
//                                                   VGPRs)
//   online softmax over the keys of each head: lane l holds head l%16 and keys 4g .. 4g+3,
//   16+4g .. 16+4g+3 (g = l/16), two cross-lane steps
//   O_w^T[512 x 16] += V^T[512 x 32] P^T          (V^T read from the same key rows with the
//                                                   transposing ds_read_b64_tr_b16, P^T in VGPRs)
// Key rows are gathered by direct global-to-LDS loads (one 1 KiB row per instruction) into a
// RING-deep ring, RING - 1 tiles ahead of the math; one barrier per tile. With fewer than 8 waves
// the ring is two deep so that two workgroups share a compute unit and fill each other's stalls.
template <int NW, int RING, int OT>
__global__ void __launch_bounds__(NW * 64, 2) attn_mfma(AttnArgs a, AttnSplit sp) {
  static_assert(RING == 2 || RING == 3, "one or two tiles in flight");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  AttnSmem<RING>& sm = *reinterpret_cast<AttnSmem<RING>*>(smem_raw);
  constexpr int kThreads = NW * 64;
  constexpr int kRowsPerWave = kNK / NW;  // key rows one wave loads per tile
  const int wave = threadIdx.x >> 6, lane = lane_id();
  // block -> (row, split, head group of 16*NW heads)
  const int n_hg = a.H / (kHPW * NW);
  const int hg = (int)(blockIdx.x % n_hg);
  const int split = (int)((blockIdx.x / n_hg) % sp.n_splits);
  const int64_t row = blockIdx.x / n_hg / sp.n_splits;
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const int64_t p = pos_at(a.q_pos, b) + t, rp = raw_at(a.raw_pos, b) + a.raw_off;
  const int64_t wlo = window_lo(a, p, rp), whi = window_hi(a, p, rp);

  // ---- Q_w^T as B-fragments: head 16w + lane%16, dims s*32 + (lane/16)*8 .. +7 (issued first, so
  // that their latency overlaps the key list)
  const int head = (hg * NW + wave) * kHPW + (lane & 15);
  const int g = lane >> 4;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)t * a.q_ld +
                         (int64_t)head * 512 + g * 8;
  bf16x8 qf[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 32);

  // ---- key list: valid selected entries, then the window rows. All threads load their indices in
  // one burst (one memory latency, not one per 64 indices) and the waves compact them in order. In
  // dense mode the list is every visible entry in order, then the window: ids follow from the
  // position and nothing is stored.
  const int64_t nvis_d = a.dense ? dense_visible(a, p) : 0;
  auto key_id = [&](int kj) -> int32_t {
    return kj < nvis_d ? kj : -(int32_t)raw_row(a, wlo + (kj - nvis_d), rp) - 1;
  };
  if (!a.dense) {
    const int32_t* idx = a.idx + row * a.k;
    int nsel = 0;
    for (int base = 0; base < a.k; base += 4 * kThreads) {
      int32_t e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = base + r * kThreads + (int)threadIdx.x;
        e[r] = j < a.k ? idx[j] : -1;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (base + r * kThreads >= a.k) break;
        const bool ok = e[r] >= 0 && e[r] < a.n_cap;
        const uint64_t bm = __ballot(ok);
        if (lane == 0) sm.wcnt[wave] = __popcll(bm);
        __syncthreads();
        int off = nsel, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int c = sm.wcnt[w];
          off += w < wave ? c : 0;
          tot += c;
        }
        if (ok) sm.keys[off + __popcll(bm & lanemask_lt())] = e[r];
        nsel += tot;
        __syncthreads();
      }
    }
    const int nwin = whi >= wlo ? (int)(whi - wlo + 1) : 0;
    for (int j = threadIdx.x; j < nwin; j += kThreads) sm.keys[nsel + j] = -(int32_t)raw_row(a, wlo + j, rp) - 1;
    if (threadIdx.x == 0) sm.keys[a.k + a.W] = nsel + nwin;
    __syncthreads();
  }
  const int nkeys = a.dense ? (int)nvis_d + (whi >= wlo ? (int)(whi - wlo + 1) : 0) : sm.keys[a.k + a.W];
  const int kbeg = split * sp.split_keys;
  const int kend = kbeg + sp.split_keys < nkeys ? kbeg + sp.split_keys : nkeys;
  const int ntiles = __builtin_amdgcn_readfirstlane(kend > kbeg ? (kend - kbeg + kNK - 1) / kNK : 0);


  f32x4 o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4{};
  const float scale = a.scale * 1.4426950408889634f;  // logits in log2 units
  float m_run = -INFINITY, l_run = 0.f;
  if (a.sink && sp.n_splits == 1) {
    m_run = a.sink[head] * 1.4426950408889634f;
    l_run = 1.f;
  }

  // ---- key rows: row r of tile `tile` into ring slot `buf`; keys past the split's end repeat its
  // last key (finite values; their logits are masked)
  const uint16_t* ent = static_cast<const uint16_t*>(a.entries) + (int64_t)b * a.entries_seq_stride;
  const uint16_t* raw = static_cast<const uint16_t*>(a.raw) + (int64_t)b * a.raw_seq_stride;
  const uint32_t ring = lds_offset(&sm.kn[0][0][0]);
  auto load_tile = [&](int tile, int buf) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = j * NW + wave;
      int kj = kbeg + tile * kNK + r;
      kj = kj < kend ? kj : kend - 1;
      const int32_t id = __builtin_amdgcn_readfirstlane(a.dense ? key_id(kj) : sm.keys[kj]);
      const uint16_t* krow = id >= 0 ? ent + (int64_t)id * 512 : raw + (int64_t)(-id - 1) * a.raw_ld;
      copy_to_lds16(krow + lane * 8,
                    __builtin_amdgcn_readfirstlane(ring + (uint32_t)((buf * kNK + r) * kKNS * 2)));
    }
  };
  // this wave's copies of every tile but the newest `pending` ones have landed
  auto wait_tiles = [&](bool pending) {
    if constexpr (RING == 3) {
      if (pending) wait_vmcnt<kRowsPerWave>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // q has landed before the loop, so that no wait for it stays in the loop body
  __builtin_amdgcn_s_waitcnt(0);
  if (ntiles > 0) load_tile(0, 0);
  if (RING == 3 && ntiles > 1) load_tile(1, 1);
  wait_tiles(RING == 3 && ntiles > 1);
  __syncthreads();
  // per-lane LDS byte offsets: S^T A-fragments (row lane%16, dims g*8 ..) and the transposing reads
  // of V^T (rows 4g + (lane%16)/4 and 16 + 4g + (lane%16)/4, dims 4*(lane%4) ..)
  const uint32_t qk_off = (uint32_t)(((lane & 15) * kKNS + g * 8) * 2);
  const uint32_t pv_off = (uint32_t)(((4 * g + ((lane & 15) >> 2)) * kKNS + 4 * (lane & 3)) * 2);
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  auto kread = [&](int slot, int i, int sg) {  // K fragment i (key block i/2, k-step 2sg + i%2)
    const uint8_t* kt = reinterpret_cast<const uint8_t*>(&sm.kn[slot][0][0]);
    return *reinterpret_cast<const bf16x8*>(kt + qk_off + (i >> 1) * 16 * kKNS * 2 + (sg * 2 + (i & 1)) * 64);
  };
  auto vread = [&](int slot, int db, int half) {
    const uint32_t vb = ring + (uint32_t)(slot * kNK * kKNS * 2) + pv_off;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(uintptr_t)(vb + (uint32_t)(half * 16 * kKNS * 2 + db * 32)));
  };
  // With the three-deep ring the barrier sits between the softmax and P V: it publishes tile + 1,
  // whose first K fragments are then read while P V runs, so the next S^T starts from registers.
  bf16x8 kf[2][4];
  if constexpr (RING == 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[0][i] = kread(0, i, 0);
  }
  int cur = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int nxt = cur == RING - 1 ? 0 : cur + 1;
    if constexpr (RING == 2) {
      if (tile + 1 < ntiles) load_tile(tile + 1, nxt);
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[0][i] = kread(cur, i, 0);
    }
    // S^T: rows = keys 16kb + lane%16 of the tile, cols = heads. Fragments in groups of 4, the next
    // group read while the current one multiplies.
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) {
      if (sg < 7) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[(sg + 1) & 1][i] = kread(cur, i, sg + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[i >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[sg & 1][i], qf[sg * 2 + (i & 1)], sacc[i >> 1], 0, 0, 0);
      asm volatile("" ::"v"(sacc[0]), "v"(sacc[1]));
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments are read while the softmax runs
    constexpr int VG = 2;  // dim blocks per group
    v4i16 vf[2][VG][2];
#pragma unroll
    for (int i = 0; i < VG; ++i) {
      vf[0][i][0] = vread(cur, i, 0);
      vf[0][i][1] = vread(cur, i, 1);
    }
    // online softmax: this lane holds head `head`, keys 16kb + 4g + r
    const int k0 = kbeg + tile * kNK;
    float v[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = (k0 + kb * 16 + 4 * g + r < kend) ? sacc[kb][r] * scale : -INFINITY;
        v[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = group4_max(tmax);
    // lazy rescaling: the reference max moves only when a logit exceeds it by more than 2^8, so
    // weights stay below 256 and O is rescaled in few tiles
    const float m_new = tmax > m_run + kRescaleLog2 ? tmax : m_run;
    const float al = m_new == m_run ? 1.f : exp2f(m_run - m_new);
    // weights rounded to bf16 by v_cvt_pk_bf16_f32; the denominator sums the same rounded weights
    // that P V uses (v_dot2 with ones)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float psum = 0.f;
    uint32_t pw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bf16x2 pp = {(__bf16)__builtin_amdgcn_exp2f(v[m >> 1][(m & 1) * 2] - m_new),
                         (__bf16)__builtin_amdgcn_exp2f(v[m >> 1][(m & 1) * 2 + 1] - m_new)};
      psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
      pw[m] = __builtin_bit_cast(uint32_t, pp);
    }
    psum = group4_sum(psum);
    l_run = l_run * al + psum;
    m_run = m_new;
    if (__ballot(al != 1.f)) {
#pragma unroll
      for (int db = 0; db < 32; ++db) o[db] *= al;
    }
    // P^T B-fragment: k index j <-> key 4g + j (j < 4) and 16 + 4g + j - 4 (j >= 4)
    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    if constexpr (RING == 3) {
      if (tile + 1 < ntiles) {  // tile + 1 has landed; every wave is past its reads of tile - 1
        wait_tiles(false);
        __syncthreads();
      }
      if (tile + 2 < ntiles) load_tile(tile + 2, nxt == RING - 1 ? 0 : nxt + 1);
    }
    // O^T[dims 16db + lane%16 (rows) x heads] += V^T P^T; each V^T fragment is two transposing
    // reads: lane 16g + i gets dim 16db + i of keys 4g .. 4g+3, then of keys 16+4g .. 16+4g+3
    constexpr int NG = 32 / VG;
#pragma unroll
    for (int dg = 0; dg < NG; ++dg) {
      if (dg < NG - 1) {
#pragma unroll
        for (int i = 0; i < VG; ++i) {
          vf[(dg + 1) & 1][i][0] = vread(cur, (dg + 1) * VG + i, 0);
          vf[(dg + 1) & 1][i][1] = vread(cur, (dg + 1) * VG + i, 1);
        }
      }
      if constexpr (RING == 3) {
        if (dg < 4) kf[0][dg] = kread(nxt, dg, 0);  // first K fragments of tile + 1
      }
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const v4i16 lo = vf[dg & 1][i][0], hi = vf[dg & 1][i][1];
        const bf16x8 af = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dg * VG + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, o[dg * VG + i], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < VG; ++i) asm volatile("" ::"v"(o[dg * VG + i]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (RING == 2) {
      if (tile + 1 < ntiles) wait_tiles(false);  // tile + 1 has landed
      __syncthreads();
    }
    cur = nxt;
  }

  // ---- output: lane holds head `head`, dims db*16 + 4g + r
  const bool part = sp.n_splits > 1;
  if (part || (OT == CSA_BF16 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0)) {
    // bf16 rows go out through LDS: the wave writes its 16 heads x 512 dims into its own staging
    // rows over the ring, then each store instruction writes one whole 1 KiB head row
    static_assert(NW * 16 * kOutStageRowM <= RING * kNK * kKNS * 2, "output staging fits the ring");
    const int64_t pidx = row * sp.n_splits + split;
    const float inv = part ? (l_run > 0.f ? 1.f / l_run : 0.f) : 1.f / l_run;
    uint8_t* stg = reinterpret_cast<uint8_t*>(&sm.kn[0][0][0]) + (size_t)wave * 16 * kOutStageRowM;
    __syncthreads();  // every wave is past its last read of the ring (the condition is uniform)
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const uint32_t w0 = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      *reinterpret_cast<uint2*>(stg + (lane & 15) * kOutStageRowM + (db * 16 + 4 * g) * 2) = make_uint2(w0, w1);
    }
    __syncthreads();  // lanes read what other lanes wrote
    uint16_t* dst = part ? sp.part_o + pidx * a.H * 512 : static_cast<uint16_t*>(a.out) + row * a.H * 512;
    const int head0 = head - (lane & 15);  // first head of this wave
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(stg + i * kOutStageRowM + lane * 16);
      *reinterpret_cast<uint4*>(dst + (int64_t)(head0 + i) * 512 + lane * 8) = v;
    }
    if (part && g == 0) {
      sp.part_ml[(pidx * a.H + head) * 2] = m_run;
      sp.part_ml[(pidx * a.H + head) * 2 + 1] = l_run;
    }
  } else {
    const float inv = 1.f / l_run;
    const int64_t ob = (row * a.H + head) * 512 + 4 * g;
#pragma unroll
    for (int db = 0; db < 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_elem<OT>(a.out, ob + db * 16 + r, o[db][r] * inv);
  }
}

// ---------------------------------------------------------------- MFMA, wave pairs (bf16, D = 512)
//
// One workgroup per (query row, split, group of 16 * NW heads). The waves form pairs; a pair owns
// 32 heads and each of its two waves owns half of the 512 dims, so a wave keeps Q and O of 32 heads
// x 256 dims in registers and every K or V^T fragment it reads from LDS feeds a 32-head MFMA
// (twice the reuse of a 16-head wave; LDS bandwidth is what bounds this loop). Per 32-key tile:
//   S_w^T[32 keys x 32 heads] = K[32 x its 256 dims] Q_w^T   (v_mfma_f32_32x32x16_bf16)
//   the two partial logit tiles meet through LDS; both waves add them (a + b = b + a, so both
//   hold the same logits) and run the same online softmax: lane l holds head l%32 and 16 keys,
//   one v_permlane32_swap per reduction
//   O_w^T[its 256 dims x 32 heads] += V^T P^T                (V^T by the transposing
//                                                             ds_read_b64_tr_b16, P^T in VGPRs)
// The K fragment row of lane l is key pi(l%32), pi = swap of bits 2 and 3, so that the keys of the
// logit accumulator a lane holds are exactly the keys of the P^T fragment it feeds to P V.
// Key rows come by direct global-to-LDS loads into a three-deep ring. Two barriers per tile and
// wave: after the partial logits are written, and after P V (the exchange buffer is free again).
constexpr int kPairRing = 3;

// Row order of a key tile in the pairs kernel's ring: each group of 16 rows is stored transposed as a
// 4 x 4 grid (logical row q at 4(q % 4) + q / 4). With rows 1072 bytes (12 banks mod 64) apart, the 16
// rows a K-fragment read spans cover 16 distinct 4-bank groups, and the 4 rows of a transposing V^T
// read pass (lanes 0-31: rows q .. q + 3, 64 bytes each) land 48 banks apart: both without conflicts
// (in logical order the V^T rows were 12 banks apart and overlapped).
__host__ __device__ constexpr int pair_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

constexpr int kStageRow = 592;  // a staged 584-byte record, rounded up to 16 bytes
size_t attn_keys_lds(const AttnArgs& a);
// byte offset of the record staging rows (FMT 1) in the pairs kernel's dynamic LDS
template <int NW>
__host__ __device__ inline size_t attn_stage_offset(const AttnArgs& a);

template <int NW>
struct PairSmem {
  uint16_t kn[kPairRing][kNK][kKNS];  // 3 x 34304 B
  uint4 sx[NW][4][64];                // partial logits, 4 KiB per wave
  int32_t wcnt[16];
  int32_t keys[1];
};
// output staging after the loop: 32 rows of 256 bf16 per wave, rows 16 bytes apart in bank terms,
// laid over the ring and the exchange buffers (which come first in PairSmem)
constexpr int kOutStageRow = 528;
static_assert(8 * 32 * kOutStageRow <= sizeof(PairSmem<8>::kn) + sizeof(PairSmem<8>::sx), "output staging fits the ring");

// Several splits: the workgroups of a row (its splits and head groups) are grouped on one XCD.
__host__ __device__ inline bool pairs_xcd_grouped(int H, int NW, int n_splits) { return n_splits > 1; }

template <int NW>
__host__ __device__ inline size_t attn_stage_offset(const AttnArgs& a) {
  const size_t keys = a.dense ? 4 : (size_t)(a.k + a.W + 1) * 4;
  return (sizeof(PairSmem<NW>) - sizeof(int32_t) + keys + 15) & ~(size_t)15;
}
// the fused QK-norm / RoPE's LDS follows everything else: the cos / sin table of the row's position
// (rope_dims / 2 pairs), then the query gain gamma_q (512 floats; ones when there is no norm, so
// that the per-value code has no branch)
template <int NW>
__host__ __device__ inline size_t pairs_rope_offset(const AttnArgs& a) {
  const size_t keys = a.dense ? 4 : (size_t)(a.k + a.W + 1) * 4;  // attn_keys_lds
  const size_t end = a.entry_fmt ? attn_stage_offset<NW>(a) + (size_t)kNK * kStageRow : sizeof(PairSmem<NW>) + keys;
  return (end + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t rope_tab_bytes(const AttnArgs& a) {
  return a.fuse_fid && a.rope_dims > 0 ? (size_t)(a.rope_dims / 2) * 8 : 0;
}
template <int NW>
size_t pairs_lds(const AttnArgs& a) {
  const size_t g = a.fuse_fid ? 512 * sizeof(float) : 0;
  return pairs_rope_offset<NW>(a) + rope_tab_bytes(a) + g;
}

template <int NW, int OT, int FMT>
__global__ void __launch_bounds__(NW * 64, 1) attn_pairs(AttnArgs a, AttnSplit sp) {
  static_assert(NW == 2 || NW == 4 || NW == 8, "whole wave pairs, at most 8 waves");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  PairSmem<NW>& sm = *reinterpret_cast<PairSmem<NW>*>(smem_raw);
  constexpr int kThreads = NW * 64;
  constexpr int kRowsPerWave = kNK / NW;
  constexpr int kHeadsPerBlock = 16 * NW;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int n_hg = a.H / kHeadsPerBlock;
  int hg, split;
  int64_t row;
  if (pairs_xcd_grouped(a.H, NW, sp.n_splits)) {
    // the splits and head groups of a row run on one XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so the row's q and its gathered keys are read once into that XCD's L2
    const int64_t j = blockIdx.x >> 3;
    hg = (int)(j % n_hg);
    split = (int)((j / n_hg) % sp.n_splits);
    row = (j / n_hg / sp.n_splits) * 8 + (blockIdx.x & 7);
    if (row >= (int64_t)a.B * a.T) return;  // padding workgroup of the last row group
  } else {
    hg = (int)(blockIdx.x % n_hg);
    split = (int)((blockIdx.x / n_hg) % sp.n_splits);
    row = blockIdx.x / n_hg / sp.n_splits;
  }
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  const int64_t p = pos_at(a.q_pos, b) + t, rp = raw_at(a.raw_pos, b) + a.raw_off;
  const int64_t wlo = window_lo(a, p, rp), whi = window_hi(a, p, rp);

  const int half = wave & 1;                    // dims 256*half .. +255
  const int hl = lane & 31, hh = lane >> 5;     // head within the pair; k half of a fragment
  const int head = hg * kHeadsPerBlock + (wave >> 1) * 32 + hl;

  // fused QK-norm / RoPE: the query gain and the cos / sin of the row's position for every rotated
  // pair go to LDS once per workgroup, in the block that normalises q (after the first tiles'
  // loads are issued, so neither the gain's load nor the angles hold up the gathers); the gain is
  // loaded here, into registers
  const bool rot = a.fuse_fid && a.rope_dims > 0;
  float2* rope_tab = reinterpret_cast<float2*>(smem_raw + pairs_rope_offset<NW>(a));
  float* gam = reinterpret_cast<float*>(smem_raw + pairs_rope_offset<NW>(a) + rope_tab_bytes(a));
  float4 gq4 = make_float4(1.f, 1.f, 1.f, 1.f);
  if (a.fuse_fid && a.gamma_q && threadIdx.x < 128) gq4 = reinterpret_cast<const float4*>(a.gamma_q)[threadIdx.x];

  // ---- Q_w^T B-fragments: lane l holds head `head`, dims 256*half + 16s + 8hh .. +7. They are
  // loaded after the first burst of key indices: loads complete in order, so waiting for the
  // indices does not wait for q as well.
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)t * a.q_ld +
                         (int64_t)head * 512 + 256 * half + 8 * hh;
  bf16x8 qf[16];
  auto load_q = [&]() {
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
  };

  // ---- key list (valid selected entries, then the window rows), compacted in order; in dense
  // mode every visible entry in order, then the window, with ids from the position
  const int64_t nvis_d = a.dense ? dense_visible(a, p) : 0;
  auto key_id = [&](int kj) -> int32_t {
    return kj < nvis_d ? kj : -(int32_t)raw_row(a, wlo + (kj - nvis_d), rp) - 1;
  };
  if (a.dense) load_q();
  else {
    const int32_t* idx = a.idx + row * a.k;
    int nsel = 0;
    if (a.k <= 0) load_q();
    for (int base = 0; base < a.k; base += 4 * kThreads) {
      int32_t e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = base + r * kThreads + (int)threadIdx.x;
        e[r] = j < a.k ? idx[j] : -1;
      }
      if (base == 0) load_q();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (base + r * kThreads >= a.k) break;
        const bool ok = e[r] >= 0 && e[r] < a.n_cap;
        const uint64_t bm = __ballot(ok);
        if (lane == 0) sm.wcnt[wave] = __popcll(bm);
        __syncthreads();
        int off = nsel, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int c = sm.wcnt[w];
          off += w < wave ? c : 0;
          tot += c;
        }
        if (ok) sm.keys[off + __popcll(bm & lanemask_lt())] = e[r];
        nsel += tot;
        __syncthreads();
      }
    }
    const int nwin = whi >= wlo ? (int)(whi - wlo + 1) : 0;
    for (int j = threadIdx.x; j < nwin; j += kThreads) sm.keys[nsel + j] = -(int32_t)raw_row(a, wlo + j, rp) - 1;
    if (threadIdx.x == 0) sm.keys[a.k + a.W] = nsel + nwin;
    __syncthreads();
  }
  const int nkeys = a.dense ? (int)nvis_d + (whi >= wlo ? (int)(whi - wlo + 1) : 0) : sm.keys[a.k + a.W];
  const int kbeg = split * sp.split_keys;
  const int kend = kbeg + sp.split_keys < nkeys ? kbeg + sp.split_keys : nkeys;
  const int ntiles = __builtin_amdgcn_readfirstlane(kend > kbeg ? (kend - kbeg + kNK - 1) / kNK : 0);

  f32x16 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x16{};
  const float scale = a.scale * 1.4426950408889634f;  // logits in log2 units
  float m_run = -INFINITY, l_run = 0.f;
  if (a.sink && sp.n_splits == 1) {
    m_run = a.sink[head] * 1.4426950408889634f;
    l_run = 1.f;
  }

  // entries: bf16 rows of 512 (FMT 0) or 584-byte FP8 records (FMT 1, sequence stride in bytes)
  const uint8_t* ent = static_cast<const uint8_t*>(a.entries) +
                       (FMT ? (int64_t)b * a.entries_seq_stride : (int64_t)b * a.entries_seq_stride * 2);
  const uint16_t* raw = static_cast<const uint16_t*>(a.raw) + (int64_t)b * a.raw_seq_stride;
  const uint32_t ring = lds_offset(&sm.kn[0][0][0]);
  // FMT 1: record rows go by direct loads into this wave's staging rows (a record per row slot of
  // kStageRow bytes: 36 lanes x 16 bytes for codes and bf16 dims, 2 lanes x 4 bytes for the scales
  // and the pad), one tile ahead of the ring, and are converted into the ring slot at the point
  // where the wave waits for its next tile. Window rows always go straight into the ring.
  uint8_t* stage = smem_raw + attn_stage_offset<NW>(a) + (size_t)wave * kRowsPerWave * kStageRow;
  uint32_t stage_mask = 0;  // bit j: row j of this wave's staged tile is a record
  // row r of tile `tile` into ring slot `buf`; keys past the split's end repeat its last key
  // (finite values; their logits are masked). Lane l reads the key id of row l%32 (one LDS round
  // trip per tile), and the rows of this wave are taken from it with readlane. With FMT 1 only the
  // window rows are loaded here, and the count of those loads is returned.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto row_addr = [&](int tile, int32_t& id) -> uint64_t {
    int kl = kbeg + tile * kNK + (lane & 31);
    kl = kl < kend ? kl : kend - 1;
    id = a.dense ? key_id(kl) : sm.keys[kl];
    // row address of row l%32, computed on the vector unit without branches
    return id >= 0 ? (uint64_t)(ent + (int64_t)id * (FMT ? kEntryBytes : 1024))
                   : (uint64_t)(raw + (int64_t)(-id - 1) * a.raw_ld);
  };
  auto readlane64 = [](uint64_t v, int r) -> uint64_t {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), r) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, r);
  };
  auto load_tile = [&](int tile, int buf) -> int {
    int32_t id;
    const uint64_t ra = row_addr(tile, id);
    int n = 0;
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = j * NW + wave_u;
      if (FMT && __builtin_amdgcn_readlane(id, r) >= 0) continue;  // a record: staged separately
      copy_to_lds16(reinterpret_cast<const uint16_t*>(readlane64(ra, r)) + lane * 8,
                    __builtin_amdgcn_readfirstlane(ring + (uint32_t)((buf * kNK + pair_row(r)) * kKNS * 2)));
      ++n;
    }
    return n;
  };
  auto stage_records = [&](int tile) {
    int kl = kbeg + tile * kNK + (lane & 31);
    kl = kl < kend ? kl : kend - 1;
    const int32_t id = a.dense ? key_id(kl) : sm.keys[kl];
    stage_mask = 0;
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = j * NW + wave_u;
      const int32_t idr = __builtin_amdgcn_readlane(id, r);
      if (idr < 0) continue;
      const uint8_t* rec = ent + (int64_t)idr * kEntryBytes;  // scalar address
      const uint32_t dst = lds_offset(stage + j * kStageRow);
      if (lane < 36) copy_to_lds16(rec + 16 * lane, __builtin_amdgcn_readfirstlane(dst));
      if (lane < 2) copy_to_lds4(rec + 576 + 4 * lane, __builtin_amdgcn_readfirstlane(dst + 576));
      stage_mask |= 1u << j;
    }
  };
  // staged records -> bf16 rows of ring slot `buf`. Lane l < 28 turns the 16 e4m3 codes of dims
  // 16l..16l+15 into bf16 with its group's scale 2^(E-127) (exact: 4 significant bits; the
  // conversion instruction was checked against the E4M3 table on this part), lanes 28..35 copy the
  // bf16 dims 448 + 8(l-28)...
  auto convert = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      if (!((stage_mask >> j) & 1u)) continue;  // wave-uniform
      const int r = j * NW + wave_u;
      const uint8_t* srow = stage + j * kStageRow;
      uint8_t* dst = reinterpret_cast<uint8_t*>(&sm.kn[buf][pair_row(r)][0]);
      if (lane < 28) {
        const uint32_t E = srow[576 + (lane >> 2)];  // the scale exponent of this lane's 64-dim group
        const float scale = __uint_as_float(E << 23);
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // 8 codes -> 8 bf16 at a time (fewer live registers)
          const uint2 u = *reinterpret_cast<const uint2*>(srow + 16 * lane + 8 * h);
          const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, scale, false));
          const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, scale, true));
          const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, scale, false));
          const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, scale, true));
          *reinterpret_cast<uint4*>(dst + 32 * lane + 16 * h) = make_uint4(o0, o1, o2, o3);
        }
      } else if (lane < 36) {
        *reinterpret_cast<uint4*>(dst + 896 + 16 * (lane - 28)) = *reinterpret_cast<const uint4*>(srow + 16 * lane);
      }
    }
  };

  // per-lane LDS byte offsets within a ring slot:
  //  K A-fragment s: row pi(l%32), dims 256*half + 16s + 8hh .. +7
  //  V^T A-fragment (dims 32dt .., keys 16ks ..), read r of two: 16-lane group g = l/16, i = l%16
  //  addresses row 16ks + 8(g/2) + 4r + i/4, dims 256*half + 32dt + 16(g%2) + 4(i%4) .. +3
  const int prow = (hl & 0x13) | ((hl & 4) << 1) | ((hl & 8) >> 1);
  const uint32_t qk_off = (uint32_t)((pair_row(prow) * kKNS + 256 * half + 8 * hh) * 2);
  const int g = lane >> 4, gi = lane & 15;
  // (rows in the ring's order: logical row 8(g/2) + 4r + i/4 sits at 4(i/4) + 2(g/2) + r)
  const uint32_t pv_off = (uint32_t)(((4 * (gi >> 2) + 2 * (g >> 1)) * kKNS + 256 * half + 16 * (g & 1) + 4 * (gi & 3)) * 2);
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  auto kread = [&](int slot, int s) {
    const uint8_t* kt = reinterpret_cast<const uint8_t*>(&sm.kn[slot][0][0]);
    return *reinterpret_cast<const bf16x8*>(kt + qk_off + s * 32);
  };
  auto vread = [&](int slot, int dt, int ks) {
    const uint32_t vb = ring + (uint32_t)(slot * kNK * kKNS * 2) + pv_off + (uint32_t)(ks * 16 * kKNS * 2 + dt * 64);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)vb);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(vb + kKNS * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // q has landed before the loop, so that no wait for it stays in the loop body
  __builtin_amdgcn_s_waitcnt(0);
  if (FMT) {
    // tile 0 complete before the loop; tile 1's window rows in flight and its records staged
    if (ntiles > 0) {
      load_tile(0, 0);
      stage_records(0);
      wait_vmcnt<0>();
      convert(0);
    }
    if (ntiles > 1) {
      load_tile(1, 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staging rows have been read
      stage_records(1);
    }
  } else {
    if (ntiles > 0) load_tile(0, 0);
    if (ntiles > 1) load_tile(1, 1);
  }
  // fused QK-norm / RoPE of the query (the values a separate pass would store): the lane's 128 dims
  // of head `head`, the other 128 of its half in lane ^ 32 and the other half in the partner wave
  // meet for the sum of squares (through the exchange buffer, free until the first tile); then
  // x * inv * gamma, the rotation of the pairs past 512 - rope_dims, and rounding to bf16. It runs
  // while the first tiles' gathers are in flight and issues no memory loads of its own. A workgroup
  // turns 128 x 512 values, so the vector work per value is kept short: squares summed two at a
  // time by v_dot2 (bf16 products are exact in fp32) and the rounding by v_cvt_pk_bf16_f32.
  if (a.fuse_fid) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    if (threadIdx.x < 128) reinterpret_cast<float4*>(gam)[threadIdx.x] = gq4;
    if (rot) {
      for (int i = threadIdx.x; i < a.rope_dims / 2; i += kThreads) {
        float c, sn;
        rope_cos_sin((double)p, i, a.rope_dims, a.rope_lt, false, c, sn);
        rope_tab[i] = make_float2(c, sn);
      }
    }
    float inv = 1.f;
    if (a.gamma_q) {
      float ss = 0.f, ss2 = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint4 u = __builtin_bit_cast(uint4, qf[s]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.x), __builtin_bit_cast(bf16x2, u.x), ss, false);
        ss2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.y), __builtin_bit_cast(bf16x2, u.y), ss2, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.z), __builtin_bit_cast(bf16x2, u.z), ss, false);
        ss2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.w), __builtin_bit_cast(bf16x2, u.w), ss2, false);
      }
      ss += ss2;
      ss += __shfl_xor(ss, 32, 64);
      float* xs = reinterpret_cast<float*>(&sm.sx[0][0][0]);
      xs[wave * 64 + lane] = ss;
      __syncthreads();  // also publishes the rotation table and the gain
      ss += xs[(wave ^ 1) * 64 + lane];
      inv = 1.f / sqrtf(ss / 512.f + a.q_eps);
    } else {
      __syncthreads();  // the rotation table is complete
    }
    const int rs = 512 - a.rope_dims;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint4 u = __builtin_bit_cast(uint4, qf[s]);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      const int d0 = 256 * half + 16 * s + 8 * hh;  // dims d0 .. d0 + 7
      // the gain and the angles as whole vectors, read before any is used (one LDS wait)
      const float4 g0 = *reinterpret_cast<const float4*>(gam + d0);
      const float4 g1 = *reinterpret_cast<const float4*>(gam + d0 + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
        y[e] = x * inv * gv[e];
      }
      if (rot && d0 + 8 > rs) {
        float2 cs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = (d0 + 2 * j - rs) >> 1;
          cs[j] = rope_tab[i < 0 ? 0 : i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y0 = y[2 * j], y1 = y[2 * j + 1];
          const bool on = d0 + 2 * j >= rs;
          y[2 * j] = on ? y0 * cs[j].x - y1 * cs[j].y : y0;
          y[2 * j + 1] = on ? y0 * cs[j].y + y1 * cs[j].x : y1;
        }
      }
      uint32_t o4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = pack_bf16x2(y[2 * j], y[2 * j + 1]);
      qf[s] = __builtin_bit_cast(bf16x8, make_uint4(o4[0], o4[1], o4[2], o4[3]));
    }
  }
  if (!FMT) {
    if (ntiles > 1) wait_vmcnt<kRowsPerWave>();
    else wait_vmcnt<0>();
  }
  __syncthreads();

  // Two groups of waves, half a tile apart: group 0 (waves 0-3) runs the logits and the exchange
  // of tile t while group 1 (waves 4-7, the same four SIMDs) runs the softmax and P V of tile t-1,
  // and the other way round, so that every SIMD has MFMA work while one of its waves is in the
  // softmax. Barriers count arrivals, not code positions: between consecutive barriers one group
  // does [logits, exchange write] and the other [exchange read, softmax, P V]. Group 1 opens with
  // one extra barrier and group 0 closes with one, so both pass 2 * ntiles + 1 barriers (numbered
  // from 0 after the prologue). Tile t + 1 is published by barrier 2t + 1 (every wave waits for its
  // own copies of it first); tile t - 1 is read for the last time before barrier 2t, so tile t + 2
  // is copied into its slot after barrier 2t, three barriers before group 0 reads it.
  const int grp = NW == 8 ? (wave >> 2) & 1 : 0;
  // this wave's copies of tile + 1 have landed (those of tile + 2 may still be in flight)
  auto wait_next = [&](int tile) {
    if (tile + 1 < ntiles) {
      if (tile + 2 < ntiles) wait_vmcnt<kRowsPerWave>();
      else wait_vmcnt<0>();
    }
  };
  // FMT 1: tile + 1 is staged (its records, issued before the window rows of tile + 2, and its own
  // window rows): wait for all but this wave's n_next2 newest loads, convert it into its slot, then
  // stage the records of tile + 2 (the staging rows were read by the conversion just before).
  auto next_ready = [&](int tile, int n_next2, int nxt_slot) {
    if (!FMT) {
      wait_next(tile);
      return;
    }
    if (tile + 1 >= ntiles) return;
    wait_vmcnt_upto16(n_next2);
    convert(nxt_slot);
    if (tile + 2 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      stage_records(tile + 2);
    }
  };
  if (grp == 1) __syncthreads();

  int cur = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int nxt = cur == kPairRing - 1 ? 0 : cur + 1;
    const int nxt2 = nxt == kPairRing - 1 ? 0 : nxt + 1;
    // the slot of tile - 1 is free once group 1 has passed its P V of tile - 1
    int n_next2 = 0;  // this wave's loads of tile + 2 issued at its load point (FMT 1: window rows)
    if (grp == 1 && tile + 2 < ntiles) n_next2 = load_tile(tile + 2, nxt2);

    // ---- partial S^T over this wave's 256 dims; fragments read two ahead of the MFMA
    f32x16 sacc = f32x16{};
    bf16x8 kf[4];
    kf[0] = kread(cur, 0);
    kf[1] = kread(cur, 1);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s + 2 < 16) kf[(s + 2) & 3] = kread(cur, s + 2);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s & 3], qf[s], sacc, 0, 0, 0);
      asm volatile("" ::"v"(sacc));
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- exchange: both waves of the pair end with the same logits
    uint4* mine = &sm.sx[wave][0][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mine[i * 64] = make_uint4(__float_as_uint(sacc[4 * i]), __float_as_uint(sacc[4 * i + 1]),
                                __float_as_uint(sacc[4 * i + 2]), __float_as_uint(sacc[4 * i + 3]));
    if (grp == 1) next_ready(tile, n_next2, nxt);
    __syncthreads();
    if (grp == 0 && tile + 2 < ntiles) n_next2 = load_tile(tile + 2, nxt2);
    const uint4* other = &sm.sx[wave ^ 1][0][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = other[i * 64];
      sacc[4 * i] += __uint_as_float(u.x);
      sacc[4 * i + 1] += __uint_as_float(u.y);
      sacc[4 * i + 2] += __uint_as_float(u.z);
      sacc[4 * i + 3] += __uint_as_float(u.w);
    }
    // ---- online softmax: lane l holds head `head` and keys 16(r/8) + 8hh + r%8 of the tile; the
    // max is taken on the raw logits (scale > 0) and the scale goes into the exponent's FMA
    const int k0 = kbeg + tile * kNK;
    if (k0 + kNK > kend) {  // last tile of the split: keys past its end are masked
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + 16 * (r >> 3) + 8 * hh + (r & 7) >= kend) sacc[r] = -INFINITY;
    }
    float tmax = fmaxf(sacc[0], sacc[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) tmax = fmaxf(tmax, fmaxf(sacc[r], sacc[r + 1]));
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale;
    }
    // lazy rescaling: the reference max moves only when a logit exceeds it by more than 2^8
    const float m_new = tmax > m_run + kRescaleLog2 ? tmax : m_run;
    const float al = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    // weights rounded to bf16 by v_cvt_pk_bf16_f32; the denominator sums the same rounded weights
    // that P V uses (v_dot2 with ones)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    bf16x2 pp[8];
    float psum = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * m], scale, -m_new));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * m + 1], scale, -m_new));
      pp[m] = bf16x2{(__bf16)p0, (__bf16)p1};
      psum = __builtin_amdgcn_fdot2_f32_bf16(pp[m], ones, psum, false);
    }
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
      psum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    l_run = l_run * al + psum;
    m_run = m_new;
    if (__ballot(al != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= al;
    }
    // P^T B-fragment of k-step ks: keys 16ks + 8hh + j, j = 0..7
    const bf16x8 pf0 = __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint32_t, pp[0]), __builtin_bit_cast(uint32_t, pp[1]),
                                                         __builtin_bit_cast(uint32_t, pp[2]), __builtin_bit_cast(uint32_t, pp[3])));
    const bf16x8 pf1 = __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint32_t, pp[4]), __builtin_bit_cast(uint32_t, pp[5]),
                                                         __builtin_bit_cast(uint32_t, pp[6]), __builtin_bit_cast(uint32_t, pp[7])));
    // ---- O^T[dims 32dt + .. x heads] += V^T P^T, V^T fragments read one dim tile ahead
    bf16x8 vf[2][2];
    vf[0][0] = vread(cur, 0, 0);
    vf[0][1] = vread(cur, 0, 1);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (dt + 1 < 8) {
        vf[(dt + 1) & 1][0] = vread(cur, dt + 1, 0);
        vf[(dt + 1) & 1][1] = vread(cur, dt + 1, 1);
      }
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt & 1][0], pf0, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt & 1][1], pf1, o[dt], 0, 0, 0);
      asm volatile("" ::"v"(o[dt]));
      __builtin_amdgcn_sched_barrier(0);
    }
    // after this barrier the pair's exchange buffer can be written again
    if (grp == 0) next_ready(tile, n_next2, nxt);
    __syncthreads();
    cur = nxt;
  }
  if (grp == 0) __syncthreads();

  // ---- output: lane holds head `head`, dims 256*half + 32dt + 8(r/4) + 4hh + r%4
  const int dbase = 256 * half + 4 * hh;
  const bool part = sp.n_splits > 1;
  if (rot && !part) {
    // the fused back-rotation by the row's position (split rows turn back in the merge); the rotation
    // is linear, so it is applied before the division by the softmax sum
    const int rs = 512 - a.rope_dims;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (256 * half + 32 * dt + 32 <= rs) continue;  // uniform: no rotated dims in this tile
      float2 cs[8];  // the tile's angles, all read before any is used (one LDS wait)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int i = (dbase + 32 * dt + 8 * (r >> 2) + (r & 3) - rs) >> 1;
        cs[r >> 1] = rope_tab[i < 0 ? 0 : i];
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const bool on = dbase + 32 * dt + 8 * (r >> 2) + (r & 3) >= rs;
        const float y0 = o[dt][r], y1 = o[dt][r + 1], c = cs[r >> 1].x, sn = -cs[r >> 1].y;
        o[dt][r] = on ? y0 * c - y1 * sn : y0;
        o[dt][r + 1] = on ? y0 * sn + y1 * c : y1;
      }
    }
  }
  if (part || (OT == CSA_BF16 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0)) {
    // bf16 rows go out through LDS: the wave writes its 32 heads x 256 dims into its own staging
    // rows, then each store instruction writes two whole 512-byte half rows (16 bytes a lane)
    // instead of 16-byte pieces of 32 rows. Every wave has passed its last read of the ring and the
    // exchange buffers (the last barrier follows the last P V of both groups), so their space is free.
    const int64_t pidx = row * sp.n_splits + split;
    const float inv = part ? (l_run > 0.f ? 1.f / l_run : 0.f) : 1.f / l_run;
    uint8_t* stg = smem_raw + (size_t)wave * 32 * kOutStageRow;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w0 = pack_bf16x2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(stg + hl * kOutStageRow + (32 * dt + 8 * q4 + 4 * hh) * 2) = make_uint2(w0, w1);
      }
    __syncthreads();  // lanes read what other lanes wrote (the condition is uniform over the workgroup)
    uint16_t* dst = part ? sp.part_o + pidx * a.H * 512 : static_cast<uint16_t*>(a.out) + row * a.H * 512;
    const int head0 = head - hl;  // first head of this wave
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hr = 2 * i + (lane >> 5);
      const uint4 v = *reinterpret_cast<const uint4*>(stg + hr * kOutStageRow + (lane & 31) * 16);
      *reinterpret_cast<uint4*>(dst + (int64_t)(head0 + hr) * 512 + 256 * half + (lane & 31) * 8) = v;
    }
    if (part && half == 0 && hh == 0) {
      sp.part_ml[(pidx * a.H + head) * 2] = m_run;
      sp.part_ml[(pidx * a.H + head) * 2 + 1] = l_run;
    }
  } else {
    const float inv = 1.f / l_run;
    const int64_t ob = (row * a.H + head) * 512 + dbase;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) store_elem<OT>(a.out, ob + 32 * dt + 8 * (r >> 2) + (r & 3), o[dt][r] * inv);
  }
}

// Merges the n_splits partials of every (row, head): M = max m_s, L = sum l_s 2^(m_s - M) (plus the
// sink), O = sum l_s 2^(m_s - M) (O_s / l_s) / L, splits taken in order. One wave per (row, head),
// four per workgroup.
template <int OT, int kG>
__global__ void __launch_bounds__(256) attn_combine(AttnArgs a, AttnSplit sp) {
  const int64_t R = (int64_t)a.B * a.T;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head)
  if (gid >= R * a.H) return;
  const int64_t row = gid / a.H;
  const int h = (int)(gid % a.H);
  const int lane = lane_id();
  const int S = sp.n_splits;
  // splits in groups of kG (4, 8 or 16: the smallest that holds all splits, up to 16), every load
  // of a group issued before any is used; the first group is loaded together with the (m, l) pairs,
  // so that up to sixteen splits wait for memory once. A split without keys has l = 0 and a zero
  // partial, so it adds nothing.
  auto load_group = [&](int s0, uint4 (&u)[kG], float (&m)[kG], float (&l)[kG]) {
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int s = s0 + j < S ? s0 + j : S - 1;  // past the last split: its copy, with l = 0
      const int64_t pidx = row * S + s;
      const float2 ml = *reinterpret_cast<const float2*>(sp.part_ml + (pidx * a.H + h) * 2);
      m[j] = ml.x;
      l[j] = s0 + j < S ? ml.y : 0.f;
      u[j] = *reinterpret_cast<const uint4*>(sp.part_o + (pidx * a.H + h) * 512 + lane * 8);
    }
  };
  // the fused back-rotation: the row's position is loaded before the partials and the first 64
  // pairs' angles (lane i: pair i) are formed while the partials are in flight
  const bool rot = a.fuse_fid && a.rope_dims > 0;
  double pq = 0.0;
  if (rot) pq = (double)(pos_at(a.q_pos, row / a.T) + row % a.T);
  uint4 u[kG];
  float m[kG], l[kG];
  load_group(0, u, m, l);
  float rc = 1.f, rsn = 0.f;
  if (rot && lane < a.rope_dims / 2) rope_cos_sin(pq, lane, a.rope_dims, a.rope_lt, true, rc, rsn);
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < kG; ++j)
    if (l[j] > 0.f) M = fmaxf(M, m[j]);
  for (int s = kG; s < S; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(sp.part_ml + ((row * S + s) * a.H + h) * 2);
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float sink2 = -INFINITY;
  if (a.sink) {
    sink2 = a.sink[h] * 1.4426950408889634f;
    M = fmaxf(M, sink2);
  }
  float L = a.sink ? exp2f(sink2 - M) : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kG) {
    if (s0 > 0) load_group(s0, u, m, l);
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      // past the last split l = 0, so the weight is 0 and the zero partial adds nothing
      const float wgt = l[j] > 0.f ? l[j] * exp2f(m[j] - M) : 0.f;
      L += wgt;
      const uint32_t w4[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(__uint_as_float((w4[i >> 1] >> ((i & 1) * 16)) << 16), wgt, acc[i]);
    }
  }
  float inv = 1.f / L;
  const int64_t ob = (row * a.H + h) * 512 + lane * 8;
  if (rot) {
    // the back-rotation by the row's position, on O / L (the division is the one the store would
    // make); lane i of a round holds pair i's angle, the lanes holding rotated dims fetch theirs
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    inv = 1.f;
    const int rs = 512 - a.rope_dims, npair = a.rope_dims / 2;
    for (int i0 = 0; i0 < npair; i0 += 64) {  // uniform
      float c = rc, sn = rsn;
      if (i0 > 0) {
        c = 1.f;
        sn = 0.f;
        if (i0 + lane < npair) rope_cos_sin(pq, i0 + lane, a.rope_dims, a.rope_lt, true, c, sn);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int d = lane * 8 + e;
        const int src = ((d - rs) >> 1) - i0;  // the lane holding this pair's angle
        const float cc = __shfl(c, src & 63, 64), ss = __shfl(sn, src & 63, 64);
        if (d >= rs && src >= 0 && src < 64) {
          const float y0 = acc[e], y1 = acc[e + 1];
          acc[e] = y0 * cc - y1 * ss;
          acc[e + 1] = y0 * ss + y1 * cc;
        }
      }
    }
  }
  if (OT == CSA_BF16 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + ob) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) store_elem<OT>(a.out, ob + j, acc[j] * inv);
  }
}

// LDS of the deepest variant (8 waves, three-deep ring); the 4-wave variant uses a two-deep ring
// so that two workgroups share a compute unit
// LDS of the compacted key list (dense mode stores none)
size_t attn_keys_lds(const AttnArgs& a) { return a.dense ? 4 : (size_t)(a.k + a.W + 1) * 4; }

int attn_mfma_lds(const AttnArgs& a) {
  const size_t deepest = sizeof(AttnSmem<3>) > sizeof(PairSmem<8>) ? sizeof(AttnSmem<3>) : sizeof(PairSmem<8>);
  return (int)(deepest + attn_keys_lds(a));
}

bool use_attn_mfma(const AttnArgs& a) {
  // records: the pairs kernel (8 waves for 128 heads, 4 for 64; staging rows within the LDS) or
  // the generic one
  if (a.entry_fmt && !((a.H == 128 && pairs_lds<8>(a) <= (size_t)kMaxLds) ||
                       (a.H == 64 && pairs_lds<4>(a) <= (size_t)kMaxLds)))
    return false;
  return a.in_dtype == CSA_BF16 && a.D == 512 && (a.H == 64 || a.H == 128) && a.raw_ld % 4 == 0 &&
         a.q_ld % 8 == 0 && a.q_seq_stride % 8 == 0 && a.entries_seq_stride % 4 == 0 && a.raw_seq_stride % 4 == 0 &&
         attn_mfma_lds(a) <= kMaxLds;
}

constexpr int kDecodeRows = 8;     // fewer query rows per sequence than this: decode regime
#ifndef CSA_DECODE_SPLIT_KEYS
#define CSA_DECODE_SPLIT_KEYS 288
#endif
constexpr int kSplitKeys = CSA_DECODE_SPLIT_KEYS;  // keys per split in the decode regime (a multiple of 32)
constexpr int kDenseSplitKeys = 512;  // dense mode (thousands of keys per row): 16 tiles per split

// most keys any query row of the call can have (dense: every entry slot visible; the positions
// live on the device, so the plan takes the capacity)
int64_t attn_max_keys(const AttnArgs& a) {
  if (!a.dense) return (int64_t)a.k + a.W;
  return a.n_cap + a.W;
}

AttnSplit plan_split(const AttnArgs& a) {
  const int64_t maxkeys = attn_max_keys(a);
  AttnSplit sp{1, (int)maxkeys, nullptr, nullptr};
  if (!use_attn_mfma(a) || a.T >= kDecodeRows) return sp;
  int split = a.dense ? kDenseSplitKeys : kSplitKeys;
  if (a.dense && maxkeys / kDenseSplitKeys >= 2) {
    // as many splits as whole 512-key runs, the keys spread evenly over them (rounded up to a
    // tile): 8192 entries + the window make 16 splits of 544 keys rather than 16 of 512 and a
    // 17th of 128, which would start a second round of workgroups at 16 sequences
    const int64_t s0 = maxkeys / kDenseSplitKeys;
    split = (int)(ceil_div(ceil_div(maxkeys, s0), kNK) * kNK);
  }
  const int S = (int)ceil_div(maxkeys, split);
  if (S <= 1) return sp;
  sp.n_splits = S;
  sp.split_keys = split;
  return sp;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int NW, int RING, int OT>
hipError_t launch_mfma(const AttnArgs& a, const AttnSplit& sp, int64_t R, hipStream_t s) {
  const int lds = (int)(sizeof(AttnSmem<RING>) + attn_keys_lds(a));
  hipError_t e;
  if ((e = allow_lds((const void*)attn_mfma<NW, RING, OT>, lds)) != hipSuccess) return e;
  const int64_t n_hg = a.H / (kHPW * NW);
  hipLaunchKernelGGL((attn_mfma<NW, RING, OT>), dim3((unsigned)(R * sp.n_splits * n_hg)), dim3(NW * 64), lds, s, a,
                     sp);
  return hipGetLastError();
}

// Waves per workgroup (16 heads each): a query row's 128 heads share one attn_pairs workgroup (8
// waves, each key row loaded once); 64-head layers use attn_mfma. The choice depends on the layer's
// shape only, never on the batch or the number of rows: the two kernels round differently, and a
// sequence's output must not depend on what else is in the batch. (Dealing a row's 128 heads to
// more workgroups of fewer wave pairs for small-batch decode was measured slower: one pair per
// compute unit leaves two of its four SIMDs idle and nothing hides a pair's own latency chain.)
#ifndef CSA_DECODE_NW
#define CSA_DECODE_NW 8
#endif
int attn_waves(const AttnArgs& a) {
  if (a.H != 128) return 4;
  return a.T < kDecodeRows && !a.dense ? CSA_DECODE_NW : 8;
}

template <int NW, int OT, int FMT>
hipError_t launch_pairs_fmt(const AttnArgs& a, const AttnSplit& sp, int64_t R, hipStream_t s) {
  const int lds = (int)pairs_lds<NW>(a);
  hipError_t e;
  if ((e = allow_lds((const void*)attn_pairs<NW, OT, FMT>, lds)) != hipSuccess) return e;
  const int64_t n_hg = a.H / (16 * NW);
  const int64_t blocks = pairs_xcd_grouped(a.H, NW, sp.n_splits) ? ceil_div(R, 8) * 8 * sp.n_splits * n_hg
                                                                   : R * sp.n_splits * n_hg;
  hipLaunchKernelGGL((attn_pairs<NW, OT, FMT>), dim3((unsigned)blocks), dim3(NW * 64), lds, s, a, sp);
  return hipGetLastError();
}
template <int NW, int OT>
hipError_t launch_pairs(const AttnArgs& a, const AttnSplit& sp, int64_t R, hipStream_t s) {
  return a.entry_fmt ? launch_pairs_fmt<NW, OT, 1>(a, sp, R, s) : launch_pairs_fmt<NW, OT, 0>(a, sp, R, s);
}

template <int OT>
hipError_t launch_mfma_for(const AttnArgs& a, const AttnSplit& sp, int64_t R, hipStream_t s) {
  if (attn_waves(a) == 8) return launch_pairs<8, OT>(a, sp, R, s);
  if (a.H == 128) return launch_pairs<4, OT>(a, sp, R, s);  // decode: two 64-head groups per row
  // 64-head layers over records: the pairs kernel with one wave group (it alone stages and converts
  // records)
  if (a.entry_fmt) return launch_pairs_fmt<4, OT, 1>(a, sp, R, s);
  // Too few workgroups to share compute units: a three-deep ring keeps two gathers in flight per
  // workgroup. Otherwise a two-deep ring lets two workgroups share a compute unit.
  if (R * sp.n_splits * (a.H / (kHPW * 4)) < 256) return launch_mfma<4, 3, OT>(a, sp, R, s);
  return launch_mfma<4, 2, OT>(a, sp, R, s);
}

}  // namespace

bool attn_fuses_fid(const AttnArgs& a) {
  if (!use_attn_mfma(a) || a.rope_dims < 0 || a.rope_dims > 512 || (a.rope_dims & 1)) return false;
  // the launches that run attn_pairs, with the rotation table and the gain inside the LDS
  if (attn_waves(a) == 8) return pairs_lds<8>(a) <= (size_t)kMaxLds;
  if (a.H == 128 || a.entry_fmt) return pairs_lds<4>(a) <= (size_t)kMaxLds;
  return false;
}

size_t attn_workspace(const AttnArgs& a) {
  const AttnSplit sp = plan_split(a);
  if (sp.n_splits <= 1) return 0;
  // a dense plan for fewer keys never has more splits than whole 512-key runs plus one
  const int64_t S = a.dense ? ceil_div(attn_max_keys(a), kDenseSplitKeys) + 1 : sp.n_splits;
  const int64_t parts = (int64_t)a.B * a.T * S;
  return align256((size_t)parts * a.H * 512 * 2) + align256((size_t)parts * a.H * 2 * 4);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.T;
  if (R == 0) return hipSuccess;
  hipError_t e;
  if (use_attn_mfma(a)) {
    AttnSplit sp = plan_split(a);
    if (sp.n_splits > 1) {
      if (ws == nullptr || ws_bytes < attn_workspace(a)) return hipErrorInvalidValue;
      const int64_t parts = R * sp.n_splits;
      sp.part_o = static_cast<uint16_t*>(ws);
      sp.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256((size_t)parts * a.H * 512 * 2));
    }
    e = a.out_dtype == CSA_BF16 ? launch_mfma_for<CSA_BF16>(a, sp, R, s) : launch_mfma_for<CSA_F32>(a, sp, R, s);
    if (e != hipSuccess) return e;
    if (sp.n_splits > 1) {
      const dim3 cg((unsigned)ceil_div(R * a.H, 4));
      const bool bf = a.out_dtype == CSA_BF16;
      if (sp.n_splits <= 4) {
        if (bf) hipLaunchKernelGGL((attn_combine<CSA_BF16, 4>), cg, dim3(256), 0, s, a, sp);
        else hipLaunchKernelGGL((attn_combine<CSA_F32, 4>), cg, dim3(256), 0, s, a, sp);
      } else if (sp.n_splits <= 8) {
        if (bf) hipLaunchKernelGGL((attn_combine<CSA_BF16, 8>), cg, dim3(256), 0, s, a, sp);
        else hipLaunchKernelGGL((attn_combine<CSA_F32, 8>), cg, dim3(256), 0, s, a, sp);
      } else {
        if (bf) hipLaunchKernelGGL((attn_combine<CSA_BF16, 16>), cg, dim3(256), 0, s, a, sp);
        else hipLaunchKernelGGL((attn_combine<CSA_F32, 16>), cg, dim3(256), 0, s, a, sp);
      }
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
