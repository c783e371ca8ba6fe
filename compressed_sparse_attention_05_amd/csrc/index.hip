// Steps 2+3: the lightning indexer fused with top-k selection.
//
//   s[t, i] = sum_h w[h] * max(0, q_I[t, h, :] . k_I[i, :]),  i < n_vis(p_t)
// ("The Exchange Rates of a Million Tokens", section 3: ReLU-gated dot products; "Anatomy of a
// Frontier Model", bullet "Compressed Sparse Attention (CSA)": 64 heads x 128 dims, FP4 q/k.)
//
// Three paths:
//  * index_prefill_mfma (bf16, H_I = 64, D_I = 128, many query rows per sequence): a workgroup
//    holds QW consecutive query rows of one sequence, one per wave, with each wave's q_I (64 heads x
//    128 dims) resident in VGPRs as MFMA A-fragments. Key tiles of 64 entries stream through a
//    three-deep LDS ring (direct global-to-LDS loads) and are shared by the QW waves. Per tile a
//    wave runs 32
//    v_mfma_f32_32x32x16_bf16 (heads along the accumulator rows, entries along its columns),
//    reduces w_h * ReLU over the 32 heads it holds in registers plus one cross-half shuffle, and
//    offers the 64 scores to its query's streaming top-k buffer in LDS. The T x N score matrix is
//    never written.
//  * index_prefill_fp4 (MXFP4, same shapes): the same fused structure with the scaled
//    v_mfma_scale_f32_16x16x128_f8f6f4 on e2m1 codes and e8m0 block scales, one MFMA per 16 entries
//    and 16 heads covering all 128 dims.
//  * decode (few query rows, long contexts): scores of every (row, entry) are written to the
//    workspace by a key-streaming MFMA kernel (bf16, or MXFP4 through the scaled
//    v_mfma_scale_f32_16x16x128_f8f6f4 with e8m0 block scales), then selected by the top-k pass.
//  * index_generic (any dims, fp32 / bf16 / MXFP4): one wave per query row, scalar FMA scores,
//    same streaming selection.
#include "kernels.h"
#include "topk_wave.h"

namespace csa {

namespace {

// ---------------------------------------------------------------- element access

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  const float v = mag[code & 7u];
  return (code & 8u) ? -v : v;
}

// Element d of an indexer row; for MXFP4 `row` addresses the code bytes and `sc` its scales.
template <int DT>
__device__ __forceinline__ float idx_elem(const void* row, const uint8_t* sc, int d);
template <>
__device__ __forceinline__ float idx_elem<CSA_F32>(const void* row, const uint8_t*, int d) {
  return static_cast<const float*>(row)[d];
}
template <>
__device__ __forceinline__ float idx_elem<CSA_BF16>(const void* row, const uint8_t*, int d) {
  return bf2f(static_cast<const uint16_t*>(row)[d]);
}
template <>
__device__ __forceinline__ float idx_elem<CSA_MXFP4>(const void* row, const uint8_t* sc, int d) {
  const uint8_t byte = static_cast<const uint8_t*>(row)[d >> 1];
  const uint32_t code = (d & 1) ? (byte >> 4) : (byte & 15u);
  return ldexpf(e2m1_value(code), (int)sc[d >> 5] - 127);
}

template <int DT>
__device__ __forceinline__ int64_t row_units(int D_I) {
  return DT == CSA_MXFP4 ? D_I / 2 : D_I;  // elements, or code bytes for MXFP4
}

template <int DT>
__device__ __forceinline__ const void* advance(const void* p, int64_t units) {
  if (DT == CSA_F32) return static_cast<const float*>(p) + units;
  if (DT == CSA_BF16) return static_cast<const uint16_t*>(p) + units;
  return static_cast<const uint8_t*>(p) + units;
}

__device__ __forceinline__ const float* head_weights(const IndexArgs& a, int64_t row) {
  return a.w_ld ? a.w + row * a.w_ld : a.w;
}

// ---------------------------------------------------------------- generic fused path

constexpr int kGenWaves = 4;

template <int DT>
__global__ void __launch_bounds__(kGenWaves * 64) index_generic(IndexArgs a, int cap) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * kGenWaves + wave;
  if (row >= (int64_t)a.B * a.T) return;
  const int b = (int)(row / a.T), t = (int)(row % a.T);
  uint64_t* buf = reinterpret_cast<uint64_t*>(smem) + (int64_t)wave * cap;
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(smem) + kGenWaves * cap) + wave * 256;
  const int64_t nv = n_visible(pos_at(a.q_pos, b) + t, a.m, a.n_cap);
  const int64_t ru = row_units<DT>(a.D_I);
  const int nsb = a.D_I / 32;
  const void* q = advance<DT>(a.q, (int64_t)b * a.q_seq_stride + (int64_t)t * a.q_ld);
  const uint8_t* qs = DT == CSA_MXFP4 ? a.q_scale + row * a.H_I * nsb : nullptr;
  const float* w = head_weights(a, row);
  WaveTopK tk;
  tk.init(buf, hist, cap, a.k);
  for (int64_t base = 0; base < nv; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < nv;
    float s = 0.f;
    if (valid) {
      const void* krow = advance<DT>(a.keys, (int64_t)b * a.keys_seq_stride + i * ru);
      const uint8_t* ks = DT == CSA_MXFP4 ? a.k_scale + ((int64_t)b * a.n_cap + i) * nsb : nullptr;
      for (int h = 0; h < a.H_I; ++h) {
        const void* qh = advance<DT>(q, (int64_t)h * ru);
        const uint8_t* qhs = DT == CSA_MXFP4 ? qs + h * nsb : nullptr;
        float dot = 0.f;
        for (int d = 0; d < a.D_I; ++d) dot = fmaf(idx_elem<DT>(qh, qhs, d), idx_elem<DT>(krow, ks, d), dot);
        s = fmaf(w[h], relu(dot), s);
      }
    }
    tk.offer(make_cand(s, (uint32_t)i), valid);
  }
  tk.finish(a.out_idx + row * a.k, a.out_score ? a.out_score + row * a.k : nullptr);
}

// ---------------------------------------------------------------- fused MFMA prefill path

constexpr int kNE = 64;            // entries per key tile
constexpr int kTileBytes = kNE * 256;  // one tile of bf16 keys (128 dims), no padding
constexpr int kRing = 3;           // key tiles in flight: the one read and two being loaded

// A key tile in LDS is 16 blocks of 1 KB; block q = (r/16)%2 + 2*(c/4) + 8*(r/32) holds rows
// r = 32*nt + 16*(q%2) + 0..15 and 16-byte chunks c = 4*((q/2)%4) + 0..3 (dims 8c .. 8c+7) as
// slot p = r%16 + 16*(c%4). This is the order in which v_mfma_f32_32x32x16_bf16 reads its B
// fragments: at k-step s a lane l reads row 32*nt + l%32, chunk 2s + l/32, so a lane's 16 reads
// sit at one per-lane base plus offsets fixed at compile time, and every 16 consecutive lanes hit
// 16 distinct 16-byte bank groups. Each block is written by one direct-to-LDS load instruction
// (64 lanes x 16 bytes, lane p to slot p): 16 rows x 64 contiguous bytes of the key array.
__device__ __forceinline__ int key_block_row(int q, int p) { return 32 * (q >> 3) + 16 * (q & 1) + (p & 15); }
__device__ __forceinline__ int key_block_chunk(int q, int p) { return 4 * ((q >> 1) & 3) + (p >> 4); }
__device__ __forceinline__ int key_read_base(int lane) {  // bytes
  return 16 * ((lane & 15) + 16 * (lane >> 5) + 64 * ((lane >> 4) & 1));
}
__device__ __forceinline__ constexpr int key_read_off(int s, int nt) {  // bytes
  return 512 * (s & 1) + 2048 * (s >> 1) + 8192 * nt;
}


template <int QW>
__global__ void __launch_bounds__(QW * 64) index_prefill_mfma(IndexArgs a, int cap, int t_blocks) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint64_t* bufs = reinterpret_cast<uint64_t*>(smem + kRing * kTileBytes);
  uint32_t* hists = reinterpret_cast<uint32_t*>(bufs + (int64_t)QW * cap);

  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int b = blockIdx.x / t_blocks;
  const int tb = t_blocks - 1 - (int)(blockIdx.x % t_blocks);  // heaviest (latest) rows first
  const int t0 = tb * QW;
  const int t = t0 + wave;
  const bool active = t < a.T;
  const int tq = active ? t : t0;
  const int64_t row = (int64_t)b * a.T + tq;
  const int64_t qp0 = pos_at(a.q_pos, b);
  const int64_t nv = active ? n_visible(qp0 + t, a.m, a.n_cap) : 0;
  const int t_last = (t0 + QW < a.T ? t0 + QW : a.T) - 1;
  const int64_t nv_max = n_visible(qp0 + t_last, a.m, a.n_cap);

  // q_I of this wave's row as A-fragments: heads mt*32 + lane%32, dims s*16 + (lane/32)*8 .. +7
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)tq * a.q_ld;
  bf16x8 qf[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[mt][s] = *reinterpret_cast<const bf16x8*>(qrow + (mt * 32 + (lane & 31)) * 128 + s * 16 + (lane >> 5) * 8);
  // head weights of the accumulator rows this lane holds: head = mt*32 + (r/4)*8 + (lane/32)*4 + r%4
  const float* w = head_weights(a, row);
  float wr[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[mt][r] = w[mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)];

  WaveTopK tk;
  tk.init(bufs + (int64_t)wave * cap, hists + wave * 256, cap, a.k);

  const uint16_t* kseq = static_cast<const uint16_t*>(a.keys) + (int64_t)b * a.keys_seq_stride;
  const int ntiles = __builtin_amdgcn_readfirstlane((int)ceil_div(nv_max, kNE));  // uniform
  static_assert(16 % QW == 0, "each wave loads 16 / QW blocks of a key tile");
  const uint32_t ring_lds = lds_offset(smem);
  // The 16 / QW blocks this wave loads of each tile are q = j*QW + wave. Block j + 1 sits 32 key
  // rows (8 KB) past block j, so in a tile whose rows are all visible both are one per-lane byte
  // offset from a wave-uniform address; the last tile clamps its rows to the last visible entry.
  static_assert(QW == 8, "blocks wave and wave + 8 are 32 key rows apart");
  const uint32_t lane_off = (uint32_t)(key_block_row(wave, lane) * 256 + key_block_chunk(wave, lane) * 16);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(ring_lds + wave * 1024);
  const int full_tiles = __builtin_amdgcn_readfirstlane((int)(nv_max / kNE));  // tiles with every row visible
  auto load_tile = [&](int tile, int buf) {
    const uint32_t dst = wave_lds + buf * kTileBytes;
    if (tile < full_tiles) {
      const uint8_t* base = reinterpret_cast<const uint8_t*>(kseq) + (int64_t)tile * kTileBytes;
#pragma unroll
      for (int j = 0; j < 16 / QW; ++j) copy_to_lds16_sbase(base + j * 8192, lane_off, dst + j * QW * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < 16 / QW; ++j) {
        const int q = j * QW + wave;
        int64_t e = (int64_t)tile * kNE + key_block_row(q, lane);
        e = e < nv_max ? e : nv_max - 1;  // rows past the last visible entry are never offered
        copy_to_lds16(kseq + e * 128 + key_block_chunk(q, lane) * 8, dst + j * QW * 1024);
      }
    }
  };
  // waits for this wave's copies of every tile but the newest `pending` ones (2 instructions each)
  auto wait_tiles = [&](int pending) {
    static_assert(16 / QW == 2, "vmcnt immediates assume two copies per wave and tile");
    if (pending) wait_vmcnt<2>();
    else wait_vmcnt<0>();
  };

  // Software pipeline over 32-entry column tiles: while the matrix cores run one column tile, the
  // VALU reduces the heads of the previous one. The source order below is the issue order (each
  // sched_barrier pins it): every MFMA is followed by the ReLU + weighted sums of one accumulator
  // row of both head tiles of the other column tile, which run while the MFMA is in flight.
  //   phase A of tile t: MFMA column 0 of t  |  reduce column 1 of t-1, read column 1 of t
  //   barrier: tile t+1 published
  //   phase B of tile t: MFMA column 1 of t  |  reduce column 0 of t, read column 0 of t+1
  //   and, within phase B, offer the 64 scores of tile t-1 (column 0 from phase B of t-1, column 1
  //   from phase A of t)
  f32x16 acc0[2], acc1[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) acc1[mt] = f32x16{};
  float part0 = 0.f;
  const int lbase = key_read_base(lane);

  // p4[r & 3] += w_h * ReLU(acc[mt][r]) for both head tiles mt
  auto reduce_r = [&](float (&p4)[4], const f32x16 (&acc)[2], int r) {
    p4[r & 3] = fmaf(wr[0][r], relu(acc[0][r]), p4[r & 3]);
    p4[r & 3] = fmaf(wr[1][r], relu(acc[1][r]), p4[r & 3]);
  };

  // Every prologue load (q_I, w) has landed before the loop, so that no wait for them is left in
  // the loop body.
  __builtin_amdgcn_s_waitcnt(0);
  if (ntiles > 0) load_tile(0, 0);
  if (ntiles > 1) load_tile(1, 1);
  wait_tiles(ntiles > 1);
  __syncthreads();
  // Column 0 of a tile is read during phase B of the tile before (after the barrier that publishes
  // it), so phase A starts on fragments already in registers.
  bf16x8 kf0[8], kf1[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kf0[s] = *reinterpret_cast<const bf16x8*>(smem + lbase + key_read_off(s, 0));
  int cur = 0;  // ring slot of the tile being read
  for (int tile = 0; tile < ntiles; ++tile) {
    const uint8_t* kt = smem + cur * kTileBytes + lbase;
    const int nxt = cur == kRing - 1 ? 0 : cur + 1;
    if (tile + 2 < ntiles) load_tile(tile + 2, cur == 0 ? 2 : cur - 1);
    float sc;
    float p4[4] = {0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc0[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], kf0[s], s ? acc0[0] : f32x16{}, 0, 0, 0);
      asm volatile("" ::"v"(acc0[0]));
      reduce_r(p4, acc1, 2 * s);
      __builtin_amdgcn_sched_barrier(0);
      acc0[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], kf0[s], s ? acc0[1] : f32x16{}, 0, 0, 0);
      asm volatile("" ::"v"(acc0[1]));
      kf1[s] = *reinterpret_cast<const bf16x8*>(kt + key_read_off(s, 1));
      reduce_r(p4, acc1, 2 * s + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const float part1 = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      // lanes < 32 end with column 0 of t-1 (both head halves), lanes >= 32 with column 1
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1), false, false);
      sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    // tile + 1 has landed and every wave is past its reads of tile - 1
    if (tile + 1 < ntiles) {
      wait_tiles(tile + 2 < ntiles);
      __syncthreads();
    }
    const uint8_t* kn = smem + nxt * kTileBytes + lbase;
#pragma unroll
    for (int j = 0; j < 4; ++j) p4[j] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc1[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], kf1[s], s ? acc1[0] : f32x16{}, 0, 0, 0);
      asm volatile("" ::"v"(acc1[0]));
      reduce_r(p4, acc0, 2 * s);
      __builtin_amdgcn_sched_barrier(0);
      acc1[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], kf1[s], s ? acc1[1] : f32x16{}, 0, 0, 0);
      asm volatile("" ::"v"(acc1[1]));
      // column 0 of tile + 1 (an unused read of the next ring slot after the last tile)
      kf0[s] = *reinterpret_cast<const bf16x8*>(kn + key_read_off(s, 0));
      reduce_r(p4, acc0, 2 * s + 1);
      // the 64 scores of tile - 1 go to the streaming top-k while this phase's MFMAs are in flight
      if (s == 1 && active && tile > 0) {
        const uint32_t i = (uint32_t)(tile - 1) * kNE + lane;
        tk.offer(make_cand(sc, i), i < (uint32_t)nv);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    part0 = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    asm volatile("" ::"v"(part0));  // keeps the reduction inside phase B
    cur = nxt;
  }
  if (ntiles > 0) {
    float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) reduce_r(p4, acc1, r);
    const float part1 = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1), false, false);
    const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (active) {
      const int64_t i = (int64_t)(ntiles - 1) * kNE + lane;
      tk.offer(make_cand(sc, (uint32_t)i), i < nv);
    }
  }
  if (active) tk.finish(a.out_idx + row * a.k, a.out_score ? a.out_score + row * a.k : nullptr);
}

constexpr int kPrefillQW = 8;

int prefill_lds(int cap) { return kRing * kTileBytes + kPrefillQW * (cap * 8 + 256 * 4); }

// ---------------------------------------------------------------- fused MXFP4 prefill path

// The MXFP4 form of index_prefill_mfma: QW = 8 consecutive query rows of one sequence, one per wave,
// each wave's q_I (64 heads x 128 dims: 4 KiB of codes and 256 scale bytes) held as the A operands of
// v_mfma_scale_f32_16x16x128_f8f6f4 (head mt*16 + lane%16, code bytes 16(lane/16) .. +15 = dims
// 32(lane/16) .. +31, with that block's e8m0 scale). Key tiles of 128 entries (8 KiB of codes and
// 512 scale bytes) stream through a three-deep LDS ring by direct global-to-LDS loads, shared by
// the 8 waves: wave w loads column group w (16 entries, stored so that lane l's B operand, entry
// l%16 and code bytes 16(l/16) .. +15, is LDS bytes 16l .. 16l + 15 of the group: one conflict-free
// 16-byte read), waves 0 and 1 load the scales. One MFMA per (column group, head tile) forms all 128
// dims of the dot products with the block scales applied; w_h * ReLU is summed over the 16 heads a
// lane holds, and three lane swaps (two 32-lane, one 16-lane) turn the 4 column groups' partial sums
// into one score per lane, entry base + lane, offered to the wave's streaming top-k. The T x N score
// matrix is never written.
constexpr int kF4NE = 128;                             // entries per key tile
constexpr int kF4CodeBytes = kF4NE * 64;               // 128 dims at 4 bits
constexpr int kF4TileBytes = kF4CodeBytes + kF4NE * 4;  // + 4 scale bytes per entry
constexpr int kF4Ring = 3;
constexpr int kF4QW = 8;

__global__ void __launch_bounds__(kF4QW * 64) index_prefill_fp4(IndexArgs a, int cap, int t_blocks) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint64_t* bufs = reinterpret_cast<uint64_t*>(smem + kF4Ring * kF4TileBytes);
  uint32_t* hists = reinterpret_cast<uint32_t*>(bufs + (int64_t)kF4QW * cap);

  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int b = blockIdx.x / t_blocks;
  const int tb = t_blocks - 1 - (int)(blockIdx.x % t_blocks);  // heaviest (latest) rows first
  const int t0 = tb * kF4QW;
  const int t = t0 + wave;
  const bool active = t < a.T;
  const int tq = active ? t : t0;
  const int64_t row = (int64_t)b * a.T + tq;
  const int64_t qp0 = pos_at(a.q_pos, b);
  const int64_t nv = active ? n_visible(qp0 + t, a.m, a.n_cap) : 0;
  const int t_last = (t0 + kF4QW < a.T ? t0 + kF4QW : a.T) - 1;
  const int64_t nv_max = n_visible(qp0 + t_last, a.m, a.n_cap);

  const int g = lane >> 4, c = lane & 15;
  const uint8_t* qcodes = static_cast<const uint8_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)tq * a.q_ld;
  const uint8_t* qsc = a.q_scale + row * (64 * 4);
  i32x8 qa[4];
  int qs[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(qcodes + (mt * 16 + c) * 64 + g * 16);
    qa[mt] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    qs[mt] = qsc[(mt * 16 + c) * 4 + g];
  }
  // head weights of the accumulator rows this lane holds: head mt*16 + 4(lane/16) + r
  const float* w = head_weights(a, row);
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[mt][r] = w[mt * 16 + g * 4 + r];

  WaveTopK tk;
  tk.init(bufs + (int64_t)wave * cap, hists + wave * 256, cap, a.k);

  const uint8_t* kcodes = static_cast<const uint8_t*>(a.keys) + (int64_t)b * a.keys_seq_stride;
  const uint8_t* kscale = a.k_scale + (int64_t)b * a.n_cap * 4;
  const int ntiles = __builtin_amdgcn_readfirstlane((int)ceil_div(nv_max, kF4NE));  // uniform
  const uint32_t ring_lds = lds_offset(smem);
  // A tile whose rows are all visible is loaded from wave-uniform addresses plus per-lane byte
  // offsets; in the last tile, rows past the last visible entry are loaded as that entry (in bounds)
  // and never offered.
  const uint32_t code_off = (uint32_t)((wave * 16 + c) * 64 + g * 16);
  const uint32_t scale_off = (uint32_t)((wave * 64 + lane) * 4);  // waves 0 and 1
  const uint32_t code_lds = __builtin_amdgcn_readfirstlane(ring_lds + wave * 1024);
  const uint32_t scale_lds = __builtin_amdgcn_readfirstlane(ring_lds + kF4CodeBytes + wave * 256);
  const int full_tiles = __builtin_amdgcn_readfirstlane((int)(nv_max / kF4NE));
  auto load_tile = [&](int tile, int slot) {
    const uint32_t sb = slot * kF4TileBytes;
    if (tile < full_tiles) {
      copy_to_lds16_sbase(kcodes + (int64_t)tile * kF4CodeBytes, code_off, code_lds + sb);
      if (wave < 2) copy_to_lds4_sbase(kscale + (int64_t)tile * kF4NE * 4, scale_off, scale_lds + sb);
    } else {
      int64_t e = (int64_t)tile * kF4NE + wave * 16 + c;
      e = e < nv_max ? e : nv_max - 1;
      copy_to_lds16(kcodes + e * 64 + g * 16, code_lds + sb);
      if (wave < 2) {
        int64_t es = (int64_t)tile * kF4NE + wave * 64 + lane;
        es = es < nv_max ? es : nv_max - 1;
        copy_to_lds4(kscale + es * 4, scale_lds + sb);
      }
    }
  };
  // waits until this wave's copies of every tile but the newest `pending` one have landed
  auto wait_tiles = [&](bool pending) {
    if (!pending) wait_vmcnt<0>();
    else if (wave < 2) wait_vmcnt<2>();
    else wait_vmcnt<1>();
  };

  // the q_I and w loads land before the loop, so no wait for them is left inside it
  __builtin_amdgcn_s_waitcnt(0);
  if (ntiles > 0) load_tile(0, 0);
  if (ntiles > 1) load_tile(1, 1);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int slot = tile % kF4Ring;
    wait_tiles(tile + 1 < ntiles);
    __syncthreads();  // tile published; every wave is past its reads of tile - 1
    if (tile + 2 < ntiles) load_tile(tile + 2, (tile + 2) % kF4Ring);
    const uint8_t* tp = smem + slot * kF4TileBytes;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // the 16 MFMAs of the half (four column groups x four head tiles) are issued first, each into an
      // accumulator of its own (pinned in place by empty asm uses), then the ReLU and weighted sums
      // read them: no sum waits for the MFMA just issued, and the other wave of the SIMD fills the gap
      // (issuing all 32 of the tile first was measured slower)
      i32x4 kv[4];
      int ks[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int grp = half * 4 + q;
        kv[q] = *reinterpret_cast<const i32x4*>(tp + grp * 1024 + lane * 16);
        ks[q] = tp[kF4CodeBytes + (grp * 16 + c) * 4 + g];
      }
      f32x4 acc[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x8 kb = i32x8{kv[q][0], kv[q][1], kv[q][2], kv[q][3], 0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc[q][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb, f32x4{}, 4, 4, 0, qs[mt], 0, ks[q]);
          asm volatile("" ::"v"(acc[q][mt]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float sp = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sp = fmaf(wr[mt][r], relu(acc[q][mt][r]), sp);
        p[q] = sp;
      }
      // p[q] at lane l: column group q, entry l%16, the heads of lane group l/16. After the swaps lane l
      // holds the sum over the four lane groups of column group l/16, entry l%16: entry 64 half + l.
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
      const float h02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
      const float h13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h02), __float_as_uint(h13), false, false);
      const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const uint32_t i = (uint32_t)tile * kF4NE + half * 64 + lane;
      if (active) tk.offer(make_cand(sc, i), i < (uint32_t)nv);
    }
  }
  if (active) tk.finish(a.out_idx + row * a.k, a.out_score ? a.out_score + row * a.k : nullptr);
}

int prefill_fp4_lds(int cap) { return kF4Ring * kF4TileBytes + kF4QW * (cap * 8 + 256 * 4); }

// ---------------------------------------------------------------- decode scores

// Loads one 64-entry tile of bf16 keys as B-fragments of v_mfma_f32_16x16x32_bf16: for column
// group g and k-step s, lane l holds entry base + g*16 + l%16, dims s*32 + (l/16)*8 .. +7.
__device__ __forceinline__ void load_keys16(uint4 (&kb)[16], const uint16_t* kseq, int64_t base, int64_t nv,
                                            int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t e = base + g * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kb[g * 4 + s] = e < nv ? *reinterpret_cast<const uint4*>(kseq + e * 128 + s * 32 + (lane >> 4) * 8)
                             : make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------- decode scores, streamed

// Decode writes scores[row, i] for i < n_vis(row), n_valid[row] = n_vis(row), and the maxima of every
// g0 consecutive scores (gmax[row, i / g0]) that the selection's lower bound starts from. A row's
// visible count is formed where its q_I is loaded.
// score of entry base + lane (valid: i < nv) to the row and its g0-group maximum (-inf for lanes past nv)
__device__ __forceinline__ void store_scores(float* scores, float* gmax, int64_t row, int64_t n_cap, int64_t gstride,
                                             int g0, int64_t base, int64_t nv, float mine) {
  const int lane = lane_id();
  const int64_t i = base + lane;
  const bool valid = i < nv;
  if (valid) scores[row * n_cap + i] = mine;
  if (g0 == 0) return;  // short rows: the selection needs no group maxima
  // maximum over aligned groups of g0 (16, 32 or 64) lanes by lane permutations on the vector unit:
  // two quad permutations and the half-row and row mirrors (groups of 4, 8, 16), then the 16- and
  // 32-lane swaps
  float v = valid ? mine : -INFINITY;
  auto dpp_max = [](float x, auto ctrl) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false)));
  };
  v = dpp_max(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  v = dpp_max(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  v = dpp_max(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v = dpp_max(v, std::integral_constant<int, 0x140>{});  // row_mirror
  if (g0 >= 32) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  if (g0 >= 64) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  if ((lane & (g0 - 1)) == 0 && valid) gmax[row * gstride + i / g0] = v;
}

// The (row, 512-entry unit) space is walked grid-stride by workgroups of 8 waves, so at every step
// the whole chip reads adjacent 128 KiB units of the key arrays. The unit's row has its q_I staged
// in LDS once (A-fragments are read from there), which keeps a wave at ~128 VGPRs and four waves
// per SIMD in flight; each wave multiplies one 64-entry tile of the unit.
// v_mfma_f32_16x16x32_bf16 with heads along the rows (4 M-tiles) and 16 entries along the columns:
// lane l reads entry l%16, dims s*32 + (l/16)*8 .. +7 of k-step s (16 rows x 64 contiguous bytes per
// load instruction).
constexpr int kStreamWaves = 8;
constexpr int kUnit = kStreamWaves * 64;
constexpr int kQLd = 136;  // LDS row stride (bf16) of the staged q_I heads

// (at most 128 VGPRs: two workgroups of eight waves per compute unit)
__global__ void __launch_bounds__(kStreamWaves * 64, 4) score_bf16_stream(IndexArgs a, float* scores, int32_t* n_valid,
                                                                        int64_t units_per_row, uint32_t* zero,
                                                                        int64_t zero_words, float* gmax, int g0,
                                                                        int64_t gstride, int64_t sld) {
  __shared__ __align__(16) uint16_t qs[64 * kQLd];
  __shared__ float ws[64];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  // the selection's counters start at zero (they are read only after this kernel)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < zero_words; i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = 0u;
  const int64_t R = (int64_t)a.B * a.T;
  const int64_t total = R * units_per_row;
  // every row's whole units first, then each row's last partial unit (when n_cap is not a multiple of
  // the unit): the partial units then share the walk's last step instead of adding a step of their own
  const int64_t upr_full = a.n_cap / kUnit, full = R * upr_full;
  int64_t cur_row = -1;
  int64_t nv_cur = 0;
  for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int64_t row = u < full ? u / upr_full : u - full;
    const int64_t unit = u < full ? u % upr_full : upr_full;
    const int64_t base = unit * kUnit + wave * 64;
    const int b = (int)(row / a.T), tq = (int)(row % a.T);
    if (row != cur_row) {  // uniform across the workgroup
      __syncthreads();
      cur_row = row;
      nv_cur = n_visible(pos_at(a.q_pos, b) + tq, a.m, a.n_cap);
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)tq * a.q_ld;
      for (int c = threadIdx.x; c < 64 * 16; c += kStreamWaves * 64)
        *reinterpret_cast<uint4*>(&qs[(c >> 4) * kQLd + (c & 15) * 8]) = *reinterpret_cast<const uint4*>(qrow + c * 8);
      if (threadIdx.x < 64) ws[threadIdx.x] = head_weights(a, row)[threadIdx.x];
      if (threadIdx.x == 0 && unit == 0) n_valid[row] = (int32_t)nv_cur;
      __syncthreads();
    }
    const int64_t nv = nv_cur;
    if (base >= nv) continue;
    const uint16_t* kseq = static_cast<const uint16_t*>(a.keys) + (int64_t)b * a.keys_seq_stride;
    uint4 kb[16];
    load_keys16(kb, kseq, base, nv, lane);
    float wr[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[mt][r] = ws[mt * 16 + (lane >> 4) * 4 + r];
    float mine = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // re-read the q_I fragments from LDS for every column group instead of holding all 64 VGPRs
      asm volatile("" ::: "memory");
      f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, kb[g * 4 + s]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          // A-fragment: head mt*16 + lane%16, dims s*32 + (lane/16)*8 .. +7
          const bf16x8 qf = *reinterpret_cast<const bf16x8*>(&qs[(mt * 16 + (lane & 15)) * kQLd + s * 32 + (lane >> 4) * 8]);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, kf, acc[mt], 0, 0, 0);
        }
      }
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p4[r] = fmaf(wr[mt][r], relu(acc[mt][r]), p4[r]);
      float p = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      if ((lane >> 4) == g) mine = p;  // lane l keeps entry base + l
    }
    store_scores(scores, gmax, row, sld, gstride, g0, base, nv, mine);
  }
}

// MXFP4 variant: a tile is 64 entries x (64 code bytes + 4 scale bytes); each key group of 16 entries
// is one B operand of v_mfma_scale_f32_16x16x128_f8f6f4 (lane l: entry l%16, codes 16(l/16) .. +15,
// the e8m0 scale of those 32 dims), so no dequantisation pass exists. Waves take one tile per step,
// grid-stride, so that at every step the chip reads one contiguous stretch of the key arrays (measured
// faster than giving each wave a run of consecutive tiles, or issuing several tiles' loads at once).
constexpr int kFp4Waves = 4;

__global__ void __launch_bounds__(kFp4Waves * 64, 4) score_fp4_stream(IndexArgs a, float* scores, int32_t* n_valid,
                                                                     int64_t tiles_per_row, uint32_t* zero,
                                                                     int64_t zero_words, float* gmax, int g0,
                                                                     int64_t gstride, int64_t sld) {
  const int lane = lane_id();
  // the selection's counters start at zero (they are read only after this kernel)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < zero_words; i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = 0u;
  const int g = lane >> 4, c = lane & 15;
  const int64_t R = (int64_t)a.B * a.T;
  const int64_t total = R * tiles_per_row;
  const int64_t nwaves = (int64_t)gridDim.x * kFp4Waves;
  int64_t cur_row = -1, nv = 0;
  i32x8 qa[4];
  int qs[4];
  float wr[4][4];
  const int64_t tpr_full = a.n_cap / 64, full = R * tpr_full;  // whole tiles first, as in the bf16 walk
  for (int64_t t = (int64_t)blockIdx.x * kFp4Waves + (threadIdx.x >> 6); t < total; t += nwaves) {
    const int64_t row = t < full ? t / tpr_full : t - full;
    const int64_t base = (t < full ? t % tpr_full : tpr_full) * 64;
    const int b = (int)(row / a.T), tq = (int)(row % a.T);
    if (row != cur_row) {
      cur_row = row;
      nv = n_visible(pos_at(a.q_pos, b) + tq, a.m, a.n_cap);
      const uint8_t* qcodes = static_cast<const uint8_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)tq * a.q_ld;
      const uint8_t* qsc = a.q_scale + row * (64 * 4);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(qcodes + (mt * 16 + c) * 64 + g * 16);
        qa[mt] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        qs[mt] = qsc[(mt * 16 + c) * 4 + g];
      }
      const float* w = head_weights(a, row);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[mt][r] = w[mt * 16 + g * 4 + r];
    }
    if (base == 0 && lane == 0) n_valid[row] = (int32_t)nv;
    if (base >= nv) continue;
    const uint8_t* kcodes = static_cast<const uint8_t*>(a.keys) + (int64_t)b * a.keys_seq_stride;
    const uint8_t* ksc = a.k_scale + (int64_t)b * a.n_cap * 4;
    i32x4 kv[4];
    int ks[4];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int64_t e = base + grp * 16 + c;
      kv[grp] = e < nv ? *reinterpret_cast<const i32x4*>(kcodes + e * 64 + g * 16) : i32x4{0, 0, 0, 0};
      ks[grp] = e < nv ? ksc[e * 4 + g] : 127;
    }
    float mine = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const i32x8 kb = i32x8{kv[grp][0], kv[grp][1], kv[grp][2], kv[grp][3], 0, 0, 0, 0};
      float p = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = {};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb, acc, 4, 4, 0, qs[mt], 0, ks[grp]);
#pragma unroll
        for (int r = 0; r < 4; ++r) p = fmaf(wr[mt][r], relu(acc[r]), p);
      }
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      if (g == grp) mine = p;
    }
    store_scores(scores, gmax, row, sld, gstride, g0, base, nv, mine);
  }
}

int stream_grid() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = n;
    if (cus <= 0) cus = 256;
  }
  return 2 * cus;
}


bool use_prefill_mfma(const IndexArgs& a) {
  return a.idx_dtype == CSA_BF16 && a.H_I == 64 && a.D_I == 128 && a.T >= kPrefillQW &&
         prefill_lds(topk_cap_for(a.k, 512)) <= kMaxLds;
}
bool use_prefill_fp4(const IndexArgs& a) {
  return a.idx_dtype == CSA_MXFP4 && a.H_I == 64 && a.D_I == 128 && a.T >= kF4QW &&
         prefill_fp4_lds(topk_cap_for(a.k, 512)) <= kMaxLds;
}
// Few query rows per sequence (decode): every visible score passes through the workspace. Many
// rows always take a fused path (the MFMA kernels, else index_generic), so no T x N matrix exists.
bool use_decode_scores(const IndexArgs& a) {
  if (a.H_I != 64 || a.D_I != 128) return false;
  return (a.idx_dtype == CSA_BF16 || a.idx_dtype == CSA_MXFP4) && a.T < kPrefillQW;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// row stride of the decode score matrix: n_cap rounded up to 64 scores, so that every row starts
// 256-byte aligned (up to 32768 entries this keeps the one-launch selection: 32768 is a multiple)
int64_t score_ld(int64_t n_cap) { return (n_cap + 63) / 64 * 64; }

}  // namespace

bool index_fused_fp4(const IndexArgs& a) { return use_prefill_fp4(a); }

size_t index_topk_workspace(const IndexArgs& a) {
  if (!use_decode_scores(a)) return 0;
  const int64_t R = (int64_t)a.B * a.T;
  const int64_t sld = score_ld(a.n_cap);
  return align256((size_t)R * sld * 4) + align256((size_t)R * 4) + select_workspace((int)R, sld, a.k);
}

hipError_t launch_index_topk(const IndexArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = (int64_t)a.B * a.T;
  if (R == 0) return hipSuccess;
  hipError_t e;
  if (use_prefill_mfma(a)) {
    const int cap = topk_cap_for(a.k, 512);
    const int lds = prefill_lds(cap);
    if ((e = allow_lds((const void*)index_prefill_mfma<kPrefillQW>, lds)) != hipSuccess) return e;
    const int t_blocks = (int)ceil_div(a.T, kPrefillQW);
    hipLaunchKernelGGL(index_prefill_mfma<kPrefillQW>, dim3((unsigned)(a.B * t_blocks)), dim3(kPrefillQW * 64),
                       lds, s, a, cap, t_blocks);
    return hipGetLastError();
  }
  if (use_prefill_fp4(a)) {
    const int cap = topk_cap_for(a.k, 512);
    const int lds = prefill_fp4_lds(cap);
    if ((e = allow_lds((const void*)index_prefill_fp4, lds)) != hipSuccess) return e;
    const int t_blocks = (int)ceil_div(a.T, kF4QW);
    hipLaunchKernelGGL(index_prefill_fp4, dim3((unsigned)(a.B * t_blocks)), dim3(kF4QW * 64), lds, s, a, cap,
                       t_blocks);
    return hipGetLastError();
  }
  if (use_decode_scores(a)) {
    if (ws == nullptr || ws_bytes < index_topk_workspace(a)) return hipErrorInvalidValue;
    uint8_t* p = static_cast<uint8_t*>(ws);
    float* scores = reinterpret_cast<float*>(p);
    const int64_t sld = score_ld(a.n_cap);  // rows of the score matrix start 256-byte aligned
    p += align256((size_t)R * sld * 4);
    int32_t* nvalid = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)R * 4);
    const SelPlan pl = select_plan(sld, a.k);
    float* gm = select_gmax(p, (int)R);
    const int g0 = select_needs_gmax(sld, a.k) ? pl.g0 : 0;
    if (a.idx_dtype == CSA_MXFP4) {
      const int64_t tpr = ceil_div(a.n_cap, 64) > 0 ? ceil_div(a.n_cap, 64) : 1;
      int64_t g = ceil_div(R * tpr, kFp4Waves);
      if (g > 2 * stream_grid()) g = 2 * stream_grid();
      hipLaunchKernelGGL(score_fp4_stream, dim3((unsigned)g), dim3(kFp4Waves * 64), 0, s, a, scores, nvalid, tpr,
                         select_counters(p), R, gm, g0, pl.gstride, sld);
    } else {
      const int64_t upr = ceil_div(a.n_cap, kUnit) > 0 ? ceil_div(a.n_cap, kUnit) : 1;
      int64_t g = R * upr;
      if (g > stream_grid()) g = stream_grid();
      hipLaunchKernelGGL(score_bf16_stream, dim3((unsigned)g), dim3(kStreamWaves * 64), 0, s, a, scores, nvalid, upr,
                         select_counters(p), R, gm, g0, pl.gstride, sld);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_select(scores, sld, nvalid, (int)R, a.k, a.out_idx, a.out_score, p, true, s);
  }
  const int cap = topk_cap_for(a.k, 256);
  const int lds = kGenWaves * (cap * 8 + 256 * 4);
  const dim3 grid((unsigned)ceil_div(R, kGenWaves));
  switch (a.idx_dtype) {
    case CSA_F32:
      if ((e = allow_lds((const void*)index_generic<CSA_F32>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(index_generic<CSA_F32>, grid, dim3(kGenWaves * 64), lds, s, a, cap);
      break;
    case CSA_BF16:
      if ((e = allow_lds((const void*)index_generic<CSA_BF16>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(index_generic<CSA_BF16>, grid, dim3(kGenWaves * 64), lds, s, a, cap);
      break;
    default:
      if ((e = allow_lds((const void*)index_generic<CSA_MXFP4>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(index_generic<CSA_MXFP4>, grid, dim3(kGenWaves * 64), lds, s, a, cap);
      break;
  }
  return hipGetLastError();
}

}  // namespace csa
