// Internal launch interface between the C ABI (api.hip) and the kernel translation units.
#pragma once

#include "common.h"

namespace csa {

struct CompressArgs {
  int B, n_new, m, c;
  const int64_t* pos0;  // device [B] (nullable: all 0): entry rows start at pos0[b] / m
  int in_dtype, out_dtype;
  const void *ca, *za, *cb, *zb;
  int64_t ld, seq_stride;
  const void *halo_cb, *halo_zb;
  int64_t halo_ld, halo_seq_stride;
  const float *bias_a, *bias_b;
  void* entries;
  int64_t entries_seq_stride;
  int64_t n_cap;        // rows of `entries` per sequence (rows at or past it are not written)
  bool aligned16;
  bool overlap = true;  // pool the previous block too (CSA); false: own block only (HCA)
  int group = 1;        // threads per (entry, channel vector); set by launch_compress
  int64_t out_first = -1;  // row of `entries` receiving the first new entry (-1: pos0[b] / m)
  // Epilogue (CSA entries, compress_epilogue_ok): after rounding to the storage type, RMS norm with
  // gain gamma (nullable) and RoPE of the last rope_dims dims at the entry's last token; records: the
  // entry is packed into a 584-byte record (entries_seq_stride then counts bytes).
  bool epilogue = false;
  const float* gamma = nullptr;
  float eps = 0.f;
  int rope_dims = 0;
  double theta = 10000.0;
  bool records = false;
  // MXFP4 output (indexer keys): the entry, rounded to out_dtype, is quantised into fp4_codes
  // [B, n_cap, c/2] and fp4_scales [B, n_cap, c/32] instead of being stored (needs c % 32 == 0).
  uint8_t* fp4_codes = nullptr;
  uint8_t* fp4_scales = nullptr;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
bool compress_epilogue_ok(const CompressArgs& a);

// QK-norm and partial RoPE over B x R rows of H head vectors of D dims; row r of sequence b sits at
// position pos[b] + pos_off + r * pos_step (pos nullable: 0). gamma == nullptr: no norm;
// rope_dims == 0: no rotation; inverse: turn back.
struct NormRopeArgs {
  int B = 0, R = 0, H = 0, D = 0, dtype = 0;
  const void* x = nullptr;
  int64_t x_ld = 0, x_seq_stride = 0;
  void* y = nullptr;
  int64_t y_ld = 0, y_seq_stride = 0;
  const float* gamma = nullptr;
  float eps = 0.f;
  int rope_dims = 0;
  double theta = 10000.0;
  const int64_t* pos = nullptr;
  int64_t pos_off = 0, pos_step = 1;
  int inverse = 0;
};
hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s);

// The decode state's append for B sequences, each at its own position (decode.hip).
struct AppendArgs {
  int B = 0, m = 0, D = 0, D_I = 0, H = 0, W = 0, dtype = 0;
  bool hca = false;              // HCA state: one block of m rows [c | z], no indexer keys
  const int64_t* pos = nullptr;  // device [B]
  const void* comp = nullptr;    // [B, nc]: nc = 4D + 4D_I (CSA) or 2D (HCA)
  const void* kv = nullptr;      // [B, D]
  const void* q = nullptr;       // [B, H, D]
  void* qn = nullptr;            // [B, H, D] normalised / rotated query (nullptr: no query pass)
  void* block = nullptr;         // CSA [B, 2m, nc] (block i in rows (i % 2) * m ..), HCA [B, m, nc]
  void* win = nullptr;           // [B, W, D] ring: position p in row p % W
  void* entries = nullptr;       // [B, n_cap, D] rows or [B, n_cap, 584] records
  void* keys = nullptr;          // [B, n_cap, D_I] (CSA)
  int64_t n_cap = 0;
  int entry_fmt = 0;
  const float *bias_a = nullptr, *bias_b = nullptr, *ibias_a = nullptr, *ibias_b = nullptr;
  const float *gamma_q = nullptr, *gamma_kv = nullptr;
  float eps = 0.f;
  int rope_dims = 0;
  double theta = 10000.0;
  bool aligned16 = false;        // comp, block, entries, keys 16-byte aligned
  // MXFP4 indexer (CSA): the pooled key is quantised into keys (codes [B, n_cap, D_I/2]) and
  // key_scales [B, n_cap, D_I/32]; q_idx [B, H_I*D_I] is quantised into qi_codes / qi_scales.
  int key_fmt = 0;
  uint8_t* key_scales = nullptr;
  const void* q_idx = nullptr;
  int H_I = 0;
  uint8_t* qi_codes = nullptr;
  uint8_t* qi_scales = nullptr;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
int append_max_dim();

// 584-byte FP8 entry records of B x N entries of 512 dims (entries at b*seq_stride + n*ld).
constexpr int kEntryRecordBytes = 584;
struct EntryPackArgs {
  int B = 0, N = 0, dtype = 0;
  const void* entries = nullptr;
  int64_t ld = 512, seq_stride = 0;
  void* records = nullptr;
  int64_t rec_seq_stride = 0;  // bytes
};
hipError_t launch_entry_pack(const EntryPackArgs& a, hipStream_t s);
int norm_rope_max_dim();
int compress_max_m();

// C[M, N] (row stride ldc) = A[M, K] (row stride lda) . Bm[N, K]^T (row stride ldb)
struct GemmArgs {
  int M, N, K;
  int dtype, out_dtype;
  const void* A;
  int64_t lda;
  const void* Bm;
  int64_t ldb;
  void* C;
  int64_t ldc;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// bf16 GEMM through hipBLASLt with a caller workspace of kGemmWorkspace bytes; *done is false
// (and nothing launched) when the library path does not apply, so that launch_gemm runs instead.
constexpr size_t kGemmWorkspace = 32u << 20;
bool gemm_library_eligible(const GemmArgs& a);
hipError_t launch_gemm_library(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s, bool* done);

// MXFP4 quantisation of R rows of D values (D % 32 == 0; row r at x + r * ld elements) into
// codes [R, D/2] and scales [R, D/32], both contiguous.
struct QuantArgs {
  int64_t R = 0;
  int D = 0, dtype = 0;
  const void* x = nullptr;
  int64_t ld = 0;
  uint8_t* codes = nullptr;
  uint8_t* scales = nullptr;
};
hipError_t launch_mxfp4_quant(const QuantArgs& a, hipStream_t s);

struct IndexArgs {
  int B, T;
  const int64_t* q_pos;        // device [B] (nullable: all 0): row t of sequence b at q_pos[b] + t
  int m, H_I, D_I, k;
  int idx_dtype;
  const void* q;
  int64_t q_ld, q_seq_stride;  // elements (bf16/f32) or bytes of codes (MXFP4)
  const uint8_t* q_scale;      // MXFP4: [B, T, H_I, D_I/32]
  const float* w;
  int64_t w_ld;
  const void* keys;
  int64_t keys_seq_stride;     // elements (bf16/f32) or bytes of codes (MXFP4)
  const uint8_t* k_scale;      // MXFP4: [B, n_cap, D_I/32]
  int64_t n_cap;
  int32_t* out_idx;
  float* out_score;
};
size_t index_topk_workspace(const IndexArgs& a);
bool index_fused_fp4(const IndexArgs& a);  // MXFP4 query rows take the fused streaming path
hipError_t launch_index_topk(const IndexArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

struct TopkArgs {
  const float* scores;
  int64_t ld;
  const int32_t* n_valid;  // device [R]
  int R, k;
  int32_t* out_idx;
  float* out_score;
};
size_t topk_workspace(int R, int64_t n, int k);

// Selection over long materialised score rows (select.hip): a lower bound T0 of each row's k-th
// largest score from the maxima of G ~ 2k groups of gs consecutive scores, the entries >= T0 as
// candidates, then the exact top-k among them. g0 = min(gs, 64): the granularity at which the
// maxima are stored (gstride per row).
struct SelPlan {
  int gs, g0;
  int64_t gstride;
};
SelPlan select_plan(int64_t ld, int k);
bool select_needs_gmax(int64_t ld, int k);       // false: rows short enough to take their bound from themselves
size_t select_workspace(int R, int64_t ld, int k);
uint32_t* select_counters(void* ws);      // [R] words that must be zero before launch_select(have_gmax)
float* select_gmax(void* ws, int R);      // [R, gstride] group maxima
// have_gmax: the caller has written the maxima and zeroed the counters (the decode indexer does both)
hipError_t launch_select(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k, int32_t* out_idx,
                         float* out_score, void* ws, bool have_gmax, hipStream_t s);
hipError_t launch_topk_from_scores(const TopkArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

struct AttnArgs {
  int B, T;
  const int64_t* q_pos;    // device [B] (nullable: all 0): row t of sequence b at q_pos[b] + t
  int H, D, k, W;
  float scale;
  int in_dtype, out_dtype;
  const void* q;
  int64_t q_ld, q_seq_stride;
  const void* entries;
  int64_t entries_seq_stride, n_cap;
  const int32_t* idx;
  const void* raw;
  int64_t raw_ld, raw_seq_stride;
  const int64_t* raw_pos;  // device [B] (nullable: all 0): kv_raw row r of sequence b is position
  int64_t raw_off = 0;     // raw_pos[b] + raw_off + r (any sign; rows of negative positions are not read)
  int64_t raw_len;
  const float* sink;
  void* out;
  int dense = 0;  // attend to every visible entry in order (HCA); idx is not read and k is unused
  int m = 1;      // tokens per entry (dense only: entry i is visible to p iff (i+1)*m - 1 <= p)
  int64_t raw_ring = 0;  // > 0: kv_raw is a ring of raw_ring rows, position u in row u % raw_ring
  int entry_fmt = 0;  // 0: entries are in_dtype rows of D; 1: 584-byte FP8 records (D = 512), whose
                      // entries_seq_stride counts bytes
  // QK-norm / partial RoPE folded into the attention (fuse_fid, where attn_fuses_fid): each query
  // head is RMS-normalised with gain gamma_q (nullable: no norm, eps q_eps) and its last rope_dims dims
  // turned by its position as it is loaded (then rounded to bf16, as a stored query would be), and the
  // output's last rope_dims dims are turned back by the position before it is stored.
  bool fuse_fid = false;
  const float* gamma_q = nullptr;
  float q_eps = 0.f;
  int rope_dims = 0;
  double rope_lt = 0.0;  // log2(theta)
};
size_t attn_workspace(const AttnArgs& a);
bool attn_fuses_fid(const AttnArgs& a);  // the kernels this call runs take the fused QK-norm / RoPE
hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

// Copies rows: dst[b, r, :] = src[b, r, :] for r < rows, `cols` elements of `esize` bytes.
hipError_t launch_copy_rows(int B, int rows, int cols, int esize, const void* src, int64_t src_ld,
                            int64_t src_seq, void* dst, int64_t dst_ld, int64_t dst_seq,
                            hipStream_t s);

int probe_fail(const char* msg);
int probe_status(hipError_t e, const char* what);

constexpr int kMaxLds = 160 * 1024;  // LDS of one gfx950 compute unit
constexpr int kMaxTopK = 4096;       // largest top_k the kernels take

// Sets the dynamic-LDS ceiling of a kernel once (needed above 64 KiB).
hipError_t allow_lds(const void* kernel, int bytes);

}  // namespace csa
