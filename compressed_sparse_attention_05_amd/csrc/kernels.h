// Internal launch interface between the C ABI (api.hip) and the kernel translation units.
#pragma once

#include "common.h"

namespace csa {

struct CompressArgs {
  int B, n_new, m, c;
  int64_t first_entry;
  int in_dtype, out_dtype;
  const void *ca, *za, *cb, *zb;
  int64_t ld, seq_stride;
  const void *halo_cb, *halo_zb;
  int64_t halo_ld, halo_seq_stride;
  const float *bias_a, *bias_b;
  void* entries;
  int64_t entries_seq_stride;
  bool aligned16;
  bool overlap = true;  // pool the previous block too (CSA); false: own block only (HCA)
  int group = 1;        // threads per (entry, channel vector); set by launch_compress
  int64_t out_first = -1;  // row of `entries` receiving the first new entry (-1: first_entry)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// QK-norm and partial RoPE over B x R rows of H head vectors of D dims; row r sits at position
// pos0 + r * pos_step. gamma == nullptr: no norm; rope_dims == 0: no rotation; inverse: turn back.
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
  int64_t pos0 = 0, pos_step = 1;
  int inverse = 0;
};
hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s);

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

struct IndexArgs {
  int B, T;
  int64_t q_pos0;
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

// Multi-workgroup selection over long materialised rows (select.hip).
size_t select_workspace(int R, int64_t ld, int k);
uint32_t* select_hist(void* ws);  // the [R, 4096] histogram at the start of the workspace
// 32-bit words at the start of the workspace that must be zero before launch_select(zeroed=true)
int64_t select_zero_words(int R);
hipError_t launch_select_zero(void* ws, int R, int64_t ld, int k, hipStream_t s);
// max_valid: a bound, known on the host, of every row's n_valid (-1: none); rows longer than one
// workgroup's reach whose valid prefix fits it are still selected in one pass
hipError_t launch_select(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k, int32_t* out_idx,
                         float* out_score, void* ws, bool zeroed, hipStream_t s, int64_t max_valid = -1);
hipError_t launch_topk_from_scores(const TopkArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

struct AttnArgs {
  int B, T;
  int64_t q_pos0;
  int H, D, k, W;
  float scale;
  int in_dtype, out_dtype;
  const void* q;
  int64_t q_ld, q_seq_stride;
  const void* entries;
  int64_t entries_seq_stride, n_cap;
  const int32_t* idx;
  const void* raw;
  int64_t raw_ld, raw_seq_stride, raw_pos0, raw_len;
  const float* sink;
  void* out;
  int dense = 0;  // attend to every visible entry in order (HCA); idx is not read and k is unused
  int m = 1;      // tokens per entry (dense only: entry i is visible to p iff (i+1)*m - 1 <= p)
  int64_t raw_ring = 0;  // > 0: kv_raw is a ring of raw_ring rows, position u in row u % raw_ring
  int entry_fmt = 0;  // 0: entries are in_dtype rows of D; 1: 584-byte FP8 records (D = 512), whose
                      // entries_seq_stride counts bytes
};
size_t attn_workspace(const AttnArgs& a);
hipError_t launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

// Copies rows: dst[b, r, :] = src[b, r, :] for r < rows, `cols` elements of `esize` bytes.
hipError_t launch_copy_rows(int B, int rows, int cols, int esize, const void* src, int64_t src_ld,
                            int64_t src_seq, void* dst, int64_t dst_ld, int64_t dst_seq,
                            hipStream_t s);

constexpr int kMaxLds = 160 * 1024;  // LDS of one gfx950 compute unit

// Sets the dynamic-LDS ceiling of a kernel once (needed above 64 KiB).
hipError_t allow_lds(const void* kernel, int bytes);

}  // namespace csa
