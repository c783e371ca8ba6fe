/*
 * csa.h — C ABI of the Compressed Sparse Attention (CSA) forward pass on AMD Instinct MI355X
 * (gfx950). Hand-written HIP kernels; no torch types cross this boundary.
 *
 * The layer (DeepSeek-V4's CSA, as described on the pages "Anatomy of a Frontier Model: Reading
 * DeepSeek-V4 Through Part V", section "The attention: compress, then select", and "The Exchange
 * Rates of a Million Tokens", section 3) runs four steps:
 *   1. compress   every m tokens into one K=V entry by per-channel softmax pooling with learned
 *                 position biases, each entry pooling its own block and the previous one;
 *   2. index      score each query against every causally visible entry:
 *                 s[t,i] = sum_h w_h * ReLU(q_I[t,h] . k_I[i]);
 *   3. top-k      keep the k best entries per query;
 *   4. attend     single-KV-head attention over the selected entries plus the last W raw tokens.
 *
 * Conventions (every entry point):
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major. Strides are in elements
 *     of the tensor's dtype unless stated otherwise. The library never frees or keeps them.
 *   - Scalars and the small structs below live in HOST memory and are read during the call only.
 *   - Every call validates its arguments on the host before any HIP call. On failure nothing is
 *     launched and an error code is returned; csa_last_error() then describes it (thread-local).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - No device memory is allocated by a compute call: scratch comes from the caller's workspace
 *     `ws` of `ws_bytes` bytes (256-byte aligned), sized by csa_workspace_size().
 *   - Results are deterministic: no floating-point atomics, fixed reduction orders, and top-k ties
 *     broken toward the smaller entry index. A sequence's results do not depend on the other
 *     sequences of its batch, nor on the batch size.
 *   - Positions are per sequence: a DEVICE array `const int64_t*` of B values (8-byte aligned),
 *     read by the kernels, so the sequences of one batch may sit at different lengths and a decode
 *     loop can advance them without a host round trip. Query row t of sequence b sits at absolute
 *     position pos[b] + t. NULL means every sequence is at 0; a negative query position counts as
 *     0. The host cannot see these values: calls check what they can (pointers, strides, sizes)
 *     and the kernels clamp every row they derive from a position to the buffers they were given,
 *     so a position outside an entry point's stated contract gives unspecified results, never an
 *     access outside the caller's tensors.
 *   - Visibility ("Anatomy of a Frontier Model", bullet "A sliding window in every layer": an entry
 *     is formed once its block is complete): entry i (tokens [i*m, (i+1)*m)) is visible to position
 *     p iff (i+1)*m - 1 <= p, so n_vis(p) = min(floor((p+1)/m), n_cap).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_OK 0
#define CSA_ERR_ARG (-1)          /* invalid argument (shape, stride, pointer, value)          */
#define CSA_ERR_UNSUPPORTED (-2)  /* valid but not implemented (dtype/shape combination)         */
#define CSA_ERR_WORKSPACE (-3)    /* workspace missing, misaligned or too small                  */
#define CSA_ERR_HIP (-4)          /* a HIP runtime call failed (launch error, no device)         */

/* Storage types. */
#define CSA_F32 0
#define CSA_BF16 1
#define CSA_MXFP4 2  /* indexer q/k only: e2m1 codes, 2 per byte (even element in the low nibble),
                        plus one e8m0 scale byte per 32 elements (OCP Microscaling v1.0). */

/* Operations, for csa_workspace_size. */
#define CSA_OP_COMPRESS 0
#define CSA_OP_INDEX_TOPK 1
#define CSA_OP_TOPK_FROM_SCORES 2
#define CSA_OP_SPARSE_ATTN 3
#define CSA_OP_FORWARD 4
#define CSA_OP_DENSE_ATTN 5  /* csa_dense_attn; n_cap bounds the entries a row can see */
#define CSA_OP_DECODE_STEP 6 /* csa_decode_step; T = 1, idx_dtype = the activation dtype */
#define CSA_OP_HCA_DECODE_STEP 7 /* csa_hca_decode_step; T = 1, idx_dtype = the activation dtype */
#define CSA_OP_SPARSE_ATTN_QK 8  /* csa_sparse_attn_qk; idx_dtype = the query dtype */

/* Layer dimensions. */
typedef struct csa_dims {
  int32_t m;        /* tokens per compressed entry (4 in DeepSeek-V4's CSA layers)              */
  int32_t D;        /* entry dim = query head dim; the entry is both key and value (512)         */
  int32_t H;        /* query heads, all sharing the one KV head (64 / 128)                       */
  int32_t H_I;      /* indexer heads (64)                                                        */
  int32_t D_I;      /* indexer head dim (128)                                                    */
  int32_t top_k;    /* entries kept per query (512 / 1024)                                       */
  int32_t window;   /* raw tokens attended directly, including the query's own (128)             */
  float sm_scale;   /* softmax scale; 0 selects 1/sqrt(D)                                       */
} csa_dims;

/* The ABI revision (3: per-sequence device position arrays, MXFP4 key caches). */
int csa_version(void);
/* The message of this thread's last failed call ("" after a successful one). */
const char* csa_last_error(void);

/*
 * Bytes of workspace an operation needs (written to *bytes). `T` is query rows per sequence,
 * `n_cap` the entry capacity per sequence, `d_model` the width of x (CSA_OP_FORWARD only),
 * `idx_dtype` the indexer storage type (CSA_OP_INDEX_TOPK / CSA_OP_FORWARD).
 * For CSA_OP_TOPK_FROM_SCORES pass R (rows) as B, T = 1 and the row length as n_cap.
 * Errors: CSA_ERR_ARG for an unknown op or negative sizes.
 */
int csa_workspace_size(int op, const csa_dims* dims, int B, int T, int64_t n_cap, int d_model,
                       int idx_dtype, int64_t* bytes);

/*
 * Step 1 — compressor ("The Exchange Rates of a Million Tokens", section 3: two overlapping
 * series under one joint softmax; "Anatomy of a Frontier Model", bullet "Compressed Sparse
 * Attention (CSA)": per-channel softmax pooling with learned position biases over the entry's own
 * block and the one before).
 * For each sequence b, complete block of this call (entry i = pos0[b]/m + e, e < floor(T/m)) and
 * channel j:
 *   logits = { za[i*m+r, j] + bias_a[r, j] }_{r<m}  U  { zb[(i-1)*m+r, j] + bias_b[r, j] }_{r<m}
 *   entries[i, j] = softmax(logits) . [ca[i*m+r, j] ; cb[(i-1)*m+r, j]]
 * Entry 0 pools its own block only. Tokens of an incomplete trailing block produce nothing.
 *   ca, za, cb, zb  [B, T, c] views: token stride `ld`, sequence stride `seq_stride` (elements,
 *                   shared by the four), channel stride 1; dtype `in_dtype` (F32 or BF16).
 *   pos0            device int64 [B]: the chunk's first position per sequence, a multiple of m
 *                   with pos0[b]/m + floor(T/m) <= n_cap (rows at or past n_cap are not written).
 *                   NULL: every sequence starts at 0.
 *   halo_cb/zb      the previous block's cb/zb rows [B, m, c] (stride halo_ld / halo_seq_stride),
 *                   required when pos0 is given (the rows of sequences at 0 are not read); may be
 *                   NULL when pos0 is NULL.
 *   bias_a/b        [m, c] float32.
 *   entries         [B, n_cap, c] (row stride c, sequence stride entries_seq_stride), dtype
 *                   out_dtype; rows pos0[b]/m .. pos0[b]/m + floor(T/m) - 1 are written.
 * B == 0 or T < m is a no-op. Errors: CSA_ERR_ARG for bad sizes, strides or dtypes, a NULL tensor,
 * a missing halo with pos0 given, or (pos0 NULL) floor(T/m) > n_cap.
 */
int csa_compress(int B, int T, const int64_t* pos0, int m, int c, int in_dtype,
                 const void* ca, const void* za, const void* cb, const void* zb,
                 int64_t ld, int64_t seq_stride,
                 const void* halo_cb, const void* halo_zb, int64_t halo_ld, int64_t halo_seq_stride,
                 const float* bias_a, const float* bias_b,
                 void* entries, int64_t entries_seq_stride, int64_t n_cap, int out_dtype,
                 void* stream);

/*
 * HCA compressor ("Anatomy of a Frontier Model", section "The attention: compress, then select",
 * bullet "Heavily Compressed Attention (HCA)": every 128 tokens become one entry, without overlap).
 * The pages name no other pooling; read as the CSA compressor's pooling over the entry's own block:
 * for each sequence b, complete block of this call (entry i = pos0[b]/m + e, e < floor(T/m)) and
 * channel j,
 *   entries[i, j] = softmax_r(z[i*m+r, j] + bias[r, j]) . c[i*m+r, j]        (r < m)
 *   c, z      [B, T, c] views: token stride `ld`, sequence stride `seq_stride`, channel stride 1;
 *             dtype in_dtype (F32 or BF16).
 *   pos0      device int64 [B] (NULL: all 0): multiples of m with pos0[b]/m + floor(T/m) <= n_cap.
 *   bias      [m, c] float32.
 *   entries   [B, n_cap, c] (row stride c, sequence stride entries_seq_stride), dtype out_dtype.
 * Requires 1 <= m <= 128; no halo is needed. Errors as csa_compress.
 */
int csa_hca_compress(int B, int T, const int64_t* pos0, int m, int c, int in_dtype,
                     const void* cv, const void* z, int64_t ld, int64_t seq_stride,
                     const float* bias, void* entries, int64_t entries_seq_stride, int64_t n_cap,
                     int out_dtype, void* stream);

/*
 * Steps 2+3 — lightning indexer fused with top-k ("Anatomy of a Frontier Model", bullet
 * "Compressed Sparse Attention (CSA)": 64 heads x 128 dims, top 1,024 / 512; "The Exchange Rates
 * of a Million Tokens", section 3: ReLU-gated dot products, top-k).
 *   s[t, i] = sum_h w[h] * max(0, q_idx[t, h, :] . keys[i, :])   for i < n_vis(q_pos[b] + t)
 *   out_idx[t] = the top_k entries by (s descending, i ascending), stored ascending and padded
 *   with -1 when fewer than top_k are visible.
 *   q_pos    device int64 [B] (NULL: all 0): row t of sequence b sits at q_pos[b] + t.
 *   q_idx    [B, T, H_I, D_I]: token stride q_ld, sequence stride q_seq_stride, heads D_I apart.
 *            MXFP4: codes [B, T, H_I, D_I/2] bytes and q_scale [B, T, H_I, D_I/32], both
 *            contiguous (q_ld / q_seq_stride must be 0).
 *   w        float32 head weights: [H_I] shared when w_ld == 0, else row (b*T + t) at w + row*w_ld.
 *   keys     [B, n_cap, D_I] (row stride D_I, sequence stride keys_seq_stride); MXFP4: codes
 *            [B, n_cap, D_I/2] contiguous (16-byte aligned) plus k_scale [B, n_cap, D_I/32]
 *            (4-byte aligned).
 *   out_idx  [B, T, top_k] int32.  out_score (nullable) [B, T, top_k] the scores of out_idx.
 * The T x n_cap score matrix is not stored for many query rows (fused streaming selection); for
 * few query rows (decode) the scores of every visible entry pass through the workspace.
 * Errors: CSA_ERR_ARG for bad sizes, strides, alignment or a NULL tensor; CSA_ERR_WORKSPACE.
 */
int csa_index_topk(const csa_dims* dims, int B, int T, const int64_t* q_pos, int idx_dtype,
                   const void* q_idx, int64_t q_ld, int64_t q_seq_stride, const void* q_scale,
                   const float* w, int64_t w_ld,
                   const void* keys, int64_t keys_seq_stride, const void* k_scale, int64_t n_cap,
                   int32_t* out_idx, float* out_score,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3 on its own ("Anatomy of a Frontier Model", bullet "Compressed Sparse Attention (CSA)":
 * each query keeps the 1,024 (512) compressed entries the indexer ranks highest), on caller-provided
 * float32 scores: the selection routine of csa_index_topk, exposed so that it can be checked bit
 * for bit.
 *   scores   [R, ld] float32; row r's candidates are columns 0 .. n_valid[r]-1 (clamped to ld).
 *   n_valid  device int32 [R].
 *   out_idx  [R, k] int32, ascending, -1 padded; out_score (nullable) [R, k].
 * Order: score descending (-0 == +0), then column ascending. NaN scores are not supported.
 * Errors: CSA_ERR_ARG for k outside [1, 4096], negative sizes or a NULL tensor; CSA_ERR_WORKSPACE.
 */
int csa_topk_from_scores(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                         int32_t* out_idx, float* out_score,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Step 4 — sparse single-KV-head attention ("Anatomy of a Frontier Model", sections "The
 * skeleton, and what's kept" and "The attention: compress, then select", bullets "A sliding
 * window in every layer" and "An attention sink").
 * For query row t of sequence b at p = q_pos[b] + t and head h, over the key set
 *   S_t = { entries[idx[t, j]] : idx[t, j] >= 0 }  ++  { raw row of position u : u in
 *         [max(0, p - window + 1), p] }
 *   o[t, h] = sum_{v in S_t} exp(l_v - mu) v / (sum_v exp(l_v - mu) [+ exp(sink[h] - mu)]),
 *   l_v = sm_scale * q[t, h] . v,  mu = the largest logit (and sink[h] when given).
 *   q_pos    device int64 [B] (NULL: all 0).
 *   q        [B, T, H, D]: token stride q_ld, sequence stride q_seq_stride, heads D apart.
 *   entries  [B, n_cap, D] (row stride D); idx [B, T, top_k] int32 (values outside [0, n_cap)
 *            are skipped).
 *   kv_raw   [B, raw_len, D]: row stride raw_ld, sequence stride raw_seq_stride; row r of sequence
 *            b holds position raw_pos[b] + r (raw_pos: device int64 [B], NULL: all 0; values may
 *            be negative). The rows must cover every query's window: window positions outside
 *            [raw_pos[b], raw_pos[b] + raw_len) are not read and drop out of the key set.
 *   sink     nullable float32 [H].
 *   out      [B, T, H, D] contiguous, out_dtype F32 or BF16.
 * Errors: CSA_ERR_ARG for bad sizes, strides, alignment or a NULL tensor; CSA_ERR_UNSUPPORTED for
 * D > 1024; CSA_ERR_WORKSPACE.
 */
int csa_sparse_attn(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
                    const void* q, int64_t q_ld, int64_t q_seq_stride,
                    const void* entries, int64_t entries_seq_stride, int64_t n_cap,
                    const int32_t* idx,
                    const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                    const int64_t* raw_pos, int64_t raw_len,
                    const float* sink,
                    void* out, int out_dtype,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * HCA attention ("Anatomy of a Frontier Model", bullet "Heavily Compressed Attention (HCA)":
 * queries attend to all entries densely; bullets "A sliding window in every layer" and "An
 * attention sink"): csa_sparse_attn with the selection replaced by every entry visible to the
 * query, in order: S_t = { entries[i] : i < min(floor((p+1)/m), n_cap) } ++ the window rows.
 * Arguments as csa_sparse_attn, without idx; dims->m is the HCA block (128) and dims->top_k is not
 * used. Workspace: csa_workspace_size(CSA_OP_DENSE_ATTN, dims, B, T, n_cap, ...).
 */
int csa_dense_attn(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
                   const void* q, int64_t q_ld, int64_t q_seq_stride,
                   const void* entries, int64_t entries_seq_stride, int64_t n_cap,
                   const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                   const int64_t* raw_pos, int64_t raw_len,
                   const float* sink,
                   void* out, int out_dtype,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * QK-norm and partial RoPE ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE":
 * queries and compressed entries are RMS-normalised per head, RoPE turns only the last 64 of the 512
 * dims, and each output is turned back by its own position so that only relative position remains).
 * For B x R rows of H head vectors of D dims (dtype F32 or BF16, x and y alike), row r of sequence
 * b at x + b*x_seq_stride + r*x_ld + h*D (elements), at position pos0[b] + pos_off + r*pos_step
 * (pos0: device int64 [B], NULL: all 0; pos_off, pos_step: host values):
 *   gamma != NULL:  v = v / sqrt(mean(v^2) + eps) * gamma          (gamma [D] fp32, device)
 *   rope_dims > 0:  the last rope_dims dims, in adjacent pairs (2i, 2i+1) of that slice, turn by
 *                   the angle pos * rope_theta^(-2i/rope_dims): (a, b) -> (a cos - b sin,
 *                   a sin + b cos); inverse != 0 turns by the negative angle (no norm then).
 * y may equal x (in place, same strides); other overlaps are undefined. Norm in fp32, angles and
 * their sine/cosine in fp64. Errors: CSA_ERR_ARG for negative sizes, odd D, rope_dims odd or
 * outside [0, D], D > 4096, a missing pointer, rope_theta <= 0 with rope_dims > 0, or gamma with
 * inverse. Asynchronous on `stream`; allocates nothing.
 */
int csa_norm_rope(int B, int R, int H, int D, int dtype,
                  const void* x, int64_t x_ld, int64_t x_seq_stride,
                  void* y, int64_t y_ld, int64_t y_seq_stride,
                  const float* gamma, float eps,
                  int rope_dims, float rope_theta, const int64_t* pos0, int64_t pos_off,
                  int64_t pos_step, int inverse, void* stream);

/*
 * The pages' compressed-entry record ("Anatomy of a Frontier Model", section "The KV cache,
 * recomputed": 512 numbers, 448 in FP8 and the 64 RoPE dims in BF16, with seven one-byte UE8M0
 * scales and a pad byte, 584 bytes; bullet "QK-norm and partial RoPE": the 448 position-free dims
 * are the FP8 ones). Byte layout: e4m3 codes of dims 0..447 | bf16 of dims 448..511, little-endian |
 * scale exponents E_0..E_6 | 0. Dims 64g..64g+63 have scale 2^(E_g - 127), the smallest power of two
 * that keeps the group's largest magnitude within 448 (127 for an all-zero group); codes are OCP
 * E4M3, rounded to nearest with ties to even, the sign bit from the value's sign.
 *
 * csa_entry_pack: entries [B, N, 512] (dtype F32 or BF16; row n of sequence b at
 * b*seq_stride + n*ld elements, ld >= 512) -> records (row n of sequence b at
 * b*records_seq_stride + n*584 bytes; 8-byte aligned). F32 RoPE dims are rounded to bf16 (RNE).
 * CSA_ERR_ARG on negative sizes, a NULL pointer, small strides or misalignment.
 */
int csa_entry_pack(int B, int N, int in_dtype, const void* entries, int64_t ld, int64_t seq_stride,
                   void* records, int64_t records_seq_stride, void* stream);

/*
 * MXFP4 quantisation (OCP Microscaling Formats v1.0) of R rows of D values, the storage of the FP4
 * indexer's keys and queries ("Anatomy of a Frontier Model", sections "The KV cache, recomputed" and
 * "Precision: FP8 everywhere, FP4 experts"). Per block of 32 consecutive values: shared exponent
 * X = floor(log2(max |x|)) - 2 clamped to [-127, 127], stored as the byte X + 127; each value
 * x / 2^X rounded to the nearest e2m1 value (ties to the even code, magnitudes past 6 saturate to 6),
 * sign bit = sign of x; codes hold two values per byte, the even-indexed one in the low nibble.
 *   x       [R, D] of dtype (F32 or BF16), row stride ld elements (ld >= D); D % 32 == 0.
 *   codes   [R, D/2] bytes, contiguous, 4-byte aligned.  scales [R, D/32] bytes, contiguous.
 * Inf / NaN inputs are not supported. Errors: CSA_ERR_ARG for bad sizes, a NULL or misaligned tensor.
 */
int csa_mxfp4_quantize(int64_t R, int D, int dtype, const void* x, int64_t ld, void* codes, void* scales,
                       void* stream);

/*
 * csa_sparse_attn over an entry cache of 584-byte records (see csa_entry_pack): as
 * csa_sparse_attn, with `records` [B, n_cap, 584] bytes (16-byte aligned base, sequence stride in
 * bytes, a multiple of 8) in place of the entries; D must be 512. q and kv_raw keep in_dtype. The
 * attention sees each entry's stored values exactly (FP8 times its scale, bf16 RoPE dims). The
 * workspace is the one csa_workspace_size gives for CSA_OP_SPARSE_ATTN.
 */
int csa_sparse_attn_fp8(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
                        const void* q, int64_t q_ld, int64_t q_seq_stride,
                        const void* records, int64_t records_seq_stride, int64_t n_cap,
                        const int32_t* idx,
                        const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                        const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out,
                        int out_dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_dense_attn over a cache of 584-byte records (the HCA layers keep the same entry format as the
 * CSA layers in "Anatomy of a Frontier Model", section "The KV cache, recomputed"): as
 * csa_dense_attn with `records` [B, n_cap, 584] bytes in place of the entries (16-byte aligned,
 * sequence stride in bytes, a multiple of 8); D must be 512. Workspace: CSA_OP_DENSE_ATTN.
 */
int csa_dense_attn_fp8(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
                       const void* q, int64_t q_ld, int64_t q_seq_stride,
                       const void* records, int64_t records_seq_stride, int64_t n_cap,
                       const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                       const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out,
                       int out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Weights of one CSA layer (device pointers). */
typedef struct csa_weights {
  /* Fused projection, [n_tot, d_model] row-major (one output column per row), dtype of x, with
     n_tot = 4D + 4D_I + H*D + H_I*D_I + D and rows in this order:
     ca | za | cb | zb (D each) | ica | iza | icb | izb (D_I each) | q (H*D) | q_I (H_I*D_I) | kv (D). */
  const void* w_proj;
  const float* bias_a;   /* [m, D]   */
  const float* bias_b;   /* [m, D]   */
  const float* ibias_a;  /* [m, D_I] */
  const float* ibias_b;  /* [m, D_I] */
  const float* w_head;   /* [H_I]    */
  const float* sink;     /* nullable [H] */
  /* QK-norm and partial RoPE ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE"),
     off when gamma_q, gamma_kv are NULL and rope_dims is 0. When on, the queries (at their
     positions), the chunk's raw KV (at its token positions) and the new entries (entry i at
     position (i+1)*m - 1) are RMS-normalised and rotated before the attention, and the output is
     rotated back by the query position (see csa_norm_rope). The caches' context rows are read as
     stored, i.e. already normalised and rotated. */
  const float* gamma_q;  /* nullable [D]: norm gain of the query heads (NULL: no query norm)     */
  const float* gamma_kv; /* nullable [D]: norm gain of entries and raw KV (NULL: no such norm)    */
  float norm_eps;        /* eps of both norms                                                     */
  int32_t rope_dims;     /* trailing dims turned by RoPE (64), 0: none; even, <= D                */
  float rope_theta;      /* RoPE base (10000), > 0 when rope_dims > 0                             */
} csa_weights;

/*
 * csa_sparse_attn with the layer's QK-norm and partial RoPE ("Anatomy of a Frontier Model", bullet
 * "QK-norm and partial RoPE"; the forms of csa_norm_rope): the query heads are RMS-normalised with
 * gain w->gamma_q (NULL: no norm, eps w->norm_eps) and their last w->rope_dims dims turned by RoPE at
 * the row's position before the logits, and each head's output is turned back by that position; the
 * entries and raw KV are read as stored (already normalised and rotated). For a decode over caches the
 * caller keeps itself. w->sink is the attention sink (nullable); the other fields of w are not read.
 * Where the attention kernel takes the options (bf16 queries on its matrix-core path, a 16-byte aligned
 * gain, and the rotation table and gain fit its LDS) they cost no pass of their own; otherwise the query
 * is normalised into the workspace and the output turned back in place. Arguments otherwise as csa_sparse_attn. Workspace:
 * csa_workspace_size(CSA_OP_SPARSE_ATTN_QK, dims, B, T, n_cap, 0, in_dtype). Errors as csa_sparse_attn,
 * and those of csa_norm_rope for the options.
 */
int csa_sparse_attn_qk(const csa_dims* dims, const csa_weights* w, int B, int T, const int64_t* q_pos,
                       int in_dtype, const void* q, int64_t q_ld, int64_t q_seq_stride,
                       const void* entries, int64_t entries_seq_stride, int64_t n_cap, const int32_t* idx,
                       const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                       const int64_t* raw_pos, int64_t raw_len, void* out, int out_dtype,
                       void* ws, size_t ws_bytes, void* stream);

/* Caches the layer reads and extends (device pointers, all of the activation dtype). Sequence b's
   chunk starts at position pos0[b] (see csa_forward). */
typedef struct csa_cache {
  void* entries;         /* [B, n_cap, D]: rows < pos0[b]/m are the context; new rows appended   */
  void* keys;            /* [B, n_cap, D_I] indexer keys, same row numbering                     */
  int64_t n_cap;
  void* win;             /* [B, win_cap, D] raw KV: row r of sequence b = position
                            pos0[b] - (window-1) + r. Rows [0, window-1) hold the context's last raw
                            tokens (only those at positions >= 0 are read); rows
                            [window-1, window-1+T) are written.                                   */
  int64_t win_cap;
  const void* halo;      /* [B, m, 2D + 2D_I] cb | zb | icb | izb of block pos0[b]/m - 1; required
                            when pos0 is given (rows of sequences at 0 are not read), may be NULL
                            when pos0 is NULL                                                     */
  void* halo_out;        /* nullable [B, m, 2D + 2D_I]: receives this chunk's last block (needs
                            T % m == 0), i.e. the next chunk's halo                               */
  int32_t entry_fmt;     /* 0: entries are rows of the activation dtype; 1: 584-byte FP8 records
                            [B, n_cap, 584] (see csa_entry_pack; D = 512, bf16 layer): new entries
                            are packed and the attention reads the records                        */
  int32_t key_fmt;       /* 0: keys are rows of the activation dtype; 1: MXFP4 indexer ("Anatomy of a
                            Frontier Model", "The KV cache, recomputed": 128 FP4 values and a scale
                            byte per 32; "Precision: FP8 everywhere, FP4 experts": the indexer's
                            query-key product in FP4): keys holds the e2m1 codes [B, n_cap, D_I/2]
                            (16-byte aligned, contiguous) and key_scales the e8m0 scales
                            [B, n_cap, D_I/32] (4-byte aligned); new keys are quantised from their stored values (see
                            csa_mxfp4_quantize), the chunk's indexer queries likewise, and the
                            indexer runs on the MXFP4 operands                                      */
  void* key_scales;      /* [B, n_cap, D_I/32] when key_fmt = 1, else unused                       */
} csa_cache;

/* Decode state of B sequences (device pointers, activation dtype unless stated). */
typedef struct csa_decode_state {
  void* entries;         /* [B, n_cap, D] rows, or [B, n_cap, 584] FP8 records when entry_fmt = 1  */
  int32_t entry_fmt;     /* 0: rows of the activation dtype, 1: FP8 records (see csa_entry_pack)    */
  void* keys;            /* [B, n_cap, D_I] indexer keys (CSA only)                                  */
  int64_t n_cap;
  void* win;             /* [B, window, D] ring of raw KV: position p in row p % window              */
  void* block;           /* CSA: [B, 2m, 4D + 4D_I] compressor inputs ca|za|cb|zb (D each) and the
                            indexer's ica|iza|icb|izb (D_I each); token r of block i sits in row
                            (i % 2)*m + r, so the previous block's rows stay in the other half.
                            HCA: [B, m, 2D], c | z of the current block's tokens (row p % m).       */
  int32_t key_fmt;       /* 0: keys of the activation dtype; 1: MXFP4 (see csa_cache.key_fmt): keys
                            = codes [B, n_cap, D_I/2], key_scales [B, n_cap, D_I/32]; a completed
                            block's key is quantised from its stored value, and each step's q_idx
                            (given in the activation dtype) is quantised before the indexer         */
  void* key_scales;
} csa_decode_state;

/*
 * One decode step of B sequences, sequence b at its own position pos[b] (the layer of "Anatomy of a
 * Frontier Model", "The attention: compress, then select", run token by token). One launch appends
 * every sequence's token: its compressor inputs go to block row ((pos/m) % 2)*m + pos % m and its
 * raw KV (normalised and rotated at pos when the weights carry QK-norm / RoPE) to window row
 * pos % window; when the token completes its block ((pos+1) % m == 0) entry i = (pos+1)/m - 1 and
 * its indexer key are pooled from the block and the previous one (the CSA pooling over both),
 * normalised and rotated at pos when on, and stored (packed into a record when entry_fmt = 1).
 * Then the query (normalised and rotated at pos when on) is indexed against the floor((pos+1)/m)
 * visible entries, the top-k are selected, and the attention runs over them plus the window
 * [max(0, pos-window+1), pos]; the output is rotated back by pos when RoPE is on.
 *   pos    device int64 [B] (required): pos[b] >= 0 with (pos[b]+1)/m <= n_cap.
 *   q      [B, H, D], q_idx [B, H_I, D_I], kv [B, D], comp [B, 4D + 4D_I] (columns as in block),
 *          each sequence contiguous (sequence strides H*D, H_I*D_I, D, 4D + 4D_I).
 *   w      the layer weights: bias_a/bias_b, ibias_a/ibias_b, w_head, sink, the QK-norm / RoPE
 *          fields (w_proj is not used: the step takes projected rows).
 *   out    [B, H, D] (out_dtype); out_idx nullable [B, top_k].
 * Before a sequence's first step the caller fills its state's context: the entries and keys of the
 * floor(pos/m) complete blocks before pos, the window rows of positions pos-window+1 .. pos-1, and
 * the block rows of the previous block and of the current block's tokens before pos; the calls then
 * go pos, pos+1, ... Workspace: csa_workspace_size(CSA_OP_DECODE_STEP, dims, B, 1, n_cap, 0, dtype).
 * Errors: CSA_ERR_ARG for bad sizes, pointers, a NULL pos, records with D != 512 or fp32 entries.
 */
int csa_decode_step(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype,
                    const void* q, const void* q_idx, const void* kv, const void* comp,
                    const csa_decode_state* state, void* out, int out_dtype, int32_t* out_idx,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csa_decode_step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Arguments and results are those of
 * csa_decode_step, without the workspace: the step's scratch is an array of
 * CSA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on (from the first call on
 * that device until the process ends). The call allocates nothing. Every call on a GPU shares that
 * GPU's array, so calls that overlap on one GPU (other streams, other threads) race; calls in order
 * on one stream are safe (each step writes before it reads whatever of the scratch it uses).
 * Errors: those of csa_decode_step; CSA_ERR_WORKSPACE when the step needs more scratch than
 * CSA_STATIC_SCRATCH_BYTES (csa_workspace_size(CSA_OP_DECODE_STEP, ...) gives the need);
 * CSA_ERR_HIP when the array's device address cannot be taken.
 */
#define CSA_STATIC_SCRATCH_BYTES (64u << 20)
int csa_decode_step_noalloc(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos,
                            int dtype, const void* q, const void* q_idx, const void* kv,
                            const void* comp, const csa_decode_state* state, void* out, int out_dtype,
                            int32_t* out_idx, void* stream);

/*
 * One decode step of an HCA layer ("Anatomy of a Frontier Model", bullet "Heavily Compressed
 * Attention (HCA)": blocks of m = 128 tokens pooled without overlap, attention over every visible
 * entry plus the window), sequence b at pos[b], over a decode state whose `block` is [B, m, 2D]:
 * the c | z compressor inputs of the current block's tokens (keys unused). The token's c|z row goes
 * to block row pos % m and its raw KV to window row pos % window; when it completes the block,
 * entry (pos+1)/m - 1 is pooled from the block's rows with weights bias_a [m, D] (normalised and
 * rotated at pos, packed into a record when entry_fmt = 1). Then the query (normalised and rotated
 * at pos when on) attends to the floor((pos+1)/m) entries and the window; the output is rotated
 * back by pos when RoPE is on.
 *   pos [B] device int64 (required); q [B, H, D], kv [B, D], comp [B, 2D]; out [B, H, D].
 * Workspace: csa_workspace_size(CSA_OP_HCA_DECODE_STEP, dims, B, 1, n_cap, 0, dtype). dims->top_k
 * and the indexer sizes are not used. Errors as csa_decode_step.
 */
int csa_hca_decode_step(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos,
                        int dtype, const void* q, const void* kv, const void* comp,
                        const csa_decode_state* state, void* out, int out_dtype, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * The layer's fused input projection C = A W^T on the library's own kernels: the GEMM csa_forward
 * falls back to when hipBLASLt declines a shape (the pages give no projection; one dense product over
 * the concatenated weights makes every per-token vector the layer reads, see csa_weights.w_proj).
 *   A  [M, K] of in_dtype (F32 or BF16), row stride lda >= K elements.
 *   Wt [N, K] of in_dtype, row stride ldb >= K (one output column per row).
 *   C  [M, N] of out_dtype (F32 or BF16), row stride ldc >= N; fp32 accumulation, bf16 out rounded
 *      to nearest even.
 * BF16 inputs with K % 64 == 0, lda, ldb multiples of 8 and 16-byte aligned A, Wt run the matrix-core
 * kernel (128 x 128 tiles); everything else a one-output-per-thread kernel. Device pointers,
 * asynchronous on `stream`. Errors: CSA_ERR_ARG for negative sizes, small strides or NULL pointers.
 */
int csa_projection_gemm(int M, int N, int K, int in_dtype, const void* A, int64_t lda, const void* Wt, int64_t ldb,
                        void* C, int64_t ldc, int out_dtype, void* stream);

/*
 * The whole layer ("Anatomy of a Frontier Model", section "The attention: compress, then select":
 * compress, then select, then attend; "The Exchange Rates of a Million Tokens", section 3) for a
 * chunk of T tokens per sequence, sequence b at positions pos0[b] .. pos0[b]+T-1: projection
 * (x @ w_proj^T), both compressors (entries and indexer keys, appended at rows pos0[b]/m ..),
 * indexer + top-k, sparse attention over the selected entries and the window.
 *   pos0     device int64 [B] (NULL: every sequence starts at 0): multiples of m with
 *            (pos0[b] + T)/m <= n_cap.
 *   x        [B, T, d_model] contiguous, dtype F32 or BF16 (also the cache/projection dtype).
 *   cache    see csa_cache; window - 1 + T <= win_cap.
 *   out      [B, T, H, D] contiguous, out_dtype F32 or BF16.
 *   out_idx  nullable [B, T, top_k]: receives the selected entries.
 * Errors: CSA_ERR_ARG for bad sizes, pointers, a missing halo with pos0 given; CSA_ERR_UNSUPPORTED
 * for QK-norm / RoPE or records where one entry's channel vectors do not fit one wave
 * (D / 8 > 64 in bf16); CSA_ERR_WORKSPACE.
 */
int csa_forward(const csa_dims* dims, const csa_weights* w, int B, int T, const int64_t* pos0,
                int d_model, int dtype, const void* x, const csa_cache* cache,
                void* out, int out_dtype, int32_t* out_idx,
                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
