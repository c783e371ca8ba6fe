// The C ABI: argument validation (host only, before any HIP call), workspace carving and dispatch
// to the kernels. Declarations and the meaning of every argument are in include/csa.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "kernels.h"

namespace csa {

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err.clear();
    return CSA_OK;
  }
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int esize(int dt) { return dt == CSA_F32 ? 4 : 2; }

bool is_act_dtype(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }

constexpr int kMaxTopK = 4096;

__global__ void copy_rows_kernel(int rows, int cols, int esz, const uint8_t* src, int64_t src_ld, int64_t src_seq,
                                 uint8_t* dst, int64_t dst_ld, int64_t dst_seq) {
  const int b = blockIdx.y;
  const int64_t nbytes = (int64_t)rows * cols * esz;
  const int64_t rowb = (int64_t)cols * esz;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nbytes; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / rowb, c = i % rowb;
    dst[(b * dst_seq + r * dst_ld) * esz + c] = src[(b * src_seq + r * src_ld) * esz + c];
  }
}

}  // namespace

hipError_t launch_copy_rows(int B, int rows, int cols, int esz, const void* src, int64_t src_ld, int64_t src_seq,
                            void* dst, int64_t dst_ld, int64_t dst_seq, hipStream_t s) {
  if (B == 0 || rows == 0 || cols == 0) return hipSuccess;
  const int64_t nbytes = (int64_t)rows * cols * esz;
  unsigned gx = (unsigned)ceil_div(nbytes, 256);
  if (gx > 4096) gx = 4096;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(gx, (unsigned)B), dim3(256), 0, s, rows, cols, esz,
                     static_cast<const uint8_t*>(src), src_ld, src_seq, static_cast<uint8_t*>(dst), dst_ld, dst_seq);
  return hipGetLastError();
}

hipError_t allow_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = done.find(key);
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done[key] = bytes;
  return e;
}

}  // namespace csa

using namespace csa;

namespace {

// uses_topk = false: the dense (HCA) attention, which ignores top_k
int check_dims(const csa_dims* d, bool uses_topk = true) {
  if (!d) return fail(CSA_ERR_ARG, "dims is NULL");
  if (d->m < 1 || d->m > compress_max_m()) return fail(CSA_ERR_ARG, "m=%d out of [1, %d]", d->m, compress_max_m());
  if (d->D < 1 || d->H < 1 || d->H_I < 1 || d->D_I < 1) return fail(CSA_ERR_ARG, "dims must be positive");
  if (uses_topk && (d->top_k < 1 || d->top_k > kMaxTopK))
    return fail(CSA_ERR_ARG, "top_k=%d out of [1, %d]", d->top_k, kMaxTopK);
  if (d->window < 1) return fail(CSA_ERR_ARG, "window=%d must be >= 1", d->window);
  if (!(d->sm_scale >= 0.f) || std::isinf(d->sm_scale)) return fail(CSA_ERR_ARG, "sm_scale must be finite and >= 0");
  return CSA_OK;
}

float scale_of(const csa_dims* d) { return d->sm_scale > 0.f ? d->sm_scale : 1.0f / std::sqrt((float)d->D); }

IndexArgs make_index_args(const csa_dims* d, int B, int T, int64_t q_pos0, int idx_dtype, const void* q_idx,
                          int64_t q_ld, int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld,
                          const void* keys, int64_t keys_seq_stride, const void* k_scale, int64_t n_cap,
                          int32_t* out_idx, float* out_score) {
  IndexArgs a{};
  a.B = B;
  a.T = T;
  a.q_pos0 = q_pos0;
  a.m = d->m;
  a.H_I = d->H_I;
  a.D_I = d->D_I;
  a.k = d->top_k;
  a.idx_dtype = idx_dtype;
  a.q = q_idx;
  a.q_ld = q_ld;
  a.q_seq_stride = q_seq_stride;
  a.q_scale = static_cast<const uint8_t*>(q_scale);
  a.w = w;
  a.w_ld = w_ld;
  a.keys = keys;
  a.keys_seq_stride = keys_seq_stride;
  a.k_scale = static_cast<const uint8_t*>(k_scale);
  a.n_cap = n_cap;
  a.out_idx = out_idx;
  a.out_score = out_score;
  if (idx_dtype == CSA_MXFP4) {  // contiguous MXFP4 tensors, strides in code bytes
    a.q_ld = (int64_t)d->H_I * d->D_I / 2;
    a.q_seq_stride = (int64_t)T * a.q_ld;
    a.keys_seq_stride = n_cap * d->D_I / 2;
  }
  return a;
}

// AttnArgs with contiguous strides, for workspace sizing (the real call may need less).
AttnArgs sizing_attn(const csa_dims* d, int B, int T, int dtype) {
  AttnArgs a{};
  a.B = B;
  a.T = T;
  a.H = d->H;
  a.D = d->D;
  a.k = d->top_k;
  a.W = d->window;
  a.in_dtype = dtype;
  a.out_dtype = CSA_F32;
  a.q_ld = (int64_t)d->H * d->D;
  a.q_seq_stride = (int64_t)T * a.q_ld;
  a.entries_seq_stride = 0;
  a.raw_ld = d->D;
  a.raw_seq_stride = 0;
  return a;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CSA_OK;
  if (!ws) return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(ws, 256)) return fail(CSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return CSA_OK;
}

int64_t n_tot_of(const csa_dims* d) {
  return 4LL * d->D + 4LL * d->D_I + (int64_t)d->H * d->D + (int64_t)d->H_I * d->D_I + d->D;
}

int validate_index(const csa_dims* d, int B, int T, int64_t q_pos0, int idx_dtype, const void* q_idx, int64_t q_ld,
                   int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld, const void* keys,
                   int64_t keys_seq_stride, const void* k_scale, int64_t n_cap, const int32_t* out_idx) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (q_pos0 < 0) return fail(CSA_ERR_ARG, "q_pos0 must be >= 0");
  if (n_cap < 0 || n_cap > 0x7FFFFFFFLL) return fail(CSA_ERR_ARG, "n_cap out of range");
  if (idx_dtype != CSA_F32 && idx_dtype != CSA_BF16 && idx_dtype != CSA_MXFP4)
    return fail(CSA_ERR_ARG, "unknown idx_dtype %d", idx_dtype);
  if ((int64_t)B * T == 0) return CSA_OK;
  if (!q_idx || !w || !out_idx || (!keys && n_cap > 0)) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (w_ld < 0) return fail(CSA_ERR_ARG, "w_ld must be >= 0");
  if (w_ld > 0 && w_ld < d->H_I) return fail(CSA_ERR_ARG, "w_ld must be 0 or >= H_I");
  if (idx_dtype == CSA_MXFP4) {
    if (d->D_I % 32) return fail(CSA_ERR_ARG, "MXFP4 needs D_I %% 32 == 0");
    if (!q_scale || (!k_scale && n_cap > 0)) return fail(CSA_ERR_ARG, "MXFP4 needs q_scale and k_scale");
    if (q_ld != 0 || q_seq_stride != 0) return fail(CSA_ERR_ARG, "MXFP4 q must be contiguous (q_ld = q_seq_stride = 0)");
    if (keys_seq_stride != 0 && keys_seq_stride != n_cap * d->D_I / 2)
      return fail(CSA_ERR_ARG, "MXFP4 keys must be contiguous");
    if (!aligned(q_idx, 16) || (keys && !aligned(keys, 16))) return fail(CSA_ERR_ARG, "MXFP4 codes must be 16-byte aligned");
  } else {
    if (q_ld < (int64_t)d->H_I * d->D_I) return fail(CSA_ERR_ARG, "q_ld < H_I*D_I");
    if (B > 1 && q_seq_stride < (int64_t)T * q_ld) return fail(CSA_ERR_ARG, "q_seq_stride too small");
    if (B > 1 && keys_seq_stride < n_cap * d->D_I) return fail(CSA_ERR_ARG, "keys_seq_stride too small");
    const size_t a = esize(idx_dtype) == 2 ? 16 : 4;
    if (!aligned(q_idx, a) || (keys && !aligned(keys, a))) return fail(CSA_ERR_ARG, "misaligned q_idx/keys");
    if (idx_dtype == CSA_BF16 && d->H_I == 64 && d->D_I == 128 &&
        ((q_ld % 8) || (q_seq_stride % 8) || (keys_seq_stride % 8)))
      return fail(CSA_ERR_ARG, "bf16 indexer strides must be multiples of 8 elements");
  }
  return CSA_OK;
}

// Workspace of csa_decode_step: the rotated query, one compressed entry
// per sequence (records), the selected indices, and the index / attention scratch.
struct DecodeWs {
  size_t win, q, ent, idx, scratch, total;
};
DecodeWs decode_ws(const csa_dims* d, int B, int64_t n_cap, int dtype) {
  const size_t es = dtype == CSA_F32 ? 4 : 2;
  DecodeWs w{};
  w.win = 0;  // the attention reads the window straight from the state's ring
  w.q = w.win;
  w.ent = w.q + align256((size_t)B * d->H * d->D * es);
  w.idx = w.ent + align256((size_t)B * d->D * es);
  w.scratch = w.idx + align256((size_t)B * d->top_k * 4);
  IndexArgs ia = make_index_args(d, B, 1, 0, dtype, nullptr, 0, 0, nullptr, nullptr, 0, nullptr, 0, nullptr, n_cap,
                                 nullptr, nullptr);
  const size_t iw = index_topk_workspace(ia);
  const size_t aw = attn_workspace(sizing_attn(d, B, 1, dtype));
  w.total = w.scratch + align256(iw > aw ? iw : aw);
  return w;
}

// Workspace of csa_hca_decode_step: the rotated query, one compressed entry per sequence (records),
// the dense attention's split partials.
DecodeWs hca_decode_ws(const csa_dims* d, int B, int64_t n_cap, int dtype) {
  const size_t es = dtype == CSA_F32 ? 4 : 2;
  DecodeWs w{};
  w.win = 0;
  w.q = 0;
  w.ent = align256((size_t)B * d->H * d->D * es);
  w.idx = w.ent + align256((size_t)B * d->D * es);
  w.scratch = w.idx;
  AttnArgs a = sizing_attn(d, B, 1, dtype);
  a.dense = 1;
  a.m = d->m;
  a.k = 0;
  a.n_cap = n_cap;
  a.q_pos0 = n_cap * d->m;  // every entry visible: the most keys a row can have
  w.total = w.scratch + align256(attn_workspace(a));
  return w;
}

int attn_call(const char* name, bool dense, const csa_dims* dims, int B, int T, int64_t q_pos0, int in_dtype,
              const void* q, int64_t q_ld, int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride,
              int64_t n_cap, const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
              int64_t raw_pos0, int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws,
              size_t ws_bytes, void* stream, int entry_fmt = 0, int64_t raw_ring = 0) {
  int rc = check_dims(dims, !dense);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (q_pos0 < 0 || n_cap < 0 || raw_len < 0) return fail(CSA_ERR_ARG, "negative position or size");
  if (dims->D > 1024) return fail(CSA_ERR_UNSUPPORTED, "D > 1024");
  if ((int64_t)B * T == 0) return CSA_OK;
  if (!q || (!dense && !idx) || !kv_raw || !out || (!entries && n_cap > 0))
    return fail(CSA_ERR_ARG, "NULL tensor pointer");
  const int64_t H = dims->H, D = dims->D;
  if (q_ld < H * D) return fail(CSA_ERR_ARG, "q_ld < H*D");
  if (B > 1 && q_seq_stride < (int64_t)T * q_ld) return fail(CSA_ERR_ARG, "q_seq_stride too small");
  if (entry_fmt && D != 512) return fail(CSA_ERR_ARG, "entry records hold D = 512");
  if (B > 1 && entries_seq_stride < n_cap * (entry_fmt ? (int64_t)kEntryRecordBytes : D))
    return fail(CSA_ERR_ARG, "entries_seq_stride too small");
  if (raw_ld < D) return fail(CSA_ERR_ARG, "raw_ld < D");
  if (B > 1 && raw_seq_stride < raw_len * raw_ld) return fail(CSA_ERR_ARG, "raw_seq_stride too small");
  const int64_t need_lo = q_pos0 - dims->window + 1 > 0 ? q_pos0 - dims->window + 1 : 0;
  const int64_t need_hi = q_pos0 + T - 1;
  if (raw_ring > 0 && (T != 1 || raw_ring < dims->window))
    return fail(CSA_ERR_ARG, "a raw KV ring serves one query row and holds at least the window");
  if (raw_pos0 > need_lo || raw_pos0 + raw_len - 1 < need_hi)
    return fail(CSA_ERR_ARG, "kv_raw rows [%lld, %lld] do not cover the windows [%lld, %lld]", (long long)raw_pos0,
                (long long)(raw_pos0 + raw_len - 1), (long long)need_lo, (long long)need_hi);
  const size_t al = esize(in_dtype) == 2 ? 16 : 4;
  if (!aligned(q, al) || !aligned(kv_raw, al) || (entries && !aligned(entries, entry_fmt ? 16 : al)))
    return fail(CSA_ERR_ARG, "misaligned q / entries / kv_raw");
  if (entry_fmt && entries_seq_stride % 8) return fail(CSA_ERR_ARG, "record sequence stride must be a multiple of 8 bytes");
  AttnArgs a{};
  a.B = B;
  a.T = T;
  a.q_pos0 = q_pos0;
  a.H = dims->H;
  a.D = dims->D;
  a.k = dense ? 0 : dims->top_k;
  a.W = dims->window;
  a.scale = scale_of(dims);
  a.dense = dense ? 1 : 0;
  a.m = dims->m;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.q = q;
  a.q_ld = q_ld;
  a.q_seq_stride = q_seq_stride;
  a.entries = entries;
  a.entries_seq_stride = entries_seq_stride;
  a.n_cap = n_cap;
  a.idx = idx;
  a.raw = kv_raw;
  a.raw_ld = raw_ld;
  a.raw_seq_stride = raw_seq_stride;
  a.raw_pos0 = raw_pos0;
  a.raw_len = raw_len;
  a.sink = sink;
  a.out = out;
  a.entry_fmt = entry_fmt;
  a.raw_ring = raw_ring;
  rc = check_ws(ws, ws_bytes, attn_workspace(a));
  if (rc) return rc;
  return hip_status(launch_attn(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), name);
}

}  // namespace

extern "C" {

int csa_version(void) { return 1; }

const char* csa_last_error(void) { return g_err.c_str(); }

int csa_workspace_size(int op, const csa_dims* dims, int B, int T, int64_t n_cap, int d_model, int idx_dtype,
                       int64_t* bytes) {
  if (!bytes) return fail(CSA_ERR_ARG, "bytes is NULL");
  *bytes = 0;
  if (B < 0 || T < 0 || n_cap < 0 || d_model < 0) return fail(CSA_ERR_ARG, "negative size");
  switch (op) {
    case CSA_OP_COMPRESS:
      return CSA_OK;
    case CSA_OP_SPARSE_ATTN: {
      int rc = check_dims(dims);
      if (rc) return rc;
      *bytes = (int64_t)attn_workspace(sizing_attn(dims, B, T, idx_dtype == CSA_F32 ? CSA_F32 : CSA_BF16));
      return CSA_OK;
    }
    case CSA_OP_DENSE_ATTN: {
      int rc = check_dims(dims, false);
      if (rc) return rc;
      AttnArgs a = sizing_attn(dims, B, T, idx_dtype == CSA_F32 ? CSA_F32 : CSA_BF16);
      a.dense = 1;
      a.m = dims->m;
      a.k = 0;
      a.n_cap = n_cap;
      a.q_pos0 = n_cap * dims->m;  // every entry visible: the most keys a row can have
      *bytes = (int64_t)attn_workspace(a);
      return CSA_OK;
    }
    case CSA_OP_DECODE_STEP: {
      int rc = check_dims(dims);
      if (rc) return rc;
      *bytes = (int64_t)decode_ws(dims, B, n_cap, idx_dtype).total;
      return CSA_OK;
    }
    case CSA_OP_HCA_DECODE_STEP: {
      int rc = check_dims(dims, false);
      if (rc) return rc;
      *bytes = (int64_t)hca_decode_ws(dims, B, n_cap, idx_dtype).total;
      return CSA_OK;
    }
    case CSA_OP_TOPK_FROM_SCORES: {
      if (!dims) return fail(CSA_ERR_ARG, "dims is NULL");
      *bytes = (int64_t)topk_workspace(B, n_cap, dims->top_k);
      return CSA_OK;
    }
    case CSA_OP_INDEX_TOPK:
    case CSA_OP_FORWARD: {
      int rc = check_dims(dims);
      if (rc) return rc;
      IndexArgs a = make_index_args(dims, B, T, 0, idx_dtype, nullptr, 0, 0, nullptr, nullptr, 0, nullptr, 0,
                                    nullptr, n_cap, nullptr, nullptr);
      size_t need = index_topk_workspace(a);
      if (op == CSA_OP_FORWARD) {
        const int es = idx_dtype == CSA_F32 ? 4 : 2;
        const size_t at = attn_workspace(sizing_attn(dims, B, T, idx_dtype == CSA_F32 ? CSA_F32 : CSA_BF16));
        size_t scratch = need > at ? need : at;  // index / attention scratch, or the projection's
        if (idx_dtype == CSA_BF16 && scratch < kGemmWorkspace) scratch = kGemmWorkspace;
        const size_t ent_tmp = (size_t)B * (T / dims->m) * dims->D * es;  // new entries before packing
        if (scratch < ent_tmp) scratch = ent_tmp;
        need = align256((size_t)B * T * n_tot_of(dims) * es) + align256((size_t)B * T * dims->top_k * 4) +
               align256(scratch);
      }
      *bytes = (int64_t)need;
      return CSA_OK;
    }
    default:
      return fail(CSA_ERR_ARG, "unknown op %d", op);
  }
}

int csa_compress(int B, int T, int64_t pos0, int m, int c, int in_dtype, const void* ca, const void* za,
                 const void* cb, const void* zb, int64_t ld, int64_t seq_stride, const void* halo_cb,
                 const void* halo_zb, int64_t halo_ld, int64_t halo_seq_stride, const float* bias_a,
                 const float* bias_b, void* entries, int64_t entries_seq_stride, int64_t n_cap, int out_dtype,
                 void* stream) {
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (m < 1 || m > compress_max_m()) return fail(CSA_ERR_ARG, "m=%d out of [1, %d]", m, compress_max_m());
  if (c < 1) return fail(CSA_ERR_ARG, "c must be >= 1");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (pos0 < 0 || pos0 % m) return fail(CSA_ERR_ARG, "pos0=%lld must be a non-negative multiple of m", (long long)pos0);
  const int n_new = T / m;
  if (B == 0 || n_new == 0) return CSA_OK;
  const int64_t first = pos0 / m;
  if (first + n_new > n_cap) return fail(CSA_ERR_ARG, "entries rows %lld..%lld exceed n_cap=%lld", (long long)first,
                                         (long long)(first + n_new - 1), (long long)n_cap);
  if (!ca || !za || !cb || !zb || !bias_a || !bias_b || !entries) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (ld < c) return fail(CSA_ERR_ARG, "ld=%lld < c=%d", (long long)ld, c);
  if (B > 1 && seq_stride < (int64_t)T * ld) return fail(CSA_ERR_ARG, "seq_stride too small");
  if (B > 1 && entries_seq_stride < n_cap * c) return fail(CSA_ERR_ARG, "entries_seq_stride too small");
  if (first > 0) {
    if (!halo_cb || !halo_zb) return fail(CSA_ERR_ARG, "pos0 > 0 needs the previous block (halo_cb, halo_zb)");
    if (halo_ld < c) return fail(CSA_ERR_ARG, "halo_ld < c");
    if (B > 1 && halo_seq_stride < (int64_t)m * halo_ld) return fail(CSA_ERR_ARG, "halo_seq_stride too small");
  }
  CompressArgs a{};
  a.B = B;
  a.n_new = n_new;
  a.m = m;
  a.c = c;
  a.first_entry = first;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.ca = ca;
  a.za = za;
  a.cb = cb;
  a.zb = zb;
  a.ld = ld;
  a.seq_stride = seq_stride;
  a.halo_cb = first > 0 ? halo_cb : ca;
  a.halo_zb = first > 0 ? halo_zb : za;
  a.halo_ld = first > 0 ? halo_ld : ld;
  a.halo_seq_stride = first > 0 ? halo_seq_stride : seq_stride;
  a.bias_a = bias_a;
  a.bias_b = bias_b;
  a.entries = entries;
  a.entries_seq_stride = entries_seq_stride;
  a.aligned16 = aligned(ca, 16) && aligned(za, 16) && aligned(cb, 16) && aligned(zb, 16) && aligned(a.halo_cb, 16) &&
                aligned(a.halo_zb, 16) && aligned(entries, 16);
  return hip_status(launch_compress(a, static_cast<hipStream_t>(stream)), "csa_compress");
}

int csa_hca_compress(int B, int T, int64_t pos0, int m, int c, int in_dtype, const void* cv, const void* z,
                     int64_t ld, int64_t seq_stride, const float* bias, void* entries, int64_t entries_seq_stride,
                     int64_t n_cap, int out_dtype, void* stream) {
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (m < 1 || m > compress_max_m()) return fail(CSA_ERR_ARG, "m=%d out of [1, %d]", m, compress_max_m());
  if (c < 1) return fail(CSA_ERR_ARG, "c must be >= 1");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (pos0 < 0 || pos0 % m) return fail(CSA_ERR_ARG, "pos0=%lld must be a non-negative multiple of m", (long long)pos0);
  const int n_new = T / m;
  if (B == 0 || n_new == 0) return CSA_OK;
  const int64_t first = pos0 / m;
  if (first + n_new > n_cap) return fail(CSA_ERR_ARG, "entries rows %lld..%lld exceed n_cap=%lld", (long long)first,
                                         (long long)(first + n_new - 1), (long long)n_cap);
  if (!cv || !z || !bias || !entries) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (ld < c) return fail(CSA_ERR_ARG, "ld=%lld < c=%d", (long long)ld, c);
  if (B > 1 && seq_stride < (int64_t)T * ld) return fail(CSA_ERR_ARG, "seq_stride too small");
  if (B > 1 && entries_seq_stride < n_cap * c) return fail(CSA_ERR_ARG, "entries_seq_stride too small");
  CompressArgs a{};
  a.B = B;
  a.n_new = n_new;
  a.m = m;
  a.c = c;
  a.first_entry = first;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.ca = cv;
  a.za = z;
  a.cb = cv;  // series b is not read without overlap
  a.zb = z;
  a.ld = ld;
  a.seq_stride = seq_stride;
  a.halo_cb = cv;
  a.halo_zb = z;
  a.halo_ld = ld;
  a.halo_seq_stride = seq_stride;
  a.bias_a = bias;
  a.bias_b = bias;
  a.entries = entries;
  a.entries_seq_stride = entries_seq_stride;
  a.aligned16 = aligned(cv, 16) && aligned(z, 16) && aligned(entries, 16);
  a.overlap = false;
  return hip_status(launch_compress(a, static_cast<hipStream_t>(stream)), "csa_hca_compress");
}

int csa_index_topk(const csa_dims* dims, int B, int T, int64_t q_pos0, int idx_dtype, const void* q_idx, int64_t q_ld,
                   int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld, const void* keys,
                   int64_t keys_seq_stride, const void* k_scale, int64_t n_cap, int32_t* out_idx, float* out_score,
                   void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_index(dims, B, T, q_pos0, idx_dtype, q_idx, q_ld, q_seq_stride, q_scale, w, w_ld, keys,
                          keys_seq_stride, k_scale, n_cap, out_idx);
  if (rc) return rc;
  if ((int64_t)B * T == 0) return CSA_OK;
  IndexArgs a = make_index_args(dims, B, T, q_pos0, idx_dtype, q_idx, q_ld, q_seq_stride, q_scale, w, w_ld, keys,
                                keys_seq_stride, k_scale, n_cap, out_idx, out_score);
  rc = check_ws(ws, ws_bytes, index_topk_workspace(a));
  if (rc) return rc;
  return hip_status(launch_index_topk(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), "csa_index_topk");
}

int csa_topk_from_scores(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k, int32_t* out_idx,
                         float* out_score, void* ws, size_t ws_bytes, void* stream) {
  if (R < 0 || ld < 0) return fail(CSA_ERR_ARG, "R and ld must be >= 0");
  if (k < 1 || k > kMaxTopK) return fail(CSA_ERR_ARG, "k=%d out of [1, %d]", k, kMaxTopK);
  if (ld > 0x7FFFFFFFLL) return fail(CSA_ERR_ARG, "ld too large");
  if (R == 0) return CSA_OK;
  if (!scores || !n_valid || !out_idx) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  int rc = check_ws(ws, ws_bytes, topk_workspace(R, ld, k));
  if (rc) return rc;
  TopkArgs a{scores, ld, n_valid, R, k, out_idx, out_score};
  return hip_status(launch_topk_from_scores(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), "csa_topk_from_scores");
}


int csa_sparse_attn(const csa_dims* dims, int B, int T, int64_t q_pos0, int in_dtype, const void* q, int64_t q_ld,
                    int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride, int64_t n_cap,
                    const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride, int64_t raw_pos0,
                    int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws, size_t ws_bytes,
                    void* stream) {
  return attn_call("csa_sparse_attn", false, dims, B, T, q_pos0, in_dtype, q, q_ld, q_seq_stride, entries,
                   entries_seq_stride, n_cap, idx, kv_raw, raw_ld, raw_seq_stride, raw_pos0, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream);
}

int csa_sparse_attn_fp8(const csa_dims* dims, int B, int T, int64_t q_pos0, int in_dtype, const void* q, int64_t q_ld,
                        int64_t q_seq_stride, const void* records, int64_t records_seq_stride, int64_t n_cap,
                        const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                        int64_t raw_pos0, int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws,
                        size_t ws_bytes, void* stream) {
  return attn_call("csa_sparse_attn_fp8", false, dims, B, T, q_pos0, in_dtype, q, q_ld, q_seq_stride, records,
                   records_seq_stride, n_cap, idx, kv_raw, raw_ld, raw_seq_stride, raw_pos0, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream, 1);
}

int csa_dense_attn_fp8(const csa_dims* dims, int B, int T, int64_t q_pos0, int in_dtype, const void* q, int64_t q_ld,
                       int64_t q_seq_stride, const void* records, int64_t records_seq_stride, int64_t n_cap,
                       const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride, int64_t raw_pos0, int64_t raw_len,
                       const float* sink, void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  return attn_call("csa_dense_attn_fp8", true, dims, B, T, q_pos0, in_dtype, q, q_ld, q_seq_stride, records,
                   records_seq_stride, n_cap, nullptr, kv_raw, raw_ld, raw_seq_stride, raw_pos0, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream, 1);
}

int csa_entry_pack(int B, int N, int in_dtype, const void* entries, int64_t ld, int64_t seq_stride, void* records,
                   int64_t records_seq_stride, void* stream) {
  if (B < 0 || N < 0) return fail(CSA_ERR_ARG, "B and N must be >= 0");
  if (!is_act_dtype(in_dtype)) return fail(CSA_ERR_ARG, "dtype must be F32 or BF16");
  if ((int64_t)B * N == 0) return CSA_OK;
  if (!entries || !records) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (ld < 512) return fail(CSA_ERR_ARG, "ld < 512");
  if (B > 1 && (seq_stride < (int64_t)N * ld || records_seq_stride < (int64_t)N * kEntryRecordBytes))
    return fail(CSA_ERR_ARG, "sequence stride too small");
  if (!aligned(records, 8) || records_seq_stride % 8) return fail(CSA_ERR_ARG, "records need 8-byte alignment");
  EntryPackArgs a{};
  a.B = B;
  a.N = N;
  a.dtype = in_dtype;
  a.entries = entries;
  a.ld = ld;
  a.seq_stride = seq_stride;
  a.records = records;
  a.rec_seq_stride = records_seq_stride;
  hipError_t e = launch_entry_pack(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "csa_entry_pack");
  g_err.clear();
  return CSA_OK;
}

int csa_dense_attn(const csa_dims* dims, int B, int T, int64_t q_pos0, int in_dtype, const void* q, int64_t q_ld,
                   int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride, int64_t n_cap,
                   const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride, int64_t raw_pos0, int64_t raw_len,
                   const float* sink, void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  return attn_call("csa_dense_attn", true, dims, B, T, q_pos0, in_dtype, q, q_ld, q_seq_stride, entries,
                   entries_seq_stride, n_cap, nullptr, kv_raw, raw_ld, raw_seq_stride, raw_pos0, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream);
}

int csa_norm_rope(int B, int R, int H, int D, int dtype, const void* x, int64_t x_ld, int64_t x_seq_stride, void* y,
                  int64_t y_ld, int64_t y_seq_stride, const float* gamma, float eps, int rope_dims, float rope_theta,
                  int64_t pos0, int64_t pos_step, int inverse, void* stream) {
  if (B < 0 || R < 0 || H < 0) return fail(CSA_ERR_ARG, "B, R and H must be >= 0");
  if (D < 2 || D % 2 || D > norm_rope_max_dim())
    return fail(CSA_ERR_ARG, "D=%d must be even and in [2, %d]", D, norm_rope_max_dim());
  if (!is_act_dtype(dtype)) return fail(CSA_ERR_ARG, "dtype must be F32 or BF16");
  if (rope_dims < 0 || rope_dims > D || rope_dims % 2) return fail(CSA_ERR_ARG, "rope_dims=%d must be even and in [0, D]", rope_dims);
  if (rope_dims > 0 && !(rope_theta > 0.f)) return fail(CSA_ERR_ARG, "rope_theta must be > 0");
  if (gamma && inverse) return fail(CSA_ERR_ARG, "the inverse rotation takes no norm");
  if (!(eps >= 0.f)) return fail(CSA_ERR_ARG, "eps must be >= 0");
  if ((int64_t)B * R * H == 0) return CSA_OK;
  if (!x || !y) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (x_ld < (int64_t)H * D || y_ld < (int64_t)H * D) return fail(CSA_ERR_ARG, "row stride smaller than H*D");
  if (B > 1 && (x_seq_stride < (int64_t)R * x_ld || y_seq_stride < (int64_t)R * y_ld))
    return fail(CSA_ERR_ARG, "sequence stride too small");
  NormRopeArgs a{};
  a.B = B;
  a.R = R;
  a.H = H;
  a.D = D;
  a.dtype = dtype;
  a.x = x;
  a.x_ld = x_ld;
  a.x_seq_stride = x_seq_stride;
  a.y = y;
  a.y_ld = y_ld;
  a.y_seq_stride = y_seq_stride;
  a.gamma = gamma;
  a.eps = eps;
  a.rope_dims = rope_dims;
  a.theta = rope_theta;
  a.pos0 = pos0;
  a.pos_step = pos_step;
  a.inverse = inverse ? 1 : 0;
  hipError_t e = launch_norm_rope(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "csa_norm_rope");
  g_err.clear();
  return CSA_OK;
}

int csa_decode_step(const csa_dims* dims, const csa_weights* w, int B, int64_t pos, int dtype, const void* q,
                    const void* q_idx, const void* kv, const void* comp, const csa_decode_state* st, void* out,
                    int out_dtype, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!w || !st) return fail(CSA_ERR_ARG, "weights or state is NULL");
  if (B < 0) return fail(CSA_ERR_ARG, "B must be >= 0");
  if (!is_act_dtype(dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (B == 0) return CSA_OK;
  const int m = dims->m, D = dims->D, DI = dims->D_I, H = dims->H, HI = dims->H_I, W = dims->window;
  const int64_t n_cap = st->n_cap;
  if (pos < 0 || (pos + 1) / m > n_cap) return fail(CSA_ERR_ARG, "pos=%lld outside the entry capacity", (long long)pos);
  if (!q || !q_idx || !kv || !comp || !out || !st->entries || !st->keys || !st->win || !st->block)
    return fail(CSA_ERR_ARG, "NULL tensor or state pointer");
  if (!w->bias_a || !w->bias_b || !w->ibias_a || !w->ibias_b || !w->w_head) return fail(CSA_ERR_ARG, "NULL weight pointer");
  if (st->entry_fmt != 0 && st->entry_fmt != 1) return fail(CSA_ERR_ARG, "entry_fmt must be 0 or 1");
  if (st->entry_fmt && D != 512) return fail(CSA_ERR_ARG, "entry records hold D = 512");
  const bool fid = w->gamma_q || w->gamma_kv || w->rope_dims != 0;
  if (fid && (w->rope_dims < 0 || w->rope_dims > D || w->rope_dims % 2 || (w->rope_dims > 0 && !(w->rope_theta > 0.f)) ||
              !(w->norm_eps >= 0.f)))
    return fail(CSA_ERR_ARG, "QK-norm / RoPE parameters: rope_dims even in [0, D], rope_theta > 0, norm_eps >= 0");
  const DecodeWs L = decode_ws(dims, B, n_cap, dtype);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int es = esize(dtype);
  const int64_t nc = 4LL * D + 4LL * DI;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* blk = static_cast<uint8_t*>(st->block);
  uint8_t* cur = blk + (size_t)m * nc * es;  // the current block's rows

  // the token's compressor inputs and raw KV join the state
  hipError_t e = launch_copy_rows(B, 1, (int)nc, es, comp, nc, nc, cur + (size_t)(pos % m) * nc * es, nc,
                                  2LL * m * nc, s);
  if (e != hipSuccess) return hip_status(e, "csa_decode_step: block row");
  uint8_t* wrow = static_cast<uint8_t*>(st->win) + (size_t)(pos % W) * D * es;
  if (fid) {  // normalised and rotated on the way into the ring
    rc = csa_norm_rope(B, 1, 1, D, dtype, kv, D, D, wrow, D, (int64_t)W * D, w->gamma_kv, w->norm_eps, w->rope_dims,
                       w->rope_theta, pos, 1, 0, stream);
    if (rc) return rc;
  } else if ((e = launch_copy_rows(B, 1, D, es, kv, D, D, wrow, D, (int64_t)W * D, s)) != hipSuccess) {
    return hip_status(e, "csa_decode_step: window row");
  }

  // a completed block: its entry and indexer key (own block = series a, previous block = series b)
  if ((pos + 1) % m == 0) {
    const int64_t i = (pos + 1) / m - 1;
    CompressArgs a{};
    a.B = B;
    a.n_new = 1;
    a.m = m;
    a.first_entry = i;
    a.in_dtype = dtype;
    a.out_dtype = dtype;
    a.ld = nc;
    a.seq_stride = 2LL * m * nc;
    a.halo_ld = nc;
    a.halo_seq_stride = 2LL * m * nc;
    const bool has_prev = i >= 1;
    auto run = [&](int c, int64_t col, const float* ba, const float* bb, void* dst, int64_t dst_seq,
                   int64_t out_first) {
      CompressArgs x = a;
      x.c = c;
      x.ca = cur + (size_t)col * es;
      x.za = cur + (size_t)(col + c) * es;
      x.cb = cur + (size_t)(col + 2 * c) * es;
      x.zb = cur + (size_t)(col + 3 * c) * es;
      x.halo_cb = has_prev ? blk + (size_t)(col + 2 * c) * es : x.ca;
      x.halo_zb = has_prev ? blk + (size_t)(col + 3 * c) * es : x.za;
      x.bias_a = ba;
      x.bias_b = bb;
      x.entries = dst;
      x.entries_seq_stride = dst_seq;
      x.out_first = out_first;
      x.aligned16 = aligned(x.ca, 16) && aligned(x.za, 16) && aligned(x.cb, 16) && aligned(x.zb, 16) &&
                    aligned(x.halo_cb, 16) && aligned(x.halo_zb, 16) && aligned(dst, 16) && (nc * es) % 16 == 0;
      return launch_compress(x, s);
    };
    // the entry: into its cache row, or into a scratch row that is then packed into a record
    void* erow = st->entry_fmt ? (void*)(base + L.ent) : static_cast<uint8_t*>(st->entries) + (size_t)i * D * es;
    e = run(D, 0, w->bias_a, w->bias_b, st->entry_fmt ? (void*)(base + L.ent) : st->entries,
            st->entry_fmt ? (int64_t)D : n_cap * D, st->entry_fmt ? 0 : -1);
    if (e == hipSuccess) e = run(DI, 4LL * D, w->ibias_a, w->ibias_b, st->keys, n_cap * DI, -1);
    if (e != hipSuccess) return hip_status(e, "csa_decode_step: compress");
    const int64_t eseq = st->entry_fmt ? (int64_t)D : n_cap * D;
    if (fid) {
      rc = csa_norm_rope(B, 1, 1, D, dtype, erow, D, eseq, erow, D, eseq, w->gamma_kv, w->norm_eps, w->rope_dims,
                         w->rope_theta, pos, 1, 0, stream);
      if (rc) return rc;
    }
    if (st->entry_fmt) {
      rc = csa_entry_pack(B, 1, dtype, erow, D, D, static_cast<uint8_t*>(st->entries) + (size_t)i * kEntryRecordBytes,
                          n_cap * kEntryRecordBytes, stream);
      if (rc) return rc;
    }
    // the block becomes the previous one
    e = launch_copy_rows(B, m, (int)nc, es, cur, nc, 2LL * m * nc, blk, nc, 2LL * m * nc, s);
    if (e != hipSuccess) return hip_status(e, "csa_decode_step: block shift");
  }

  // the query, normalised and rotated at pos
  const void* qq = q;
  if (fid) {
    rc = csa_norm_rope(B, 1, H, D, dtype, q, (int64_t)H * D, (int64_t)H * D, base + L.q, (int64_t)H * D,
                       (int64_t)H * D, w->gamma_q, w->norm_eps, w->rope_dims, w->rope_theta, pos, 1, 0, stream);
    if (rc) return rc;
    qq = base + L.q;
  }
  int32_t* idx = out_idx ? out_idx : reinterpret_cast<int32_t*>(base + L.idx);
  void* scratch = base + L.scratch;
  const size_t scratch_bytes = L.total - L.scratch;
  rc = csa_index_topk(dims, B, 1, pos, dtype, q_idx, (int64_t)HI * DI, (int64_t)HI * DI, nullptr, w->w_head, 0,
                      st->keys, n_cap * DI, nullptr, n_cap, idx, nullptr, scratch, scratch_bytes, stream);
  if (rc) return rc;
  // the window [pos - raw_len + 1, pos], read by the attention straight from the ring
  const int64_t raw_len = pos + 1 < W ? pos + 1 : W;
  const int64_t raw_pos0 = pos - raw_len + 1;
  rc = attn_call("csa_decode_step", false, dims, B, 1, pos, dtype, qq, (int64_t)H * D, (int64_t)H * D, st->entries,
                 n_cap * (st->entry_fmt ? (int64_t)kEntryRecordBytes : D), n_cap, idx, st->win, D, (int64_t)W * D,
                 raw_pos0, raw_len, w->sink, out, out_dtype, scratch, scratch_bytes, stream, st->entry_fmt, W);
  if (rc) return rc;
  if (fid && w->rope_dims > 0) {
    rc = csa_norm_rope(B, 1, H, D, out_dtype, out, (int64_t)H * D, (int64_t)H * D, out, (int64_t)H * D,
                       (int64_t)H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos, 1, 1, stream);
    if (rc) return rc;
  }
  g_err.clear();
  return CSA_OK;
}

int csa_hca_decode_step(const csa_dims* dims, const csa_weights* w, int B, int64_t pos, int dtype, const void* q,
                        const void* kv, const void* comp, const csa_decode_state* st, void* out, int out_dtype,
                        void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims, false);
  if (rc) return rc;
  if (!w || !st) return fail(CSA_ERR_ARG, "weights or state is NULL");
  if (B < 0) return fail(CSA_ERR_ARG, "B must be >= 0");
  if (!is_act_dtype(dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (B == 0) return CSA_OK;
  const int m = dims->m, D = dims->D, H = dims->H, W = dims->window;
  if (m > compress_max_m()) return fail(CSA_ERR_ARG, "m=%d above %d", m, compress_max_m());
  const int64_t n_cap = st->n_cap;
  if (pos < 0 || (pos + 1) / m > n_cap) return fail(CSA_ERR_ARG, "pos=%lld outside the entry capacity", (long long)pos);
  if (!q || !kv || !comp || !out || !st->entries || !st->win || !st->block || !w->bias_a)
    return fail(CSA_ERR_ARG, "NULL tensor, state or bias pointer");
  if (st->entry_fmt != 0 && st->entry_fmt != 1) return fail(CSA_ERR_ARG, "entry_fmt must be 0 or 1");
  if (st->entry_fmt && D != 512) return fail(CSA_ERR_ARG, "entry records hold D = 512");
  const bool fid = w->gamma_q || w->gamma_kv || w->rope_dims != 0;
  if (fid && (w->rope_dims < 0 || w->rope_dims > D || w->rope_dims % 2 || (w->rope_dims > 0 && !(w->rope_theta > 0.f)) ||
              !(w->norm_eps >= 0.f)))
    return fail(CSA_ERR_ARG, "QK-norm / RoPE parameters: rope_dims even in [0, D], rope_theta > 0, norm_eps >= 0");
  const DecodeWs L = hca_decode_ws(dims, B, n_cap, dtype);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int es = esize(dtype);
  const int64_t nc = 2LL * D;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* blk = static_cast<uint8_t*>(st->block);
  hipError_t e = launch_copy_rows(B, 1, (int)nc, es, comp, nc, nc, blk + (size_t)(pos % m) * nc * es, nc,
                                  (int64_t)m * nc, s);
  if (e != hipSuccess) return hip_status(e, "csa_hca_decode_step: block row");
  uint8_t* wrow = static_cast<uint8_t*>(st->win) + (size_t)(pos % W) * D * es;
  if (fid) {
    rc = csa_norm_rope(B, 1, 1, D, dtype, kv, D, D, wrow, D, (int64_t)W * D, w->gamma_kv, w->norm_eps, w->rope_dims,
                       w->rope_theta, pos, 1, 0, stream);
    if (rc) return rc;
  } else if ((e = launch_copy_rows(B, 1, D, es, kv, D, D, wrow, D, (int64_t)W * D, s)) != hipSuccess) {
    return hip_status(e, "csa_hca_decode_step: window row");
  }
  // a completed block: its entry, pooled over the block alone
  if ((pos + 1) % m == 0) {
    const int64_t i = (pos + 1) / m - 1;
    CompressArgs a{};
    a.B = B;
    a.n_new = 1;
    a.m = m;
    a.c = D;
    a.first_entry = i;
    a.in_dtype = dtype;
    a.out_dtype = dtype;
    a.ca = blk;
    a.za = blk + (size_t)D * es;
    a.cb = a.ca;
    a.zb = a.za;
    a.ld = nc;
    a.seq_stride = (int64_t)m * nc;
    a.halo_cb = a.ca;
    a.halo_zb = a.za;
    a.halo_ld = nc;
    a.halo_seq_stride = (int64_t)m * nc;
    a.bias_a = w->bias_a;
    a.bias_b = w->bias_a;
    a.overlap = false;
    void* erow = st->entry_fmt ? (void*)(base + L.ent) : static_cast<uint8_t*>(st->entries) + (size_t)i * D * es;
    a.entries = st->entry_fmt ? (void*)(base + L.ent) : st->entries;
    a.entries_seq_stride = st->entry_fmt ? (int64_t)D : n_cap * D;
    a.out_first = st->entry_fmt ? 0 : -1;
    a.aligned16 = aligned(a.ca, 16) && aligned(a.za, 16) && aligned(a.entries, 16) && (nc * es) % 16 == 0;
    if ((e = launch_compress(a, s)) != hipSuccess) return hip_status(e, "csa_hca_decode_step: compress");
    const int64_t eseq = a.entries_seq_stride;
    if (fid) {
      rc = csa_norm_rope(B, 1, 1, D, dtype, erow, D, eseq, erow, D, eseq, w->gamma_kv, w->norm_eps, w->rope_dims,
                         w->rope_theta, pos, 1, 0, stream);
      if (rc) return rc;
    }
    if (st->entry_fmt) {
      rc = csa_entry_pack(B, 1, dtype, erow, D, D, static_cast<uint8_t*>(st->entries) + (size_t)i * kEntryRecordBytes,
                          n_cap * kEntryRecordBytes, stream);
      if (rc) return rc;
    }
  }
  const void* qq = q;
  if (fid) {
    rc = csa_norm_rope(B, 1, H, D, dtype, q, (int64_t)H * D, (int64_t)H * D, base + L.q, (int64_t)H * D,
                       (int64_t)H * D, w->gamma_q, w->norm_eps, w->rope_dims, w->rope_theta, pos, 1, 0, stream);
    if (rc) return rc;
    qq = base + L.q;
  }
  const int64_t raw_len = pos + 1 < W ? pos + 1 : W;
  rc = attn_call("csa_hca_decode_step", true, dims, B, 1, pos, dtype, qq, (int64_t)H * D, (int64_t)H * D, st->entries,
                 n_cap * (st->entry_fmt ? (int64_t)kEntryRecordBytes : D), n_cap, nullptr, st->win, D, (int64_t)W * D,
                 pos - raw_len + 1, raw_len, w->sink, out, out_dtype, base + L.scratch, L.total - L.scratch, stream,
                 st->entry_fmt, W);
  if (rc) return rc;
  if (fid && w->rope_dims > 0) {
    rc = csa_norm_rope(B, 1, H, D, out_dtype, out, (int64_t)H * D, (int64_t)H * D, out, (int64_t)H * D,
                       (int64_t)H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos, 1, 1, stream);
    if (rc) return rc;
  }
  g_err.clear();
  return CSA_OK;
}

int csa_forward(const csa_dims* dims, const csa_weights* w, int B, int T, int64_t pos0, int d_model, int dtype,
                const void* x, const csa_cache* cache, void* out, int out_dtype, int32_t* out_idx, void* ws,
                size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!w || !cache) return fail(CSA_ERR_ARG, "weights or cache is NULL");
  if (B < 0 || T < 0 || d_model < 1) return fail(CSA_ERR_ARG, "bad B/T/d_model");
  if (!is_act_dtype(dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  const int m = dims->m, D = dims->D, DI = dims->D_I, H = dims->H, HI = dims->H_I, W = dims->window, k = dims->top_k;
  if (pos0 < 0 || pos0 % m) return fail(CSA_ERR_ARG, "pos0 must be a non-negative multiple of m");
  if ((int64_t)B * T == 0) return CSA_OK;
  if (!x || !out || !w->w_proj || !w->bias_a || !w->bias_b || !w->ibias_a || !w->ibias_b || !w->w_head)
    return fail(CSA_ERR_ARG, "NULL weight/input pointer");
  if (!cache->entries || !cache->keys || !cache->win) return fail(CSA_ERR_ARG, "NULL cache pointer");
  if ((pos0 + T) / m > cache->n_cap) return fail(CSA_ERR_ARG, "(pos0+T)/m exceeds n_cap");
  if ((int64_t)W - 1 + T > cache->win_cap) return fail(CSA_ERR_ARG, "window - 1 + T exceeds win_cap");
  if (pos0 > 0 && !cache->halo) return fail(CSA_ERR_ARG, "pos0 > 0 needs cache->halo");
  if (cache->halo_out && T % m) return fail(CSA_ERR_ARG, "halo_out needs T %% m == 0");
  const bool fid = w->gamma_q || w->gamma_kv || w->rope_dims != 0;
  if (fid && (w->rope_dims < 0 || w->rope_dims > D || w->rope_dims % 2 || (w->rope_dims > 0 && !(w->rope_theta > 0.f)) ||
              !(w->norm_eps >= 0.f)))
    return fail(CSA_ERR_ARG, "QK-norm / RoPE parameters: rope_dims even in [0, D], rope_theta > 0, norm_eps >= 0");
  const bool records = cache->entry_fmt != 0;
  if (cache->entry_fmt != 0 && cache->entry_fmt != 1) return fail(CSA_ERR_ARG, "entry_fmt must be 0 or 1");
  if (records && D != 512) return fail(CSA_ERR_ARG, "entry records hold D = 512");
  const int64_t ntot = n_tot_of(dims);
  const int es = esize(dtype);
  // workspace: P [B*T, ntot] | idx [B*T, k] | index scratch
  IndexArgs probe = make_index_args(dims, B, T, pos0, dtype, nullptr, 0, 0, nullptr, nullptr, 0, nullptr, 0, nullptr,
                                    cache->n_cap, nullptr, nullptr);
  const size_t p_bytes = align256((size_t)B * T * ntot * es);
  const size_t i_bytes = align256((size_t)B * T * k * 4);
  const size_t i_ws = index_topk_workspace(probe);
  const size_t a_ws = attn_workspace(sizing_attn(dims, B, T, dtype));
  size_t scratch = i_ws > a_ws ? i_ws : a_ws;  // index / attention scratch, or the projection's
  if (dtype == CSA_BF16 && scratch < kGemmWorkspace) scratch = kGemmWorkspace;
  const size_t ent_tmp = (size_t)B * (T / m) * D * es;  // new entries before packing into records
  if (scratch < ent_tmp) scratch = ent_tmp;
  const size_t x_bytes = align256(scratch);
  rc = check_ws(ws, ws_bytes, p_bytes + i_bytes + x_bytes);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(w->w_proj, 16)) return fail(CSA_ERR_ARG, "x and w_proj must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* P = static_cast<uint8_t*>(ws);
  int32_t* idx = out_idx ? out_idx : reinterpret_cast<int32_t*>(P + p_bytes);
  void* xws = P + p_bytes + i_bytes;
  auto col = [&](int64_t c) { return static_cast<void*>(P + c * es); };
  const int64_t c_ca = 0, c_za = D, c_cb = 2LL * D, c_zb = 3LL * D;
  const int64_t c_ica = 4LL * D, c_iza = c_ica + DI, c_icb = c_ica + 2LL * DI, c_izb = c_ica + 3LL * DI;
  const int64_t c_q = 4LL * D + 4LL * DI, c_qi = c_q + (int64_t)H * D, c_kv = c_qi + (int64_t)HI * DI;
  const int64_t halo_ld = 2LL * D + 2LL * DI;
  const uint8_t* halo = static_cast<const uint8_t*>(cache->halo);

  GemmArgs g{};
  g.M = B * T;
  g.N = (int)ntot;
  g.K = d_model;
  g.dtype = dtype;
  g.out_dtype = dtype;
  g.A = x;
  g.lda = d_model;
  g.Bm = w->w_proj;
  g.ldb = d_model;
  g.C = P;
  g.ldc = ntot;
  bool done = false;
  hipError_t e = launch_gemm_library(g, xws, x_bytes, s, &done);
  if (e == hipSuccess && !done) e = launch_gemm(g, s);
  if (e != hipSuccess) return hip_status(e, "csa_forward: projection");

  // new entries: into their cache rows, or (records) into the scratch, to be packed below
  void* ent_dst = records ? xws : cache->entries;
  const int64_t ent_seq = records ? (int64_t)(T / m) * D : cache->n_cap * D;
  if (records) {
    CompressArgs ca{};
    ca.B = B;
    ca.n_new = T / m;
    ca.m = m;
    ca.c = D;
    ca.first_entry = pos0 / m;
    ca.in_dtype = dtype;
    ca.out_dtype = dtype;
    ca.ca = col(c_ca);
    ca.za = col(c_za);
    ca.cb = col(c_cb);
    ca.zb = col(c_zb);
    ca.ld = ntot;
    ca.seq_stride = (int64_t)T * ntot;
    ca.halo_cb = halo ? halo : ca.ca;
    ca.halo_zb = halo ? halo + (size_t)D * es : ca.za;
    ca.halo_ld = halo ? halo_ld : ntot;
    ca.halo_seq_stride = halo ? (int64_t)m * halo_ld : (int64_t)T * ntot;
    ca.bias_a = w->bias_a;
    ca.bias_b = w->bias_b;
    ca.entries = xws;
    ca.entries_seq_stride = ent_seq;
    ca.out_first = 0;
    ca.aligned16 = aligned(ca.ca, 16) && aligned(ca.za, 16) && aligned(ca.cb, 16) && aligned(ca.zb, 16) &&
                   aligned(ca.halo_cb, 16) && aligned(ca.halo_zb, 16) && (ntot * es) % 16 == 0;
    if (ca.n_new > 0 && (e = launch_compress(ca, s)) != hipSuccess) return hip_status(e, "csa_forward: compress");
  } else {
    rc = csa_compress(B, T, pos0, m, D, dtype, col(c_ca), col(c_za), col(c_cb), col(c_zb), ntot, (int64_t)T * ntot,
                      halo ? halo : nullptr, halo ? halo + (size_t)D * es : nullptr, halo_ld, (int64_t)m * halo_ld,
                      w->bias_a, w->bias_b, cache->entries, cache->n_cap * D, cache->n_cap, dtype, stream);
    if (rc) return rc;
  }
  rc = csa_compress(B, T, pos0, m, DI, dtype, col(c_ica), col(c_iza), col(c_icb), col(c_izb), ntot, (int64_t)T * ntot,
                    halo ? halo + (size_t)2 * D * es : nullptr, halo ? halo + (size_t)(2 * D + DI) * es : nullptr,
                    halo_ld, (int64_t)m * halo_ld, w->ibias_a, w->ibias_b, cache->keys, cache->n_cap * DI,
                    cache->n_cap, dtype, stream);
  if (rc) return rc;
  // the chunk's raw KV goes to window rows [W-1, W-1+T)
  e = launch_copy_rows(B, T, D, es, col(c_kv), ntot, (int64_t)T * ntot,
                       static_cast<uint8_t*>(cache->win) + (size_t)(W - 1) * D * es, D, cache->win_cap * D, s);
  if (e != hipSuccess) return hip_status(e, "csa_forward: window copy");
  if (fid) {
    // queries (in the projection buffer), the chunk's window rows and the new entries, in place
    rc = csa_norm_rope(B, T, H, D, dtype, col(c_q), ntot, (int64_t)T * ntot, col(c_q), ntot, (int64_t)T * ntot,
                       w->gamma_q, w->norm_eps, w->rope_dims, w->rope_theta, pos0, 1, 0, stream);
    if (rc) return rc;
    void* wrows = static_cast<uint8_t*>(cache->win) + (size_t)(W - 1) * D * es;
    rc = csa_norm_rope(B, T, 1, D, dtype, wrows, D, cache->win_cap * D, wrows, D, cache->win_cap * D, w->gamma_kv,
                       w->norm_eps, w->rope_dims, w->rope_theta, pos0, 1, 0, stream);
    if (rc) return rc;
    void* erows = records ? ent_dst : static_cast<uint8_t*>(cache->entries) + (size_t)(pos0 / m) * D * es;
    rc = csa_norm_rope(B, T / m, 1, D, dtype, erows, D, ent_seq, erows, D, ent_seq, w->gamma_kv, w->norm_eps,
                       w->rope_dims, w->rope_theta, pos0 + m - 1, m, 0, stream);
    if (rc) return rc;
  }
  if (records) {
    rc = csa_entry_pack(B, T / m, dtype, ent_dst, D, ent_seq,
                        static_cast<uint8_t*>(cache->entries) + (size_t)(pos0 / m) * kEntryRecordBytes,
                        cache->n_cap * kEntryRecordBytes, stream);
    if (rc) return rc;
  }
  rc = csa_index_topk(dims, B, T, pos0, dtype, col(c_qi), ntot, (int64_t)T * ntot, nullptr, w->w_head, 0, cache->keys,
                      cache->n_cap * DI, nullptr, cache->n_cap, idx, nullptr, xws, x_bytes, stream);
  if (rc) return rc;
  rc = attn_call("csa_forward", false, dims, B, T, pos0, dtype, col(c_q), ntot, (int64_t)T * ntot, cache->entries,
                 cache->n_cap * (records ? (int64_t)kEntryRecordBytes : D), cache->n_cap, idx, cache->win, D,
                 cache->win_cap * D, pos0 - (W - 1), (int64_t)W - 1 + T, w->sink, out, out_dtype, xws, x_bytes, stream,
                 records ? 1 : 0);
  if (rc) return rc;
  if (fid && w->rope_dims > 0) {
    rc = csa_norm_rope(B, T, H, D, out_dtype, out, (int64_t)H * D, (int64_t)T * H * D, out, (int64_t)H * D,
                       (int64_t)T * H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos0, 1, 1, stream);
    if (rc) return rc;
  }
  if (cache->halo_out) {
    uint8_t* ho = static_cast<uint8_t*>(cache->halo_out);
    e = launch_copy_rows(B, m, 2 * D, es, col(c_cb + (int64_t)(T - m) * ntot), ntot, (int64_t)T * ntot, ho, halo_ld,
                         (int64_t)m * halo_ld, s);
    if (e == hipSuccess)
      e = launch_copy_rows(B, m, 2 * DI, es, col(c_icb + (int64_t)(T - m) * ntot), ntot, (int64_t)T * ntot,
                           ho + (size_t)2 * D * es, halo_ld, (int64_t)m * halo_ld, s);
    if (e != hipSuccess) return hip_status(e, "csa_forward: halo copy");
  }
  g_err.clear();
  return CSA_OK;
}

}  // extern "C"
