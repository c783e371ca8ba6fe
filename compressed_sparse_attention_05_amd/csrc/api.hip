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

// error reporting for the probe entry points (csa_probe.h), through this thread's message
int probe_fail(const char* msg) { return fail(CSA_ERR_ARG, "%s", msg); }
int probe_status(hipError_t e, const char* what) { return hip_status(e, what); }

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

// The scratch of csa_decode_step_noalloc: one array per GPU the library runs on, held until the
// process ends. Host code never uses the name itself (on the host it is a stand-in, not a device
// address): its device address is looked up once per device and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[CSA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (the current device); nullptr and an error on failure.
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
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

bool pos_ok(const int64_t* p) { return p == nullptr || aligned(p, 8); }

// QK-norm / RoPE fields of the weights: on when a gain is given or rope_dims > 0
bool fid_on(const csa_weights* w) { return w->gamma_q || w->gamma_kv || w->rope_dims != 0; }
int check_fid(const csa_weights* w, int D) {
  if (!fid_on(w)) return CSA_OK;
  if (w->rope_dims < 0 || w->rope_dims > D || w->rope_dims % 2 || (w->rope_dims > 0 && !(w->rope_theta > 0.f)) ||
      !(w->norm_eps >= 0.f))
    return fail(CSA_ERR_ARG, "QK-norm / RoPE parameters: rope_dims even in [0, D], rope_theta > 0, norm_eps >= 0");
  if (D > norm_rope_max_dim() || D % 2) return fail(CSA_ERR_UNSUPPORTED, "QK-norm / RoPE needs an even D <= %d", norm_rope_max_dim());
  return CSA_OK;
}

IndexArgs make_index_args(const csa_dims* d, int B, int T, const int64_t* q_pos, int idx_dtype, const void* q_idx,
                          int64_t q_ld, int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld,
                          const void* keys, int64_t keys_seq_stride, const void* k_scale, int64_t n_cap,
                          int32_t* out_idx, float* out_score) {
  IndexArgs a{};
  a.B = B;
  a.T = T;
  a.q_pos = q_pos;
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

int validate_index(const csa_dims* d, int B, int T, const int64_t* q_pos, int idx_dtype, const void* q_idx,
                   int64_t q_ld, int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld,
                   const void* keys, int64_t keys_seq_stride, const void* k_scale, int64_t n_cap,
                   const int32_t* out_idx) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (!pos_ok(q_pos)) return fail(CSA_ERR_ARG, "q_pos must be 8-byte aligned");
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
    if (k_scale && !aligned(k_scale, 4)) return fail(CSA_ERR_ARG, "MXFP4 key scales must be 4-byte aligned");
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

// Workspace of csa_decode_step: the normalised / rotated query, the selected indices, and the index
// / attention scratch.
struct DecodeWs {
  size_t q, idx, qi, qis, scratch, total;
};
// q | idx | the indexer query in MXFP4 (codes, scales; used by MXFP4 key states) | scratch
DecodeWs decode_ws(const csa_dims* d, int B, int64_t n_cap, int dtype) {
  const size_t es = dtype == CSA_F32 ? 4 : 2;
  const size_t nqi = (size_t)B * d->H_I * d->D_I;
  DecodeWs w{};
  w.q = 0;
  w.idx = w.q + align256((size_t)B * d->H * d->D * es);
  w.qi = w.idx + align256((size_t)B * d->top_k * 4);
  w.qis = w.qi + align256(nqi / 2);
  w.scratch = w.qis + align256(nqi / 32);
  IndexArgs ia = make_index_args(d, B, 1, nullptr, dtype, nullptr, 0, 0, nullptr, nullptr, 0, nullptr, 0, nullptr,
                                 n_cap, nullptr, nullptr);
  const size_t iw = index_topk_workspace(ia);
  const size_t aw = attn_workspace(sizing_attn(d, B, 1, dtype));
  w.total = w.scratch + align256(iw > aw ? iw : aw);
  return w;
}

// Workspace of csa_hca_decode_step: the normalised / rotated query and the dense attention's split
// partials.
DecodeWs hca_decode_ws(const csa_dims* d, int B, int64_t n_cap, int dtype) {
  const size_t es = dtype == CSA_F32 ? 4 : 2;
  DecodeWs w{};
  w.q = 0;
  w.idx = align256((size_t)B * d->H * d->D * es);
  w.qi = w.qis = w.idx;
  w.scratch = w.idx;
  AttnArgs a = sizing_attn(d, B, 1, dtype);
  a.dense = 1;
  a.m = d->m;
  a.k = 0;
  a.n_cap = n_cap;
  w.total = w.scratch + align256(attn_workspace(a));
  return w;
}

// raw_ring > 0: kv_raw is a ring of raw_ring rows (position u in row u % raw_ring) holding at least
// each query's window; raw_pos and raw_len are then not used.
// Validates the attention's arguments and fills *out (nothing is launched).
int attn_prepare(bool dense, const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
                 const void* q, int64_t q_ld, int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride,
                 int64_t n_cap, const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                 const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out, int out_dtype,
                 int entry_fmt, int64_t raw_ring, int64_t raw_off, AttnArgs* res) {
  int rc = check_dims(dims, !dense);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (n_cap < 0 || raw_len < 0) return fail(CSA_ERR_ARG, "negative size");
  if (!pos_ok(q_pos) || !pos_ok(raw_pos)) return fail(CSA_ERR_ARG, "position arrays must be 8-byte aligned");
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
  if (raw_ring > 0 && (T != 1 || raw_ring < dims->window))
    return fail(CSA_ERR_ARG, "a raw KV ring serves one query row and holds at least the window");
  if (raw_ring == 0 && raw_len < 1) return fail(CSA_ERR_ARG, "kv_raw must hold at least one row (the query's own)");
  const int64_t raw_rows = raw_ring > 0 ? raw_ring : raw_len;
  if (B > 1 && raw_seq_stride < raw_rows * raw_ld) return fail(CSA_ERR_ARG, "raw_seq_stride too small");
  const size_t al = esize(in_dtype) == 2 ? 16 : 4;
  if (!aligned(q, al) || !aligned(kv_raw, al) || (entries && !aligned(entries, entry_fmt ? 16 : al)))
    return fail(CSA_ERR_ARG, "misaligned q / entries / kv_raw");
  if (entry_fmt && entries_seq_stride % 8) return fail(CSA_ERR_ARG, "record sequence stride must be a multiple of 8 bytes");
  AttnArgs a{};
  a.B = B;
  a.T = T;
  a.q_pos = q_pos;
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
  a.raw_pos = raw_ring > 0 ? nullptr : raw_pos;
  a.raw_off = raw_ring > 0 ? 0 : raw_off;
  a.raw_len = raw_ring > 0 ? ((int64_t)1 << 62) : raw_len;
  a.sink = sink;
  a.out = out;
  a.entry_fmt = entry_fmt;
  a.raw_ring = raw_ring;
  *res = a;
  return CSA_OK;
}

int attn_run(const char* name, const AttnArgs& a, void* ws, size_t ws_bytes, void* stream) {
  if ((int64_t)a.B * a.T == 0) return CSA_OK;
  int rc = check_ws(ws, ws_bytes, attn_workspace(a));
  if (rc) return rc;
  return hip_status(launch_attn(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), name);
}

// The query's QK-norm / RoPE and the output's back-rotation folded into the attention, where its
// kernels take them ("Anatomy of a Frontier Model", bullet "QK-norm and partial RoPE"); false: the
// caller runs the separate passes.
bool attn_try_fuse(AttnArgs& a, const csa_weights* w) {
  if (!w || (!w->gamma_q && w->rope_dims == 0)) return false;
  if (w->gamma_q && !aligned(w->gamma_q, 16)) return false;  // staged as 16-byte vectors
  a.fuse_fid = true;
  a.gamma_q = w->gamma_q;
  a.q_eps = w->norm_eps;
  a.rope_dims = w->rope_dims;
  a.rope_lt = w->rope_dims > 0 ? std::log2((double)w->rope_theta) : 0.0;
  if (attn_fuses_fid(a)) return true;
  a.fuse_fid = false;
  a.gamma_q = nullptr;
  a.rope_dims = 0;
  return false;
}

int attn_call(const char* name, bool dense, const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype,
              const void* q, int64_t q_ld, int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride,
              int64_t n_cap, const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
              const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws,
              size_t ws_bytes, void* stream, int entry_fmt = 0, int64_t raw_ring = 0, int64_t raw_off = 0) {
  AttnArgs a{};
  int rc = attn_prepare(dense, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, entries, entries_seq_stride, n_cap,
                        idx, kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, sink, out, out_dtype, entry_fmt,
                        raw_ring, raw_off, &a);
  if (rc || (int64_t)B * T == 0) return rc;
  return attn_run(name, a, ws, ws_bytes, stream);
}

// Compressor arguments common to csa_compress, csa_hca_compress and csa_forward.
int compress_call(const char* name, bool overlap, int B, int T, const int64_t* pos0, int m, int c, int in_dtype,
                  const void* ca, const void* za, const void* cb, const void* zb, int64_t ld, int64_t seq_stride,
                  const void* halo_cb, const void* halo_zb, int64_t halo_ld, int64_t halo_seq_stride,
                  const float* bias_a, const float* bias_b, void* entries, int64_t entries_seq_stride, int64_t n_cap,
                  int out_dtype, void* stream, const CompressArgs* epi = nullptr) {
  if (B < 0 || T < 0) return fail(CSA_ERR_ARG, "B and T must be >= 0");
  if (m < 1 || m > compress_max_m()) return fail(CSA_ERR_ARG, "m=%d out of [1, %d]", m, compress_max_m());
  if (c < 1) return fail(CSA_ERR_ARG, "c must be >= 1");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (!pos_ok(pos0)) return fail(CSA_ERR_ARG, "pos0 must be 8-byte aligned");
  if (n_cap < 0) return fail(CSA_ERR_ARG, "n_cap must be >= 0");
  const int n_new = T / m;
  if (B == 0 || n_new == 0) return CSA_OK;
  if (!pos0 && n_new > n_cap)
    return fail(CSA_ERR_ARG, "entries rows 0..%d exceed n_cap=%lld", n_new - 1, (long long)n_cap);
  if (!ca || !za || !cb || !zb || !bias_a || !bias_b || !entries) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (ld < c) return fail(CSA_ERR_ARG, "ld=%lld < c=%d", (long long)ld, c);
  if (B > 1 && seq_stride < (int64_t)T * ld) return fail(CSA_ERR_ARG, "seq_stride too small");
  const bool records = epi && epi->records;
  const bool fp4 = epi && epi->fp4_codes;  // MXFP4 rows [B, n_cap, c/2] + scales, contiguous
  if (!fp4 && B > 1 && entries_seq_stride < n_cap * (records ? (int64_t)kEntryRecordBytes : c))
    return fail(CSA_ERR_ARG, "entries_seq_stride too small");
  if (overlap && pos0) {
    if (!halo_cb || !halo_zb)
      return fail(CSA_ERR_ARG, "per-sequence positions need the previous block (halo_cb, halo_zb)");
    if (halo_ld < c) return fail(CSA_ERR_ARG, "halo_ld < c");
    if (B > 1 && halo_seq_stride < (int64_t)m * halo_ld) return fail(CSA_ERR_ARG, "halo_seq_stride too small");
  }
  CompressArgs a{};
  if (epi) a = *epi;
  a.B = B;
  a.n_new = n_new;
  a.m = m;
  a.c = c;
  a.pos0 = pos0;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.ca = ca;
  a.za = za;
  a.cb = cb;
  a.zb = zb;
  a.ld = ld;
  a.seq_stride = seq_stride;
  const bool halo = overlap && pos0;
  a.halo_cb = halo ? halo_cb : ca;
  a.halo_zb = halo ? halo_zb : za;
  a.halo_ld = halo ? halo_ld : ld;
  a.halo_seq_stride = halo ? halo_seq_stride : seq_stride;
  a.bias_a = bias_a;
  a.bias_b = bias_b;
  a.entries = entries;
  a.entries_seq_stride = entries_seq_stride;
  a.n_cap = n_cap;
  a.overlap = overlap;
  a.aligned16 = aligned(ca, 16) && aligned(za, 16) && aligned(cb, 16) && aligned(zb, 16) && aligned(a.halo_cb, 16) &&
                aligned(a.halo_zb, 16) && aligned(entries, 16);
  if (a.epilogue && !compress_epilogue_ok(a))
    return fail(CSA_ERR_UNSUPPORTED, "%s: entry norm / RoPE / records / MXFP4 keys need one entry per wave "
                "(c / vector <= 64, 16-byte aligned rows)", name);
  return hip_status(launch_compress(a, static_cast<hipStream_t>(stream)), name);
}

int norm_rope_call(int B, int R, int H, int D, int dtype, const void* x, int64_t x_ld, int64_t x_seq_stride, void* y,
                   int64_t y_ld, int64_t y_seq_stride, const float* gamma, float eps, int rope_dims, float rope_theta,
                   const int64_t* pos, int64_t pos_off, int64_t pos_step, int inverse, void* stream) {
  if (B < 0 || R < 0 || H < 0) return fail(CSA_ERR_ARG, "B, R and H must be >= 0");
  if (D < 2 || D % 2 || D > norm_rope_max_dim())
    return fail(CSA_ERR_ARG, "D=%d must be even and in [2, %d]", D, norm_rope_max_dim());
  if (!is_act_dtype(dtype)) return fail(CSA_ERR_ARG, "dtype must be F32 or BF16");
  if (rope_dims < 0 || rope_dims > D || rope_dims % 2) return fail(CSA_ERR_ARG, "rope_dims=%d must be even and in [0, D]", rope_dims);
  if (rope_dims > 0 && !(rope_theta > 0.f)) return fail(CSA_ERR_ARG, "rope_theta must be > 0");
  if (gamma && inverse) return fail(CSA_ERR_ARG, "the inverse rotation takes no norm");
  if (!(eps >= 0.f)) return fail(CSA_ERR_ARG, "eps must be >= 0");
  if (!pos_ok(pos)) return fail(CSA_ERR_ARG, "pos0 must be 8-byte aligned");
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
  a.pos = pos;
  a.pos_off = pos_off;
  a.pos_step = pos_step;
  a.inverse = inverse ? 1 : 0;
  return hip_status(launch_norm_rope(a, static_cast<hipStream_t>(stream)), "csa_norm_rope");
}

// Shared by csa_decode_step and csa_hca_decode_step: checks and the append launch.
int decode_append(const char* name, const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype,
                  const void* q, const void* kv, const void* comp, const csa_decode_state* st, bool hca, void* qn,
                  hipStream_t s, const void* q_idx = nullptr, uint8_t* qi_codes = nullptr,
                  uint8_t* qi_scales = nullptr) {
  AppendArgs a{};
  a.B = B;
  a.m = dims->m;
  a.D = dims->D;
  a.D_I = dims->D_I;
  a.H = dims->H;
  a.W = dims->window;
  a.dtype = dtype;
  a.hca = hca;
  a.pos = pos;
  a.comp = comp;
  a.kv = kv;
  a.q = q;
  a.qn = qn;
  a.block = st->block;
  a.win = st->win;
  a.entries = st->entries;
  a.keys = st->keys;
  a.n_cap = st->n_cap;
  a.entry_fmt = st->entry_fmt;
  a.bias_a = w->bias_a;
  a.bias_b = w->bias_b;
  a.ibias_a = w->ibias_a;
  a.ibias_b = w->ibias_b;
  a.gamma_q = w->gamma_q;
  a.gamma_kv = w->gamma_kv;
  a.eps = w->norm_eps;
  a.rope_dims = w->rope_dims;
  a.theta = w->rope_theta;
  a.aligned16 = aligned(comp, 16) && aligned(st->block, 16) && aligned(st->entries, 16) &&
                (hca || aligned(st->keys, 16));
  if (!hca && st->key_fmt) {
    a.key_fmt = 1;
    a.key_scales = static_cast<uint8_t*>(st->key_scales);
    a.q_idx = q_idx;
    a.H_I = dims->H_I;
    a.qi_codes = qi_codes;
    a.qi_scales = qi_scales;
    a.aligned16 = a.aligned16 && aligned(q_idx, 16);
  }
  return hip_status(launch_append(a, s), name);
}

int check_decode_state(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype,
                       int out_dtype, const csa_decode_state* st, bool hca) {
  if (!w || !st) return fail(CSA_ERR_ARG, "weights or state is NULL");
  if (B < 0) return fail(CSA_ERR_ARG, "B must be >= 0");
  if (!is_act_dtype(dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (B == 0) return CSA_OK;
  if (!pos || !aligned(pos, 8)) return fail(CSA_ERR_ARG, "pos must be an 8-byte aligned device array [B]");
  if (st->n_cap < 1 || st->n_cap > 0x7FFFFFFFLL) return fail(CSA_ERR_ARG, "state n_cap out of range");
  if (!st->entries || !st->win || !st->block || (!hca && !st->keys)) return fail(CSA_ERR_ARG, "NULL state pointer");
  if (st->entry_fmt != 0 && st->entry_fmt != 1) return fail(CSA_ERR_ARG, "entry_fmt must be 0 or 1");
  if (!hca && st->key_fmt != 0) {
    if (st->key_fmt != 1) return fail(CSA_ERR_ARG, "key_fmt must be 0 or 1");
    if (!st->key_scales) return fail(CSA_ERR_ARG, "MXFP4 keys need key_scales");
    if (dims->D_I % 32 || dims->D_I > append_max_dim()) return fail(CSA_ERR_ARG, "MXFP4 keys need D_I %% 32 == 0");
    if (!aligned(st->keys, 16)) return fail(CSA_ERR_ARG, "MXFP4 key codes must be 16-byte aligned");
  }
  if (st->entry_fmt && (dims->D != 512 || dtype != CSA_BF16))
    return fail(CSA_ERR_ARG, "entry records hold D = 512 and take bf16 entries");
  if (dims->D > append_max_dim() || dims->D % 2) return fail(CSA_ERR_UNSUPPORTED, "D must be even and <= %d", append_max_dim());
  if (!w->bias_a || (!hca && (!w->bias_b || !w->ibias_a || !w->ibias_b || !w->w_head)))
    return fail(CSA_ERR_ARG, "NULL weight pointer");
  return check_fid(w, dims->D);
}

}  // namespace

extern "C" {

int csa_version(void) { return 3; }

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
    case CSA_OP_SPARSE_ATTN_QK: {
      int rc = check_dims(dims);
      if (rc) return rc;
      const int dt = idx_dtype == CSA_F32 ? CSA_F32 : CSA_BF16;
      *bytes = (int64_t)(align256((size_t)B * T * dims->H * dims->D * esize(dt)) +
                         attn_workspace(sizing_attn(dims, B, T, dt)));
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
      IndexArgs a = make_index_args(dims, B, T, nullptr, idx_dtype, nullptr, 0, 0, nullptr, nullptr, 0, nullptr, 0,
                                    nullptr, n_cap, nullptr, nullptr);
      size_t need = index_topk_workspace(a);
      if (op == CSA_OP_FORWARD) {
        const int es = idx_dtype == CSA_F32 ? 4 : 2;
        const size_t at = attn_workspace(sizing_attn(dims, B, T, idx_dtype == CSA_F32 ? CSA_F32 : CSA_BF16));
        size_t scratch = need > at ? need : at;  // index / attention scratch, or the projection's
        if (idx_dtype == CSA_BF16 && scratch < kGemmWorkspace) scratch = kGemmWorkspace;
        const size_t nqi = (size_t)B * T * dims->H_I * dims->D_I;
        need = align256((size_t)B * T * n_tot_of(dims) * es) + align256((size_t)B * T * dims->top_k * 4) +
               align256(nqi / 2) + align256(nqi / 32) + align256(scratch);
      }
      *bytes = (int64_t)need;
      return CSA_OK;
    }
    default:
      return fail(CSA_ERR_ARG, "unknown op %d", op);
  }
}

int csa_compress(int B, int T, const int64_t* pos0, int m, int c, int in_dtype, const void* ca, const void* za,
                 const void* cb, const void* zb, int64_t ld, int64_t seq_stride, const void* halo_cb,
                 const void* halo_zb, int64_t halo_ld, int64_t halo_seq_stride, const float* bias_a,
                 const float* bias_b, void* entries, int64_t entries_seq_stride, int64_t n_cap, int out_dtype,
                 void* stream) {
  return compress_call("csa_compress", true, B, T, pos0, m, c, in_dtype, ca, za, cb, zb, ld, seq_stride, halo_cb,
                       halo_zb, halo_ld, halo_seq_stride, bias_a, bias_b, entries, entries_seq_stride, n_cap,
                       out_dtype, stream);
}

int csa_hca_compress(int B, int T, const int64_t* pos0, int m, int c, int in_dtype, const void* cv, const void* z,
                     int64_t ld, int64_t seq_stride, const float* bias, void* entries, int64_t entries_seq_stride,
                     int64_t n_cap, int out_dtype, void* stream) {
  // series b is not read without overlap
  return compress_call("csa_hca_compress", false, B, T, pos0, m, c, in_dtype, cv, z, cv, z, ld, seq_stride, nullptr,
                       nullptr, 0, 0, bias, bias, entries, entries_seq_stride, n_cap, out_dtype, stream);
}

int csa_index_topk(const csa_dims* dims, int B, int T, const int64_t* q_pos, int idx_dtype, const void* q_idx,
                   int64_t q_ld, int64_t q_seq_stride, const void* q_scale, const float* w, int64_t w_ld,
                   const void* keys, int64_t keys_seq_stride, const void* k_scale, int64_t n_cap, int32_t* out_idx,
                   float* out_score, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_index(dims, B, T, q_pos, idx_dtype, q_idx, q_ld, q_seq_stride, q_scale, w, w_ld, keys,
                          keys_seq_stride, k_scale, n_cap, out_idx);
  if (rc) return rc;
  if ((int64_t)B * T == 0) return CSA_OK;
  IndexArgs a = make_index_args(dims, B, T, q_pos, idx_dtype, q_idx, q_ld, q_seq_stride, q_scale, w, w_ld, keys,
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

int csa_sparse_attn(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype, const void* q,
                    int64_t q_ld, int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride,
                    int64_t n_cap, const int32_t* idx, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                    const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws,
                    size_t ws_bytes, void* stream) {
  return attn_call("csa_sparse_attn", false, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, entries,
                   entries_seq_stride, n_cap, idx, kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream);
}

int csa_sparse_attn_qk(const csa_dims* dims, const csa_weights* w, int B, int T, const int64_t* q_pos, int in_dtype,
                       const void* q, int64_t q_ld, int64_t q_seq_stride, const void* entries,
                       int64_t entries_seq_stride, int64_t n_cap, const int32_t* idx, const void* kv_raw,
                       int64_t raw_ld, int64_t raw_seq_stride, const int64_t* raw_pos, int64_t raw_len, void* out,
                       int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!w) return fail(CSA_ERR_ARG, "weights NULL");
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_fid(w, dims->D);
  if (rc) return rc;
  AttnArgs at{};
  rc = attn_prepare(false, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, entries, entries_seq_stride, n_cap, idx,
                    kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, w->sink, out, out_dtype, 0, 0, 0, &at);
  if (rc || (int64_t)B * T == 0) return rc;
  const int H = dims->H, D = dims->D;
  const bool fused = attn_try_fuse(at, w);
  const bool qpass = (w->gamma_q || w->rope_dims > 0) && !fused;
  // workspace: the normalised query (when the attention does not take the options) | attention scratch
  const size_t qbytes = align256((size_t)B * T * H * D * esize(in_dtype));
  rc = check_ws(ws, ws_bytes, qbytes + attn_workspace(at));
  if (rc) return rc;
  uint8_t* base = static_cast<uint8_t*>(ws);
  if (qpass) {
    rc = norm_rope_call(B, T, H, D, in_dtype, q, q_ld, q_seq_stride, base, (int64_t)H * D, (int64_t)T * H * D,
                        w->gamma_q, w->norm_eps, w->rope_dims, w->rope_theta, q_pos, 0, 1, 0, stream);
    if (rc) return rc;
    at.q = base;
    at.q_ld = (int64_t)H * D;
    at.q_seq_stride = (int64_t)T * H * D;
  }
  rc = attn_run("csa_sparse_attn_qk", at, base + qbytes, ws_bytes - qbytes, stream);
  if (rc) return rc;
  if (w->rope_dims > 0 && !fused) {
    rc = norm_rope_call(B, T, H, D, out_dtype, out, (int64_t)H * D, (int64_t)T * H * D, out, (int64_t)H * D,
                        (int64_t)T * H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, q_pos, 0, 1, 1, stream);
    if (rc) return rc;
  }
  g_err.clear();
  return CSA_OK;
}

int csa_sparse_attn_fp8(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype, const void* q,
                        int64_t q_ld, int64_t q_seq_stride, const void* records, int64_t records_seq_stride,
                        int64_t n_cap, const int32_t* idx, const void* kv_raw, int64_t raw_ld,
                        int64_t raw_seq_stride, const int64_t* raw_pos, int64_t raw_len, const float* sink,
                        void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  return attn_call("csa_sparse_attn_fp8", false, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, records,
                   records_seq_stride, n_cap, idx, kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream, 1);
}

int csa_dense_attn(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype, const void* q,
                   int64_t q_ld, int64_t q_seq_stride, const void* entries, int64_t entries_seq_stride,
                   int64_t n_cap, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                   const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out, int out_dtype, void* ws,
                   size_t ws_bytes, void* stream) {
  return attn_call("csa_dense_attn", true, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, entries,
                   entries_seq_stride, n_cap, nullptr, kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, sink, out,
                   out_dtype, ws, ws_bytes, stream);
}

int csa_dense_attn_fp8(const csa_dims* dims, int B, int T, const int64_t* q_pos, int in_dtype, const void* q,
                       int64_t q_ld, int64_t q_seq_stride, const void* records, int64_t records_seq_stride,
                       int64_t n_cap, const void* kv_raw, int64_t raw_ld, int64_t raw_seq_stride,
                       const int64_t* raw_pos, int64_t raw_len, const float* sink, void* out, int out_dtype,
                       void* ws, size_t ws_bytes, void* stream) {
  return attn_call("csa_dense_attn_fp8", true, dims, B, T, q_pos, in_dtype, q, q_ld, q_seq_stride, records,
                   records_seq_stride, n_cap, nullptr, kv_raw, raw_ld, raw_seq_stride, raw_pos, raw_len, sink, out,
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
  return hip_status(launch_entry_pack(a, static_cast<hipStream_t>(stream)), "csa_entry_pack");
}

int csa_mxfp4_quantize(int64_t R, int D, int dtype, const void* x, int64_t ld, void* codes, void* scales,
                       void* stream) {
  if (R < 0 || D < 1 || D % 32) return fail(CSA_ERR_ARG, "need R >= 0 and D a positive multiple of 32");
  if (!is_act_dtype(dtype)) return fail(CSA_ERR_ARG, "dtype must be F32 or BF16");
  if (ld < D) return fail(CSA_ERR_ARG, "ld < D");
  if (R == 0) return CSA_OK;
  if (!x || !codes || !scales) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  if (!aligned(codes, 4) || !aligned(x, esize(dtype))) return fail(CSA_ERR_ARG, "misaligned x or codes");
  QuantArgs a{};
  a.R = R;
  a.D = D;
  a.dtype = dtype;
  a.x = x;
  a.ld = ld;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = static_cast<uint8_t*>(scales);
  return hip_status(launch_mxfp4_quant(a, static_cast<hipStream_t>(stream)), "csa_mxfp4_quantize");
}

int csa_projection_gemm(int M, int N, int K, int in_dtype, const void* A, int64_t lda, const void* Wt, int64_t ldb,
                        void* C, int64_t ldc, int out_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 0) return fail(CSA_ERR_ARG, "M, N, K must be >= 0");
  if (!is_act_dtype(in_dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (lda < K || ldb < K || ldc < N) return fail(CSA_ERR_ARG, "strides below the row lengths");
  if ((int64_t)M * N == 0) return CSA_OK;
  if (!A || !Wt || !C) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.dtype = in_dtype;
  g.out_dtype = out_dtype;
  g.A = A;
  g.lda = lda;
  g.Bm = Wt;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)), "csa_projection_gemm");
}

int csa_norm_rope(int B, int R, int H, int D, int dtype, const void* x, int64_t x_ld, int64_t x_seq_stride, void* y,
                  int64_t y_ld, int64_t y_seq_stride, const float* gamma, float eps, int rope_dims, float rope_theta,
                  const int64_t* pos0, int64_t pos_off, int64_t pos_step, int inverse, void* stream) {
  return norm_rope_call(B, R, H, D, dtype, x, x_ld, x_seq_stride, y, y_ld, y_seq_stride, gamma, eps, rope_dims,
                        rope_theta, pos0, pos_off, pos_step, inverse, stream);
}

int csa_decode_step(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype, const void* q,
                    const void* q_idx, const void* kv, const void* comp, const csa_decode_state* st, void* out,
                    int out_dtype, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_decode_state(dims, w, B, pos, dtype, out_dtype, st, false);
  if (rc || B == 0) return rc;
  if (!q || !q_idx || !kv || !comp || !out) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  const int D = dims->D, DI = dims->D_I, H = dims->H, HI = dims->H_I, W = dims->window;
  const int64_t n_cap = st->n_cap;
  const DecodeWs L = decode_ws(dims, B, n_cap, dtype);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const bool qfid = w->gamma_q || w->rope_dims > 0;
  int32_t* idx = out_idx ? out_idx : reinterpret_cast<int32_t*>(base + L.idx);
  void* scratch = base + L.scratch;
  const size_t scratch_bytes = L.total - L.scratch;
  // the attention reads the window straight from the ring; where it takes the query's norm and
  // rotation itself (and turns the output back), the append leaves the query alone
  AttnArgs at{};
  rc = attn_prepare(false, dims, B, 1, pos, dtype, q, (int64_t)H * D, (int64_t)H * D, st->entries,
                    n_cap * (st->entry_fmt ? (int64_t)kEntryRecordBytes : D), n_cap, idx, st->win, D, (int64_t)W * D,
                    nullptr, 0, w->sink, out, out_dtype, st->entry_fmt, W, 0, &at);
  if (rc) return rc;
  const bool fused = attn_try_fuse(at, w);
  const bool qpass = qfid && !fused;
  // the token joins the state; a completed block's entry and key are pooled; the query is
  // normalised and rotated at its position unless the attention does it (and, for MXFP4 keys, the
  // indexer query is quantised)
  const bool kfp4 = st->key_fmt != 0;
  rc = decode_append("csa_decode_step", dims, w, B, pos, dtype, q, kv, comp, st, false, qpass ? base + L.q : nullptr, s,
                     q_idx, base + L.qi, base + L.qis);
  if (rc) return rc;
  if (qpass) at.q = base + L.q;
  if (kfp4)
    rc = csa_index_topk(dims, B, 1, pos, CSA_MXFP4, base + L.qi, 0, 0, base + L.qis, w->w_head, 0, st->keys, 0,
                        st->key_scales, n_cap, idx, nullptr, scratch, scratch_bytes, stream);
  else
    rc = csa_index_topk(dims, B, 1, pos, dtype, q_idx, (int64_t)HI * DI, (int64_t)HI * DI, nullptr, w->w_head, 0,
                        st->keys, n_cap * DI, nullptr, n_cap, idx, nullptr, scratch, scratch_bytes, stream);
  if (rc) return rc;
  rc = attn_run("csa_decode_step", at, scratch, scratch_bytes, stream);
  if (rc) return rc;
  if (w->rope_dims > 0 && !fused) {
    rc = norm_rope_call(B, 1, H, D, out_dtype, out, (int64_t)H * D, (int64_t)H * D, out, (int64_t)H * D,
                        (int64_t)H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos, 0, 1, 1, stream);
    if (rc) return rc;
  }
  g_err.clear();
  return CSA_OK;
}

int csa_decode_step_noalloc(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype,
                            const void* q, const void* q_idx, const void* kv, const void* comp,
                            const csa_decode_state* st, void* out, int out_dtype, int32_t* out_idx, void* stream) {
  // every host-side check of csa_decode_step first, then the size of what the step needs
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_decode_state(dims, w, B, pos, dtype, out_dtype, st, false);
  if (rc || B == 0) return rc;
  if (!q || !q_idx || !kv || !comp || !out) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  const size_t need = decode_ws(dims, B, st->n_cap, dtype).total;
  if (need > (size_t)CSA_STATIC_SCRATCH_BYTES)
    return fail(CSA_ERR_WORKSPACE, "csa_decode_step_noalloc: the step needs %zu bytes of scratch, above the %zu "
                "bytes the library holds per GPU (use csa_decode_step with a workspace)", need,
                (size_t)CSA_STATIC_SCRATCH_BYTES);
  void* ptr = nullptr;
  hipError_t e = static_scratch(&ptr);
  if (e != hipSuccess) return hip_status(e, "csa_decode_step_noalloc: scratch address");
  return csa_decode_step(dims, w, B, pos, dtype, q, q_idx, kv, comp, st, out, out_dtype, out_idx, ptr,
                         (size_t)CSA_STATIC_SCRATCH_BYTES, stream);
}

int csa_hca_decode_step(const csa_dims* dims, const csa_weights* w, int B, const int64_t* pos, int dtype,
                        const void* q, const void* kv, const void* comp, const csa_decode_state* st, void* out,
                        int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims, false);
  if (rc) return rc;
  rc = check_decode_state(dims, w, B, pos, dtype, out_dtype, st, true);
  if (rc || B == 0) return rc;
  if (!q || !kv || !comp || !out) return fail(CSA_ERR_ARG, "NULL tensor pointer");
  const int D = dims->D, H = dims->H, W = dims->window;
  const int64_t n_cap = st->n_cap;
  const DecodeWs L = hca_decode_ws(dims, B, n_cap, dtype);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const bool qfid = w->gamma_q || w->rope_dims > 0;
  AttnArgs at{};
  rc = attn_prepare(true, dims, B, 1, pos, dtype, q, (int64_t)H * D, (int64_t)H * D, st->entries,
                    n_cap * (st->entry_fmt ? (int64_t)kEntryRecordBytes : D), n_cap, nullptr, st->win, D,
                    (int64_t)W * D, nullptr, 0, w->sink, out, out_dtype, st->entry_fmt, W, 0, &at);
  if (rc) return rc;
  const bool fused = attn_try_fuse(at, w);
  const bool qpass = qfid && !fused;
  rc = decode_append("csa_hca_decode_step", dims, w, B, pos, dtype, q, kv, comp, st, true,
                     qpass ? base + L.q : nullptr, s);
  if (rc) return rc;
  if (qpass) at.q = base + L.q;
  rc = attn_run("csa_hca_decode_step", at, base + L.scratch, L.total - L.scratch, stream);
  if (rc) return rc;
  if (w->rope_dims > 0 && !fused) {
    rc = norm_rope_call(B, 1, H, D, out_dtype, out, (int64_t)H * D, (int64_t)H * D, out, (int64_t)H * D,
                        (int64_t)H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos, 0, 1, 1, stream);
    if (rc) return rc;
  }
  g_err.clear();
  return CSA_OK;
}

int csa_forward(const csa_dims* dims, const csa_weights* w, int B, int T, const int64_t* pos0, int d_model, int dtype,
                const void* x, const csa_cache* cache, void* out, int out_dtype, int32_t* out_idx, void* ws,
                size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!w || !cache) return fail(CSA_ERR_ARG, "weights or cache is NULL");
  if (B < 0 || T < 0 || d_model < 1) return fail(CSA_ERR_ARG, "bad B/T/d_model");
  if (!is_act_dtype(dtype) || !is_act_dtype(out_dtype)) return fail(CSA_ERR_ARG, "dtypes must be F32 or BF16");
  if (!pos_ok(pos0)) return fail(CSA_ERR_ARG, "pos0 must be 8-byte aligned");
  const int m = dims->m, D = dims->D, DI = dims->D_I, H = dims->H, HI = dims->H_I, W = dims->window, k = dims->top_k;
  if ((int64_t)B * T == 0) return CSA_OK;
  if (!x || !out || !w->w_proj || !w->bias_a || !w->bias_b || !w->ibias_a || !w->ibias_b || !w->w_head)
    return fail(CSA_ERR_ARG, "NULL weight/input pointer");
  if (!cache->entries || !cache->keys || !cache->win) return fail(CSA_ERR_ARG, "NULL cache pointer");
  if (cache->n_cap < 0) return fail(CSA_ERR_ARG, "n_cap must be >= 0");
  if (!pos0 && T / m > cache->n_cap) return fail(CSA_ERR_ARG, "T/m exceeds n_cap");
  if ((int64_t)W - 1 + T > cache->win_cap) return fail(CSA_ERR_ARG, "window - 1 + T exceeds win_cap");
  if (pos0 && !cache->halo) return fail(CSA_ERR_ARG, "per-sequence positions need cache->halo");
  if (cache->halo_out && T % m) return fail(CSA_ERR_ARG, "halo_out needs T %% m == 0");
  rc = check_fid(w, D);
  if (rc) return rc;
  const bool fid = fid_on(w);
  const bool records = cache->entry_fmt != 0;
  const bool kfp4 = cache->key_fmt != 0;
  if (cache->entry_fmt != 0 && cache->entry_fmt != 1) return fail(CSA_ERR_ARG, "entry_fmt must be 0 or 1");
  if (cache->key_fmt != 0 && cache->key_fmt != 1) return fail(CSA_ERR_ARG, "key_fmt must be 0 or 1");
  if (kfp4 && (!cache->key_scales || DI % 32 || !aligned(cache->keys, 16) || !aligned(cache->key_scales, 4)))
    return fail(CSA_ERR_ARG, "MXFP4 keys need key_scales (4-byte aligned), D_I %% 32 == 0 and 16-byte aligned codes");
  if (records && (D != 512 || dtype != CSA_BF16)) return fail(CSA_ERR_ARG, "entry records hold D = 512 bf16 entries");
  const int64_t ntot = n_tot_of(dims);
  const int es = esize(dtype);
  // workspace: P [B*T, ntot] | idx [B*T, k] | q_I in MXFP4 (codes, scales) | index / attention /
  // projection scratch
  IndexArgs probe = make_index_args(dims, B, T, pos0, kfp4 ? CSA_MXFP4 : dtype, nullptr, 0, 0, nullptr, nullptr, 0,
                                    nullptr, 0, nullptr, cache->n_cap, nullptr, nullptr);
  const size_t p_bytes = align256((size_t)B * T * ntot * es);
  const size_t nqi = (size_t)B * T * HI * DI;
  const size_t i_bytes = align256((size_t)B * T * k * 4) + align256(nqi / 2) + align256(nqi / 32);
  const size_t i_ws = index_topk_workspace(probe);
  const size_t a_ws = attn_workspace(sizing_attn(dims, B, T, dtype));
  size_t scratch = i_ws > a_ws ? i_ws : a_ws;
  if (dtype == CSA_BF16 && scratch < kGemmWorkspace) scratch = kGemmWorkspace;
  const size_t x_bytes = align256(scratch);
  rc = check_ws(ws, ws_bytes, p_bytes + i_bytes + x_bytes);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(w->w_proj, 16)) return fail(CSA_ERR_ARG, "x and w_proj must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* P = static_cast<uint8_t*>(ws);
  int32_t* idx = out_idx ? out_idx : reinterpret_cast<int32_t*>(P + p_bytes);
  uint8_t* qi_codes = P + p_bytes + align256((size_t)B * T * k * 4);
  uint8_t* qi_scales = qi_codes + align256(nqi / 2);
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

  // new entries into their cache rows (pos0[b]/m ..), normalised, rotated and packed into records in
  // the compressor's epilogue when the layer has those options
  CompressArgs epi{};
  epi.epilogue = fid || records;
  epi.gamma = w->gamma_kv;
  epi.eps = w->norm_eps;
  epi.rope_dims = w->rope_dims;
  epi.theta = w->rope_theta;
  epi.records = records;
  rc = compress_call("csa_forward", true, B, T, pos0, m, D, dtype, col(c_ca), col(c_za), col(c_cb), col(c_zb), ntot,
                     (int64_t)T * ntot, halo, halo ? halo + (size_t)D * es : nullptr, halo_ld, (int64_t)m * halo_ld,
                     w->bias_a, w->bias_b, cache->entries,
                     cache->n_cap * (records ? (int64_t)kEntryRecordBytes : D), cache->n_cap, dtype, stream, &epi);
  if (rc) return rc;
  // new indexer keys: rows of the activation dtype, or quantised to MXFP4 in the epilogue
  CompressArgs kepi{};
  kepi.epilogue = kfp4;
  kepi.fp4_codes = kfp4 ? static_cast<uint8_t*>(cache->keys) : nullptr;
  kepi.fp4_scales = kfp4 ? static_cast<uint8_t*>(cache->key_scales) : nullptr;
  rc = compress_call("csa_forward", true, B, T, pos0, m, DI, dtype, col(c_ica), col(c_iza), col(c_icb), col(c_izb),
                     ntot, (int64_t)T * ntot, halo ? halo + (size_t)2 * D * es : nullptr,
                     halo ? halo + (size_t)(2 * D + DI) * es : nullptr, halo_ld, (int64_t)m * halo_ld, w->ibias_a,
                     w->ibias_b, cache->keys, cache->n_cap * DI, cache->n_cap, dtype, stream, &kepi);
  if (rc) return rc;
  // the chunk's raw KV goes to window rows [W-1, W-1+T) (normalised and rotated on the way when on)
  void* wrows = static_cast<uint8_t*>(cache->win) + (size_t)(W - 1) * D * es;
  if (w->gamma_kv || w->rope_dims > 0) {
    rc = norm_rope_call(B, T, 1, D, dtype, col(c_kv), ntot, (int64_t)T * ntot, wrows, D, cache->win_cap * D,
                        w->gamma_kv, w->norm_eps, w->rope_dims, w->rope_theta, pos0, 0, 1, 0, stream);
    if (rc) return rc;
  } else {
    e = launch_copy_rows(B, T, D, es, col(c_kv), ntot, (int64_t)T * ntot, wrows, D, cache->win_cap * D, s);
    if (e != hipSuccess) return hip_status(e, "csa_forward: window copy");
  }
  // window row r of sequence b holds position pos0[b] - (W - 1) + r; the attention takes the queries'
  // norm and rotation (and turns the output back) where its kernels can, else the queries are
  // normalised in place in the projection buffer
  AttnArgs at{};
  rc = attn_prepare(false, dims, B, T, pos0, dtype, col(c_q), ntot, (int64_t)T * ntot, cache->entries,
                    cache->n_cap * (records ? (int64_t)kEntryRecordBytes : D), cache->n_cap, idx, cache->win, D,
                    cache->win_cap * D, pos0, (int64_t)W - 1 + T, w->sink, out, out_dtype, records ? 1 : 0, 0,
                    -(int64_t)(W - 1), &at);
  if (rc) return rc;
  const bool fused = attn_try_fuse(at, w);
  if ((w->gamma_q || w->rope_dims > 0) && !fused) {
    rc = norm_rope_call(B, T, H, D, dtype, col(c_q), ntot, (int64_t)T * ntot, col(c_q), ntot, (int64_t)T * ntot,
                        w->gamma_q, w->norm_eps, w->rope_dims, w->rope_theta, pos0, 0, 1, 0, stream);
    if (rc) return rc;
  }
  if (kfp4) {  // the indexer queries to MXFP4, then the FP4 indexer
    QuantArgs qa{};
    qa.R = (int64_t)B * T;
    qa.D = HI * DI;
    qa.dtype = dtype;
    qa.x = col(c_qi);
    qa.ld = ntot;
    qa.codes = qi_codes;
    qa.scales = qi_scales;
    e = launch_mxfp4_quant(qa, s);
    if (e != hipSuccess) return hip_status(e, "csa_forward: q_I quantisation");
    rc = csa_index_topk(dims, B, T, pos0, CSA_MXFP4, qi_codes, 0, 0, qi_scales, w->w_head, 0, cache->keys, 0,
                        cache->key_scales, cache->n_cap, idx, nullptr, xws, x_bytes, stream);
  } else {
    rc = csa_index_topk(dims, B, T, pos0, dtype, col(c_qi), ntot, (int64_t)T * ntot, nullptr, w->w_head, 0,
                        cache->keys, cache->n_cap * DI, nullptr, cache->n_cap, idx, nullptr, xws, x_bytes, stream);
  }
  if (rc) return rc;
  rc = attn_run("csa_forward", at, xws, x_bytes, stream);
  if (rc) return rc;
  if (w->rope_dims > 0 && !fused) {
    rc = norm_rope_call(B, T, H, D, out_dtype, out, (int64_t)H * D, (int64_t)T * H * D, out, (int64_t)H * D,
                        (int64_t)T * H * D, nullptr, 0.f, w->rope_dims, w->rope_theta, pos0, 0, 1, 1, stream);
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
