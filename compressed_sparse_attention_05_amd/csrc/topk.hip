// Step 3 on materialised scores: exact top-k of each row, ties toward the smaller column.
//
// Short rows: one wave per row runs the streaming selection (topk_wave.h) straight to the output.
// Long rows: the row is cut into segments; one wave per segment keeps that segment's k best keys
// (every global top-k key is among its segment's top k), then one wave per row selects among the
// segment survivors. Both passes use the same exact key order, so the result does not depend on
// the segmentation.
#include "kernels.h"
#include "topk_wave.h"

namespace csa {

namespace {

constexpr int kWaves = 4;          // waves (rows or segments) per workgroup
constexpr int kSegLen = 8192;      // scores per segment in the segmented pass
constexpr int kDirectMax = 16384;  // rows up to this length are selected in one pass

int lds_bytes(int cap) { return kWaves * (cap * 8 + 256 * 4); }

__global__ void __launch_bounds__(kWaves * 64) topk_rows_kernel(TopkArgs a, int cap) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= a.R) return;
  uint64_t* buf = reinterpret_cast<uint64_t*>(smem) + (int64_t)wave * cap;
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(smem) + kWaves * cap) + wave * 256;
  int64_t nv = a.n_valid[row];
  nv = nv < 0 ? 0 : (nv > a.ld ? a.ld : nv);
  const float* s = a.scores + row * a.ld;
  WaveTopK tk;
  tk.init(buf, hist, cap, a.k);
  for (int64_t base = 0; base < nv; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < nv;
    const float v = valid ? s[i] : 0.f;
    tk.offer(make_cand(v, (uint32_t)i), valid);
  }
  tk.finish(a.out_idx + row * a.k, a.out_score ? a.out_score + row * a.k : nullptr);
}

// Pass 1 of long rows: segment (row, seg) keeps its top k keys in cand[row][seg][0..k),
// padded with 0 (below every real key).
__global__ void __launch_bounds__(kWaves * 64) topk_segments_kernel(TopkArgs a, int cap, int nseg,
                                                                     uint64_t* cand) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t gid = (int64_t)blockIdx.x * kWaves + wave;
  if (gid >= (int64_t)a.R * nseg) return;
  const int64_t row = gid / nseg;
  const int seg = (int)(gid % nseg);
  uint64_t* buf = reinterpret_cast<uint64_t*>(smem) + (int64_t)wave * cap;
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(smem) + kWaves * cap) + wave * 256;
  int64_t nv = a.n_valid[row];
  nv = nv < 0 ? 0 : (nv > a.ld ? a.ld : nv);
  const int64_t lo = (int64_t)seg * kSegLen;
  const int64_t hi = lo + kSegLen < nv ? lo + kSegLen : nv;
  const float* s = a.scores + row * a.ld;
  WaveTopK tk;
  tk.init(buf, hist, cap, a.k);
  for (int64_t base = lo; base < hi; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < hi;
    const float v = valid ? s[i] : 0.f;
    tk.offer(make_cand(v, (uint32_t)i), valid);
  }
  if (tk.cnt > tk.k) tk.shrink();
  uint64_t* out = cand + gid * a.k;
  for (int j = lane; j < a.k; j += 64) out[j] = j < tk.cnt ? buf[j] : 0ull;
}

// Pass 2: one wave per row selects among nseg * k survivor keys (zeros are padding).
__global__ void __launch_bounds__(kWaves * 64) topk_merge_kernel(TopkArgs a, int cap, int nseg,
                                                                  const uint64_t* cand) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= a.R) return;
  uint64_t* buf = reinterpret_cast<uint64_t*>(smem) + (int64_t)wave * cap;
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(smem) + kWaves * cap) + wave * 256;
  const uint64_t* c = cand + row * (int64_t)nseg * a.k;
  const int64_t n = (int64_t)nseg * a.k;
  WaveTopK tk;
  tk.init(buf, hist, cap, a.k);
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t i = base + lane;
    const uint64_t key = i < n ? c[i] : 0ull;
    tk.offer(key, key != 0ull);
  }
  tk.finish(a.out_idx + row * a.k, a.out_score ? a.out_score + row * a.k : nullptr);
}

}  // namespace

size_t topk_workspace(int R, int64_t n, int k) {
  if (n <= kDirectMax) return 0;
  const int64_t nseg = ceil_div(n, kSegLen);
  return (size_t)R * nseg * k * sizeof(uint64_t);
}

hipError_t launch_topk_from_scores(const TopkArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  const int cap = topk_cap_for(a.k, 512);
  const int lds = lds_bytes(cap);
  hipError_t e;
  if (a.ld <= kDirectMax) {
    if ((e = allow_lds((const void*)topk_rows_kernel, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)ceil_div(a.R, kWaves)), dim3(kWaves * 64), lds, s, a, cap);
    return hipGetLastError();
  }
  const int nseg = (int)ceil_div(a.ld, kSegLen);
  if (ws_bytes < topk_workspace(a.R, a.ld, a.k) || ws == nullptr) return hipErrorInvalidValue;
  uint64_t* cand = static_cast<uint64_t*>(ws);
  if ((e = allow_lds((const void*)topk_segments_kernel, lds)) != hipSuccess) return e;
  if ((e = allow_lds((const void*)topk_merge_kernel, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_segments_kernel, dim3((unsigned)ceil_div((int64_t)a.R * nseg, kWaves)),
                     dim3(kWaves * 64), lds, s, a, cap, nseg, cand);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)ceil_div(a.R, kWaves)), dim3(kWaves * 64), lds, s, a,
                     cap, nseg, (const uint64_t*)cand);
  return hipGetLastError();
}

}  // namespace csa
