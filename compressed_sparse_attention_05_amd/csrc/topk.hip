// Step 3 on materialised scores: exact top-k of each row, ties toward the smaller column.
//
// Short rows: one wave per row runs the streaming selection (topk_wave.h) straight to the output.
// Long rows: select.hip (group-maximum lower bound, candidates, exact selection among them). All use
// the same exact key order.
#include "kernels.h"
#include "topk_wave.h"

namespace csa {

namespace {

constexpr int kWaves = 4;          // waves (rows or segments) per workgroup
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

}  // namespace

size_t topk_workspace(int R, int64_t n, int k) {
  if (n <= kDirectMax) return 0;
  return select_workspace(R, n, k);
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
  if (ws_bytes < topk_workspace(a.R, a.ld, a.k) || ws == nullptr) return hipErrorInvalidValue;
  return launch_select(a.scores, a.ld, a.n_valid, a.R, a.k, a.out_idx, a.out_score, ws, false, s);
}

}  // namespace csa
