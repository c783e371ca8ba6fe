// The 584-byte compressed-entry record ("Anatomy of a Frontier Model", section "The KV cache,
// recomputed"; layout and rounding in record.h): one wave per entry, lane l holding dims 8l..8l+7.
#include "kernels.h"
#include "record.h"

namespace csa {

namespace {

constexpr int kPackWaves = 4;

template <int DT>
__global__ void __launch_bounds__(kPackWaves * 64) entry_pack_kernel(EntryPackArgs a) {
  const int lane = lane_id();
  const int64_t ent = (int64_t)blockIdx.x * kPackWaves + (threadIdx.x >> 6);
  if (ent >= (int64_t)a.B * a.N) return;
  const int64_t b = ent / a.N, n = ent % a.N;
  const int64_t src = b * a.seq_stride + n * a.ld + 8 * lane;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = load_elem<DT>(a.entries, src + j);
  pack_record_wave(v, static_cast<uint8_t*>(a.records) + b * a.rec_seq_stride + n * kEntryRecordBytes);
}

}  // namespace

hipError_t launch_entry_pack(const EntryPackArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.N;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, kPackWaves));
  if (a.dtype == CSA_BF16)
    hipLaunchKernelGGL(entry_pack_kernel<CSA_BF16>, grid, dim3(kPackWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(entry_pack_kernel<CSA_F32>, grid, dim3(kPackWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
