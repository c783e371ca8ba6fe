// Ceiling probes (include/csa_probe.h): HBM read bandwidth with 16-byte loads, the read of rows
// gathered by index (the attention's access pattern), and the bf16 MFMA rate of four independent
// 32x32x16 chains per wave at eight waves per compute unit.
#include "csa_probe.h"

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace csa {

namespace {

constexpr int kProbeThreads = 512;  // eight waves per workgroup
int probe_grid() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;  // one eight-wave workgroup per compute unit
}

__global__ void __launch_bounds__(kProbeThreads) probe_read(const uint4* buf, int64_t n16, uint32_t* sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  // four loads in flight per thread before any is used
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[tid] = acc;
}

// one wave per gathered row, four rows in flight per wave; row numbers are clamped into the buffer
__global__ void __launch_bounds__(kProbeThreads) probe_gather(const uint8_t* buf, int64_t buf_rows, int row16,
                                                              const int32_t* idx, int64_t n_rows, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  auto row_ptr = [&](int64_t r) {
    int64_t i = idx[r];
    i = i < 0 ? 0 : (i >= buf_rows ? buf_rows - 1 : i);
    return reinterpret_cast<const uint4*>(buf + i * (int64_t)row16 * 16);
  };
  uint32_t acc = 0;
  int64_t r = wave;
  for (; r + 3 * nw < n_rows; r += 4 * nw) {
    const uint4 *p0 = row_ptr(r), *p1 = row_ptr(r + nw), *p2 = row_ptr(r + 2 * nw), *p3 = row_ptr(r + 3 * nw);
    for (int j = lane; j < row16; j += 64) {
      const uint4 a = p0[j], b = p1[j], c = p2[j], d = p3[j];
      acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
  }
  for (; r < n_rows; r += nw) {
    const uint4* p0 = row_ptr(r);
    for (int j = lane; j < row16; j += 64) {
      const uint4 a = p0[j];
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(kProbeThreads) probe_mfma(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((lane * 3 + j) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  s = wave_sum(s);
  if (lane == 0) sink[wave] = s;
}

}  // namespace

}  // namespace csa

extern "C" {

size_t csa_probe_sink_words(void) { return (size_t)csa::probe_grid() * csa::kProbeThreads; }

int csa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return csa::probe_fail("csa_probe_hbm_read: buf must be 16-byte aligned, bytes a multiple of 16, sink non-NULL");
  hipLaunchKernelGGL(csa::probe_read, dim3((unsigned)csa::probe_grid()), dim3(csa::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return csa::probe_status(hipGetLastError(), "csa_probe_hbm_read");
}

int csa_probe_gather_read(const void* buf, size_t buf_bytes, size_t row_bytes, const int32_t* idx, int64_t n_rows,
                          uint32_t* sink, void* stream) {
  if (!buf || !sink || !idx || n_rows < 0 || row_bytes < 16 || row_bytes % 16 || row_bytes > (1u << 20) ||
      buf_bytes < row_bytes || reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(idx) % 4)
    return csa::probe_fail("csa_probe_gather_read: buf 16-byte aligned with at least one row, row_bytes a multiple of "
                           "16 (<= 1 MiB), idx 4-byte aligned, n_rows >= 0 and a sink are required");
  if (n_rows == 0) return 0;
  hipLaunchKernelGGL(csa::probe_gather, dim3((unsigned)csa::probe_grid()), dim3(csa::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf),
                     (int64_t)(buf_bytes / row_bytes), (int)(row_bytes / 16), idx, n_rows, sink);
  return csa::probe_status(hipGetLastError(), "csa_probe_gather_read");
}

int csa_probe_mfma_bf16(int iters, float* sink, void* stream) {
  if (iters < 1 || !sink) return csa::probe_fail("csa_probe_mfma_bf16: iters >= 1 and a sink are required");
  hipLaunchKernelGGL(csa::probe_mfma, dim3((unsigned)csa::probe_grid()), dim3(csa::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  return csa::probe_status(hipGetLastError(), "csa_probe_mfma_bf16");
}

}  // extern "C"
