// MXFP4 quantisation of rows of float32 / bf16 values (the indexer's FP4 keys and queries, "Anatomy
// of a Frontier Model", sections "The KV cache, recomputed" and "Precision: FP8 everywhere, FP4
// experts"; the conversion rule is in mx.h).
//
// HBM-bound: each element is read once (2 or 4 bytes) and leaves as half a byte plus 1/32 of a scale
// byte. A thread owns 8 consecutive elements (one 16-byte load in bf16), four consecutive lanes make a
// block of 32 and meet through a two-step butterfly for its maximum.
#include "kernels.h"
#include "mx.h"

namespace csa {

namespace {

template <int DT>
__global__ void __launch_bounds__(256) mxfp4_quant_kernel(QuantArgs a, bool vec) {
  const int64_t per_row = a.D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= a.R * per_row) return;  // whole blocks: per_row is a multiple of 4
  const int64_t row = gid / per_row;
  const int j0 = (int)(gid % per_row) * 8;
  const int64_t off = row * a.ld + j0;
  float v[8];
  if (vec) {
    if constexpr (DT == CSA_BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + off);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
      const float4 u0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + off);
      const float4 u1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + off + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = load_elem<DT>(a.x, off + j);
  }
  int X;
  const uint32_t pk = mxfp4_quant_lanes<8>(v, X);
  mxfp4_store_lanes<8>(a.codes + row * (a.D / 2), a.scales + row * (a.D / 32), j0, pk, X);
}

}  // namespace

hipError_t launch_mxfp4_quant(const QuantArgs& a, hipStream_t s) {
  if (a.R <= 0 || a.D <= 0) return hipSuccess;
  if (a.D % 32) return hipErrorInvalidValue;
  const int es = a.dtype == CSA_BF16 ? 2 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && ((a.ld * es) % 16 == 0);
  const int64_t threads = a.R * (a.D / 8);
  const dim3 grid((unsigned)ceil_div(threads, 256));
  if (a.dtype == CSA_BF16) hipLaunchKernelGGL(mxfp4_quant_kernel<CSA_BF16>, grid, dim3(256), 0, s, a, vec);
  else hipLaunchKernelGGL(mxfp4_quant_kernel<CSA_F32>, grid, dim3(256), 0, s, a, vec);
  return hipGetLastError();
}

}  // namespace csa
