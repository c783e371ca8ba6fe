// The fused projection x @ W^T that feeds the layer (compressor series and logits, indexer
// compressor, queries, indexer queries, raw window KV: one GEMM over the concatenated weights).
// The pages give no projection; the layer needs these per-token vectors, so one dense GEMM makes
// them all in one pass over x.
//
// bf16 path: 128 x 128 output tile per workgroup of 4 waves (2 x 2, 64 x 64 each), K in steps of
// 64 through double-buffered LDS (rows padded to 72 elements so the MFMA fragment reads are
// conflict-free), v_mfma_f32_32x32x16_bf16 with fp32 accumulation, bf16 (RNE) or fp32 output.
// Tiles are handed out so that each XCD works on a contiguous band of the tile grid, with the
// M index fastest, so the workgroups that share a weight panel run together on one L2.
// fp32 path: a plain one-output-per-thread kernel (small layers only).
#include "kernels.h"

namespace csa {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDS_K = BK + 8;

template <int OT>
__global__ void __launch_bounds__(256) gemm_bf16_mfma(GemmArgs g, int tiles_m, int tiles_n) {
  __shared__ __align__(16) uint16_t As[2][BM][LDS_K];
  __shared__ __align__(16) uint16_t Bs[2][BN][LDS_K];
  const int ntiles = tiles_m * tiles_n;
  // XCD-aware order: blocks are dispatched round-robin over the 8 XCDs; give XCD x the tile
  // band [x*ntiles/8, (x+1)*ntiles/8).
  int tile = blockIdx.x;
  if (ntiles % 8 == 0) tile = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* Bm = static_cast<const uint16_t*>(g.Bm);

  uint4 ra[4], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * 256;           // 1024 chunks of 16 B per operand tile
      const int r = c >> 3, c8 = c & 7;
      const int64_t am = m0 + r, bn = n0 + r;
      ra[j] = am < g.M ? *reinterpret_cast<const uint4*>(A + am * g.lda + k0 + c8 * 8) : make_uint4(0, 0, 0, 0);
      rb[j] = bn < g.N ? *reinterpret_cast<const uint4*>(Bm + bn * g.ldb + k0 + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + j * 256;
      const int r = c >> 3, c8 = c & 7;
      *reinterpret_cast<uint4*>(&As[buf][r][c8 * 8]) = ra[j];
      *reinterpret_cast<uint4*>(&Bs[buf][r][c8 * 8]) = rb[j];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = g.K / BK;
  fetch(0);
  put(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][wm * 64 + i * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][wn * 64 + j * 32 + (lane & 31)][ks * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) put(cur ^ 1);
    __syncthreads();
  }
  // acc[i][j][r]: row wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4, col wn*64 + j*32 + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (row >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (col < g.N) store_elem<OT>(g.C, row * g.ldc + col, acc[i][j][r]);
      }
    }
}

template <int DT, int OT>
__global__ void __launch_bounds__(256) gemm_scalar(GemmArgs g) {
  const int64_t col = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t row = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= g.M || col >= g.N) return;
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc = fmaf(load_elem<DT>(g.A, row * g.lda + k), load_elem<DT>(g.Bm, col * g.ldb + k), acc);
  store_elem<OT>(g.C, row * g.ldc + col, acc);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const bool mfma_ok = g.dtype == CSA_BF16 && g.K % BK == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
                       (reinterpret_cast<uintptr_t>(g.A) & 15) == 0 && (reinterpret_cast<uintptr_t>(g.Bm) & 15) == 0;
  if (mfma_ok) {
    const int tm = (int)ceil_div(g.M, BM), tn = (int)ceil_div(g.N, BN);
    if (g.out_dtype == CSA_BF16)
      hipLaunchKernelGGL(gemm_bf16_mfma<CSA_BF16>, dim3((unsigned)(tm * tn)), dim3(256), 0, s, g, tm, tn);
    else
      hipLaunchKernelGGL(gemm_bf16_mfma<CSA_F32>, dim3((unsigned)(tm * tn)), dim3(256), 0, s, g, tm, tn);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)ceil_div(g.N, 64), (unsigned)ceil_div(g.M, 4));
  if (g.dtype == CSA_F32 && g.out_dtype == CSA_F32)
    hipLaunchKernelGGL((gemm_scalar<CSA_F32, CSA_F32>), grid, dim3(256), 0, s, g);
  else if (g.dtype == CSA_F32)
    hipLaunchKernelGGL((gemm_scalar<CSA_F32, CSA_BF16>), grid, dim3(256), 0, s, g);
  else if (g.out_dtype == CSA_F32)
    hipLaunchKernelGGL((gemm_scalar<CSA_BF16, CSA_F32>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_scalar<CSA_BF16, CSA_BF16>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace csa
