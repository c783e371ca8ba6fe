// The layer's input projection P = x W^T is a plain dense GEMM (no fusion with the CSA steps), so
// in bf16 it goes to hipBLASLt: C[M, N] = A[M, K] B[N, K]^T, bf16 operands and output, fp32
// accumulation. One handle per device and one algorithm per shape, chosen once by the library's
// heuristic and reused, so a shape always runs the same kernel. Host code only.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kernels.h"

namespace csa {

namespace {

struct LtPlan {
  bool ok = false;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

using PlanKey = std::tuple<int, int, int, int, int64_t, int64_t, int64_t>;  // device, M, N, K, lda, ldb, ldc

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<PlanKey, LtPlan> g_plans;

// Column-major view: C^T[N, M] = B[N, K] (stored as K x N, transposed) * A^T (stored K x M).
LtPlan make_plan(hipblasLtHandle_t h, const GemmArgs& g) {
  LtPlan p;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return p;
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  if (hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, g.K, g.N, g.ldb) != HIPBLAS_STATUS_SUCCESS) return p;
  if (hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, g.K, g.M, g.lda) != HIPBLAS_STATUS_SUCCESS) return p;
  if (hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, g.N, g.M, g.ldc) != HIPBLAS_STATUS_SUCCESS) return p;
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return p;
  const uint64_t max_ws = kGemmWorkspace;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws, sizeof(max_ws));
  // the heuristic's ranking, first candidate whose workspace fits
  constexpr int kCand = 8;
  hipblasLtMatmulHeuristicResult_t res[kCand];
  int n = 0;
  const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, kCand, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS) return p;
  for (int i = 0; i < n; ++i) {
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWorkspace) {
      p.algo = res[i].algo;
      p.ws = res[i].workspaceSize;
      p.ok = true;
      break;
    }
  }
  return p;
}

}  // namespace

bool gemm_library_eligible(const GemmArgs& g) {
  return g.dtype == CSA_BF16 && g.out_dtype == CSA_BF16 && g.M > 0 && g.N > 0 && g.K > 0;
}

hipError_t launch_gemm_library(const GemmArgs& g, void* ws, size_t ws_bytes, hipStream_t s, bool* done) {
  *done = false;
  if (!gemm_library_eligible(g) || ws == nullptr || ws_bytes < kGemmWorkspace) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  LtPlan plan;
  hipblasLtHandle_t h = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto hi = g_handles.find(dev);
    if (hi == g_handles.end()) {
      if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return hipSuccess;  // own kernel instead
      g_handles[dev] = h;
    } else {
      h = hi->second;
    }
    const PlanKey key{dev, g.M, g.N, g.K, g.lda, g.ldb, g.ldc};
    auto pi = g_plans.find(key);
    if (pi == g_plans.end()) pi = g_plans.emplace(key, make_plan(h, g)).first;
    plan = pi->second;
  }
  if (!plan.ok) return hipSuccess;
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(h, plan.desc, &alpha, g.Bm, plan.la, g.A, plan.lb, &beta, g.C, plan.lc,
                                             g.C, plan.lc, &plan.algo, ws, ws_bytes, s);
  if (st != HIPBLAS_STATUS_SUCCESS) return hipErrorLaunchFailure;
  *done = true;
  return hipSuccess;
}

}  // namespace csa
