// Plain bf16 GEMMs through hipBLASLt for the large-batch shapes: C[M, N]
// (fp32, row-major) = A[M, K] (bf16, row-major) x W[N, K]^T (bf16, row-major).
// The fused epilogues (residual, SiLU.mul, RoPE + KV write) then run in the
// library's own kernel over C, the one split-K sums into.  Plans (descriptors
// and the heuristic's first algorithm) are cached per shape; the workspace is
// allocated once, so a call makes no allocation and can be captured.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <tuple>

#include "pe_internal.h"

namespace pe {

struct BlasPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t lw = nullptr, la = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool ok = false;
};

struct Blas {
  hipblasLtHandle_t h = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::map<std::tuple<int, int, int, int>, BlasPlan> plans;
};

Blas* blas_create(size_t ws_bytes) {
  Blas* b = new Blas;
  if (hipblasLtCreate(&b->h) != HIPBLAS_STATUS_SUCCESS) {
    delete b;
    return nullptr;
  }
  if (ws_bytes && hipMalloc(&b->ws, ws_bytes) != hipSuccess) {
    hipblasLtDestroy(b->h);
    delete b;
    return nullptr;
  }
  b->ws_bytes = ws_bytes;
  return b;
}

void blas_destroy(Blas* b) {
  if (!b) return;
  for (auto& kv : b->plans) {
    BlasPlan& p = kv.second;
    if (p.lw) hipblasLtMatrixLayoutDestroy(p.lw);
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  }
  if (b->ws) (void)hipFree(b->ws);
  if (b->h) hipblasLtDestroy(b->h);
  delete b;
}

// Column-major view: D[N, M] (ld N) = op_T(W as [K, N], ld K) x A as [K, M] (ld K).
static BlasPlan* plan_for(Blas* b, int M, int N, int K, bool out_bf16) {
  auto key = std::make_tuple(M, N, K, int(out_bf16));
  auto it = b->plans.find(key);
  if (it != b->plans.end()) return it->second.ok ? &it->second : nullptr;
  BlasPlan& p = b->plans[key];
  const hipblasOperation_t tw = HIPBLAS_OP_T, ta = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &tw, sizeof tw);
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &ta, sizeof ta);
  if (hipblasLtMatrixLayoutCreate(&p.lw, HIP_R_16BF, K, N, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, M, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lc, out_bf16 ? HIP_R_16BF : HIP_R_32F, N, M, N) != HIPBLAS_STATUS_SUCCESS)
    return nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  const uint64_t ws = b->ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws);
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  const hipblasStatus_t st =
      hipblasLtMatmulAlgoGetHeuristic(b->h, p.desc, p.lw, p.la, p.lc, p.lc, pref, 1, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS || n < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) return nullptr;
  p.algo = res[0].algo;
  p.ok = true;
  return &p;
}

bool blas_gemm(Blas* b, int M, int N, int K, const void* A, const void* W, float* C, hipStream_t st) {
  if (!b) return false;
  BlasPlan* p = plan_for(b, M, N, K, false);
  if (!p) return false;
  const float one = 1.f, zero = 0.f;
  return hipblasLtMatmul(b->h, p->desc, &one, W, p->lw, A, p->la, &zero, C, p->lc, C, p->lc, &p->algo, b->ws,
                         b->ws_bytes, st) == HIPBLAS_STATUS_SUCCESS;
}

// D[M, N] bf16 = A x W^T (+ R[M, N] bf16 when R is set; R may be D), fp32
// accumulation and one rounding to bf16
bool blas_gemm_bf16(Blas* b, int M, int N, int K, const void* A, const void* W, const void* R, void* D,
                    hipStream_t st) {
  if (!b) return false;
  BlasPlan* p = plan_for(b, M, N, K, true);
  if (!p) return false;
  const float one = 1.f, zero = 0.f;
  return hipblasLtMatmul(b->h, p->desc, &one, W, p->lw, A, p->la, R ? &one : &zero, R ? R : D, p->lc, D, p->lc,
                         &p->algo, b->ws, b->ws_bytes, st) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace pe
