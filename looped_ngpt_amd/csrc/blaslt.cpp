// Plain prefill projections on hipBLASLt: y[M][N] (float32 or bfloat16) = scale *
// x[M][K] (bfloat16, row stride ldx) . W[N][K]^T (bfloat16). These are
// library GEMMs with no fused epilogue (q|k|v|gate, output, down at prefill
// row counts); the fused ones (SwiGLU, decode GEMVs) stay on our kernels.
// Row-major y is the column-major N x M matrix W_c^T . x_c, with W_c the
// column-major K x N view of W and x_c the K x M view of x. One plan (layouts
// and the heuristic's first algorithm) per shape, kept by the context.
#include "blaslt.h"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <tuple>

namespace dory {

struct BlasLt {
  hipblasLtHandle_t h = nullptr;
  struct Plan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    bool ok = false;
  };
  std::map<std::tuple<int, int, int, int64_t, int>, Plan> plans;
  ~BlasLt() {
    for (auto& kv : plans) {
      Plan& p = kv.second;
      if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
      if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
      if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
      if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
    }
    if (h) hipblasLtDestroy(h);
  }
};

BlasLt* blaslt_create() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n == 0) {
    (void)hipGetLastError();
    return nullptr;
  }
  BlasLt* b = new BlasLt;
  if (hipblasLtCreate(&b->h) != HIPBLAS_STATUS_SUCCESS) {
    b->h = nullptr;
    delete b;
    return nullptr;
  }
  return b;
}

void blaslt_destroy(BlasLt* b) { delete b; }

static BlasLt::Plan* plan_for(BlasLt* b, int M, int N, int K, int64_t ldx, bool bf16_out, size_t ws_bytes) {
  auto key = std::make_tuple(M, N, K, ldx, bf16_out ? 1 : 0);
  auto it = b->plans.find(key);
  if (it != b->plans.end()) return it->second.ok ? &it->second : nullptr;
  BlasLt::Plan& p = b->plans[key];
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, K, M, ldx) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.c, bf16_out ? HIP_R_16BF : HIP_R_32F, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t wsb = ws_bytes;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                   sizeof(wsb)) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res[1];
  int got = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(b->h, p.desc, p.a, p.b, p.c, p.c, pref, 1, res, &got) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && got >= 1 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= ws_bytes;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ok) {
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
  }
  p.ok = ok;
  return ok ? &p : nullptr;
}

bool blaslt_gemm(BlasLt* b, const void* x, int64_t ldx, const void* W, void* y, bool bf16_out, int M, int N, int K,
                 float scale, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!b || M <= 0 || N <= 0 || K <= 0) return false;
  BlasLt::Plan* p = plan_for(b, M, N, K, ldx, bf16_out, ws_bytes);
  if (!p) return false;
  const float alpha = scale, beta = 0.f;
  return hipblasLtMatmul(b->h, p->desc, &alpha, W, p->a, x, p->b, &beta, y, p->c, y, p->c, &p->algo, ws, p->ws,
                         st) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace dory
