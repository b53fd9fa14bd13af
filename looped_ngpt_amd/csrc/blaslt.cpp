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
#include <utility>

namespace dory {

struct RmKey {
  bool tA, tB;
  int M, N, K, batch;
  int64_t lda, ldb, ldc, sA, sB, sC;
  int ta, tb, tc;
  bool operator<(const RmKey& o) const {
    return std::tie(tA, tB, M, N, K, batch, lda, ldb, ldc, sA, sB, sC, ta, tb, tc) <
           std::tie(o.tA, o.tB, o.M, o.N, o.K, o.batch, o.lda, o.ldb, o.ldc, o.sA, o.sB, o.sC, o.ta, o.tb, o.tc);
  }
};
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
  std::map<RmKey, Plan> rm_plans;
  static void drop(Plan& p) {
    if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
    if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
    if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  }
  ~BlasLt() {
    for (auto& kv : plans) drop(kv.second);
    for (auto& kv : rm_plans) drop(kv.second);
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

// ---------------------------------------------------------------------------
// general row-major strided-batched product (the backward's attention):
// C[M][N] = alpha opA(A) opB(B), A stored [M][K] (or [K][M] when tA), B
// stored [K][N] (or [N][K] when tB), row strides lda/ldb/ldc, batch strides
// in elements. Column-major: C^T (N x M) = opB(B view) . opA(A view).
// ---------------------------------------------------------------------------


static hipDataType dtype_of(int t) { return t == 1 ? HIP_R_16BF : HIP_R_32F; }

static bool layout(hipblasLtMatrixLayout_t* L, int t, uint64_t rows, uint64_t cols, int64_t ld, int batch,
                   int64_t stride) {
  if (hipblasLtMatrixLayoutCreate(L, dtype_of(t), rows, cols, ld) != HIPBLAS_STATUS_SUCCESS) return false;
  if (batch > 1) {
    const int32_t bc = batch;
    const int64_t so = stride;
    if (hipblasLtMatrixLayoutSetAttribute(*L, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof(bc)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutSetAttribute(*L, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &so, sizeof(so)) !=
            HIPBLAS_STATUS_SUCCESS)
      return false;
  }
  return true;
}

bool blaslt_rm(BlasLt* b, bool tA, bool tB, int M, int N, int K, const void* A, int ta, int64_t lda, int64_t sA,
               const void* B, int tb, int64_t ldb, int64_t sB, void* C, int tc, int64_t ldc, int64_t sC, int batch,
               float alpha, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!b || M <= 0 || N <= 0 || K <= 0 || batch <= 0) return false;
  const RmKey key{tA, tB, M, N, K, batch, lda, ldb, ldc, sA, sB, sC, ta, tb, tc};
  auto it = b->rm_plans.find(key);
  if (it == b->rm_plans.end()) {
    BlasLt::Plan& p = b->rm_plans[key];
    const hipblasOperation_t op1 = tB ? HIPBLAS_OP_T : HIPBLAS_OP_N, op2 = tA ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op1, sizeof(op1)) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op2, sizeof(op2)) ==
                   HIPBLAS_STATUS_SUCCESS;
    // first operand: the column-major view of B; second: of A
    ok = ok && (tB ? layout(&p.a, tb, K, N, ldb, batch, sB) : layout(&p.a, tb, N, K, ldb, batch, sB));
    ok = ok && (tA ? layout(&p.b, ta, M, K, lda, batch, sA) : layout(&p.b, ta, K, M, lda, batch, sA));
    ok = ok && layout(&p.c, tc, N, M, ldc, batch, sC);
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
    it = b->rm_plans.find(key);
  }
  BlasLt::Plan* p = &it->second;
  if (!p->ok) return false;
  const float beta = 0.f;
  return hipblasLtMatmul(b->h, p->desc, &alpha, B, p->a, A, p->b, &beta, C, p->c, C, p->c, &p->algo, ws, p->ws,
                         st) == HIPBLAS_STATUS_SUCCESS;
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
