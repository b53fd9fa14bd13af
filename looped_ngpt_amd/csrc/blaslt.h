// hipBLASLt for the plain prefill projections (see blaslt.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dory {

struct BlasLt;
// nullptr when no device is present or the library cannot start
BlasLt* blaslt_create();
void blaslt_destroy(BlasLt* b);
// y[M][N] (float32, or bfloat16 when bf16_out) = scale * x[M][K] . W[N][K]^T,
// bfloat16 operands; false when the library has no algorithm for the shape
// (the caller then uses its own GEMM)
bool blaslt_gemm(BlasLt* b, const void* x, int64_t ldx, const void* W, void* y, bool bf16_out, int M, int N, int K,
                 float scale, void* ws, size_t ws_bytes, hipStream_t st);

// C[M][N] = alpha opA(A) opB(B), row-major, strided-batched: A stored [M][K]
// ([K][M] when tA), B stored [K][N] ([N][K] when tB), row strides lda, ldb,
// ldc and batch strides sA, sB, sC in elements; element types 0 float32,
// 1 bfloat16; float32 accumulation. false: no algorithm for the shape.
bool blaslt_rm(BlasLt* b, bool tA, bool tB, int M, int N, int K, const void* A, int ta, int64_t lda, int64_t sA,
               const void* B, int tb, int64_t ldb, int64_t sB, void* C, int tc, int64_t ldc, int64_t sC, int batch,
               float alpha, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace dory
