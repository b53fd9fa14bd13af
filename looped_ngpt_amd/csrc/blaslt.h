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

}  // namespace dory
