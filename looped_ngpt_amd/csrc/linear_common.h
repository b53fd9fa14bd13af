// Device helpers shared by the projection kernels: epilogues, SiLU and the
// bfloat16 pair dot product.
#pragma once

#include "common.h"

namespace dory {

enum { EPI_F32 = 0, EPI_SWIGLU = 1 };

__device__ __forceinline__ float silu_(float v) { return v / (1.0f + expf(-v)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  // v_dot2c_f32_bf16: c + a.lo * b.lo + a.hi * b.hi in float32, no unpacking
  return __builtin_amdgcn_fdot2_f32_bf16(*(const bf16x2_t*)&a, *(const bf16x2_t*)&b, c, false);
}

}  // namespace dory
