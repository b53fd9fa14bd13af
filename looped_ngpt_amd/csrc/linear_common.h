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

// Raw loads for 8 consecutive input elements (row m, columns j0..j0+7, one
// head) of an AttnX-fed projection: four 16-byte loads and the head's sum p;
// issued early, turned into bfloat16 later.
typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
struct AttnXRaw {
  u64x2_t a[4];
  unsigned long long l;
};

__device__ __forceinline__ void attn_x_load(const AttnX& ax, int m, int j0, AttnXRaw& r) {
  const int h = j0 / ax.hd, d0 = j0 % ax.hd;
  const unsigned long long* ap = ax.acc + ((size_t)m * ax.nq + h) * (ax.hd + kAttnAccPad);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.a[i] = *(const u64x2_t*)(ap + d0 + 2 * i);
  r.l = ap[ax.hd];
}

__device__ __forceinline__ u32x4 attn_x_make(const AttnXRaw& r) {
  const float il = (float)(1.0 / (double)(long long)r.l);
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v0 = (float)(long long)r.a[i][0] * il, v1 = (float)(long long)r.a[i][1] * il;
    out[i] = (uint32_t)from_f<bf16>(v0) | ((uint32_t)from_f<bf16>(v1) << 16);
  }
  return out;
}

}  // namespace dory
