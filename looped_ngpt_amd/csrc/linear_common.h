// Device helpers shared by the projection kernels: epilogues, SiLU and the
// bfloat16 pair dot product.
#pragma once

#include "common.h"
#include "kernels.h"

namespace dory {

enum { EPI_F32 = 0, EPI_SWIGLU = 1 };

__device__ __forceinline__ float silu_(float v) { return v / (1.0f + expf(-v)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  // v_dot2c_f32_bf16: c + a.lo * b.lo + a.hi * b.hi in float32, no unpacking
  return __builtin_amdgcn_fdot2_f32_bf16(*(const bf16x2_t*)&a, *(const bf16x2_t*)&b, c, false);
}

// Raw loads for 8 consecutive input elements (row m, columns j0..j0+7, one
// head) of an AttnX-fed projection: four 16-byte loads of bin 0's value sums
// and the head's sums p of every bin; issued early, turned into bfloat16
// later. The other bins' value sums are read only where a workgroup used
// them (their sum p is nonzero): scores far below the bound.
typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
struct AttnXRaw {
  u64x2_t a[4];
  u64x2_t l[2];  // sum p of bins 0..3 (words past acc_nb are zero)
  const unsigned long long* ap;
};

__device__ __forceinline__ void attn_x_load(const AttnX& ax, int m, int j0, AttnXRaw& r) {
  const int h = j0 / ax.hd, d0 = j0 % ax.hd;
  const unsigned long long* hp = ax.acc + ((size_t)m * ax.nq + h) * attn_acc_stride(ax.hd, ax.nb);
  r.ap = hp + d0;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.a[i] = *(const u64x2_t*)(r.ap + 2 * i);
  const unsigned long long* lp = hp + ax.nb * ax.hd;
  r.l[0] = *(const u64x2_t*)lp;
  r.l[1] = *(const u64x2_t*)(lp + 2);
}

__device__ __forceinline__ u32x4 attn_x_make(const AttnX& ax, const AttnXRaw& r) {
  float v[8];
  if ((r.l[0][1] | r.l[1][0] | r.l[1][1]) == 0) {
    const float il = (float)(1.0 / (double)(long long)r.l[0][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)(long long)r.a[i][0] * il;
      v[2 * i + 1] = (float)(long long)r.a[i][1] * il;
    }
  } else {
    // bin b counts units of 2^(-16b) relative to bin 0
    const long long lb[4] = {(long long)r.l[0][0], (long long)r.l[0][1], (long long)r.l[1][0],
                             (long long)r.l[1][1]};
    double L = 0.0, A[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[2 * i] = (double)(long long)r.a[i][0];
      A[2 * i + 1] = (double)(long long)r.a[i][1];
    }
    for (int b = 0; b < ax.nb && b < kAttnAccBinsMax; ++b) {
      const double f = ldexp(1.0, -kAttnAccBinBits * b);
      L += (double)lb[b] * f;
      if (b == 0 || lb[b] == 0) continue;
      const unsigned long long* bp = r.ap + b * ax.hd;
#pragma unroll
      for (int i = 0; i < 8; ++i) A[i] += (double)(long long)bp[i] * f;
    }
    const double il = 1.0 / L;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)(A[i] * il);
  }
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (uint32_t)from_f<bf16>(v[2 * i]) | ((uint32_t)from_f<bf16>(v[2 * i + 1]) << 16);
  return out;
}

}  // namespace dory
