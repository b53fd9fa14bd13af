// Device helpers shared by the gfx950 kernels: bfloat16 <-> float, wave64 and
// workgroup reductions, 16-byte vector types.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dory {

constexpr int kNumCUs = 256;  // MI355X compute units (the grids of the decode GEMVs are sized to it)

typedef uint16_t bf16;  // bfloat16 stored as its bit pattern
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte vector

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
// Round to nearest even; NaN stays NaN.
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

// Low and high bfloat16 halves of a 32-bit word, widened.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Butterfly steps of a 64-lane wave without the LDS crossbar (a ds_bpermute
// round trip costs ~4x a whole DPP reduction): xsum<K>(v) = v + v[lane ^ K]
// and xmax<K> likewise, bit for bit, since each lane adds the same two values
// as its partner (float addition is commutative). K = 1, 2: DPP quad_perm;
// 4: row_shl:4 into banks 0 and 2, row_shr:4 into banks 1 and 3; 8:
// row_ror:8; 16, 32: gfx950's v_permlane16_swap / v_permlane32_swap, whose
// two results are the even and odd rows (lower and upper halves) of v. Every
// lane of the wave must be active.
template <int CTRL, int BANKS = 0xF>
__device__ __forceinline__ float dpp_mov(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, BANKS, false));
}

template <int K>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8 || K == 16 || K == 32, "power of two below 64");
  if constexpr (K == 32 || K == 16) {
    const auto r = K == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    a = v;
    if constexpr (K == 1) b = dpp_mov<0xB1>(0.f, v);       // quad_perm [1,0,3,2]
    else if constexpr (K == 2) b = dpp_mov<0x4E>(0.f, v);  // quad_perm [2,3,0,1]
    else if constexpr (K == 4) b = dpp_mov<0x104, 0x5>(dpp_mov<0x114, 0xA>(0.f, v), v);
    else b = dpp_mov<0x128>(0.f, v);                       // row_ror:8
  }
}

template <int K>
__device__ __forceinline__ float xsum(float v) {
  float a, b;
  lane_pair<K>(v, a, b);
  return a + b;
}

template <int K>
__device__ __forceinline__ float xmax(float v) {
  float a, b;
  lane_pair<K>(v, a, b);
  return fmaxf(a, b);
}

// Sum / max over the wave, every lane gets the result; the pairing (32, 16,
// 8, 4, 2, 1) is the classic butterfly's, so the rounding is too.
__device__ __forceinline__ float wave_sum(float v) {
  v = xsum<32>(v);
  v = xsum<16>(v);
  v = xsum<8>(v);
  v = xsum<4>(v);
  v = xsum<2>(v);
  return xsum<1>(v);
}

__device__ __forceinline__ float wave_max(float v) {
  v = xmax<32>(v);
  v = xmax<16>(v);
  v = xmax<8>(v);
  v = xmax<4>(v);
  v = xmax<2>(v);
  return xmax<1>(v);
}

// Sum over a workgroup of NT threads (NT a multiple of 64). `sh` holds at
// least NT/64 floats. Deterministic: waves are added in a fixed order.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r += sh[i];
  return r;
}

// As block_sum, without the leading barrier: for a slot `sh` that no wave can
// still be reading (a barrier has passed since its last read, as when the
// slots of consecutive sums rotate). Same arithmetic, same result.
template <int NT>
__device__ __forceinline__ float block_sum_slot(float v, float* sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r += sh[i];
  return r;
}

__device__ __forceinline__ float inv_norm(float sumsq) { return 1.0f / sqrtf(fmaxf(sumsq, 1e-30f)); }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// Value cache of one kv head: blocks of 32 positions, each stored [hd][32]
// (the 32 values of one dimension contiguous), so the values of a 32-position
// tile are one contiguous run of 32*hd elements. vslots = slots rounded up
// to 32; vt_off = element offset of dimension d of the value in `slot`.
__host__ __device__ __forceinline__ int vslots_of(int slots) { return (slots + 31) & ~31; }
__host__ __device__ __forceinline__ size_t vt_off(int slot, int d, int hd) {
  return (size_t)(slot & ~31) * hd + (size_t)d * 32 + (slot & 31);
}

// Kernel launch that honours the timing tap's pending events.
template <typename F, typename... Args>
inline void dory_launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  const LaunchEvents e = take_next_launch_events();
  if (e.start)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, e.start, e.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

}  // namespace dory
