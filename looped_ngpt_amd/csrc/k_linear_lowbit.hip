// Low-bit weights for the layer projections, two formats.
//
// MXFP8: the OCP Microscaling (MX) v1.0 format with E4M3 elements, blocks of
// 32 consecutive weights of an output row along the contraction dimension K,
// one E8M0 scale byte per block (X + 127, the block standing for
// e4m3(q) * 2^X). The pages name MXFP8 checkpoints of the model ("Dory1.0-4B:
// A Looped Normalized-GPT", AI summary, Key Contributions 4) without defining
// the format; this is the published definition.
//
// NVFP4-style: E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives), two
// per byte with the even element in the low nibble, blocks of 16 along K with
// one E4M3 scale byte each, and one float32 scale g per tensor: code q of
// block scale s stands for e2m1(q) * e4m3(s) * g. The pages say the NVFP4
// checkpoints choose each block scale by least squared error over the 126
// positive E4M3 values (same page, Methodology in Plain English); the search
// below tries all of them.
//
//  * k_quant_mxfp8: bfloat16 [N][K] -> codes [N][K] + scales [N][K/32];
//    X = floor(log2(max |w|)) - 8, all-zero blocks X = -127; elements
//    rounded to nearest, ties to the even code, saturating at 448.
//  * k_absmax / k_quant_nvfp4 / k_tensor_scale: tensor amax, then per block
//    the least-error E4M3 scale (float64, fixed order of operations, so the
//    choice is reproducible), the codes, and g in place of the amax.
//  * k_dequant: codes -> bfloat16 for the prefill GEMM (MXFP8: exact while
//    X >= -124; NVFP4: e2m1 * e4m3 without g, always exact; the GEMM applies g).
//  * k_gemv_rows_lb / k_gemv_pro_lb / k_gemv_pro1_lb: the decode GEMVs of k_linear.hip for
//    these weights. A lane takes 16-byte chunks of codes (16 E4M3 or 32 E2M1);
//    the hardware converts them (v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly,
//    v_perm_b32 repacks the floats' high halves into bfloat16 pairs;
//    v_cvt_scalef32_pk_bf16_fp4 with scale 1 gives E2M1 pairs as bfloat16),
//    v_dot2_f32_bf16 multiplies them with the activations, and each block's
//    partial sum takes its scale once.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "linear_common.h"

namespace dory {
namespace {

// E8M0 byte -> 2^(byte - 127) as a float (byte 0 is the subnormal 2^-127)
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// E4M3 code of v = w / 2^X (|v| < 512, exact), the sign taken from w
__device__ __forceinline__ uint32_t e4m3_code(float w, float v) {
  const uint32_t sign = (__float_as_uint(w) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;                                   // saturate
  } else if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);              // subnormal steps of 2^-9; 8 is the smallest normal
  } else {
    int e;
    (void)frexpf(a, &e);
    const int E = e - 1;                            // floor(log2 a), -6..8
    const float m = rintf((ldexpf(a, -E) - 1.f) * 8.f);
    code = (uint32_t)((E + 7) << 3) + (uint32_t)m;  // m == 8 carries into the next binade
  }
  return code | sign;
}

__global__ __launch_bounds__(256) void k_quant_mxfp8(const bf16* __restrict__ W, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ s, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = (const u32x4*)(W + b * 32);
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = src[i];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(w[i][j])), fabsf(bf_hi(w[i][j]))));
  int X = -127;
  if (amax > 0.f) {
    int e;
    (void)frexpf(amax, &e);
    X = min(max(e - 1 - 8, -127), 127);
  }
  uint32_t words[8];  // element 2k, 2k+1 of the block -> bytes 2k, 2k+1
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf_lo(w[i][j]), hi = bf_hi(w[i][j]);
      const uint32_t pair = e4m3_code(lo, ldexpf(lo, -X)) | (e4m3_code(hi, ldexpf(hi, -X)) << 8);
      const int k = 4 * i + j;  // pair index 0..15 inside the block
      if (k & 1)
        words[k >> 1] |= pair << 16;
      else
        words[k >> 1] = pair;
    }
  const u32x4 out[2] = {u32x4{words[0], words[1], words[2], words[3]}, u32x4{words[4], words[5], words[6], words[7]}};
  u32x4* dst = (u32x4*)(q + b * 32);
  dst[0] = out[0];
  dst[1] = out[1];
  s[b] = (uint8_t)(X + 127);
}

// ---------------------------------------------------------------------------
// NVFP4-style quantiser
// ---------------------------------------------------------------------------
__global__ void k_zero_word(uint32_t* p) { *p = 0u; }

// max |w| over n bfloat16 values into *amax_bits (float bits of a
// non-negative value order like unsigned integers)
__global__ __launch_bounds__(256) void k_absmax(const bf16* __restrict__ W, int64_t n, uint32_t* amax_bits) {
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf(to_f(W[i])));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __float_as_uint(m));
}

// g = float32(amax / 2688), 1 for an all-zero tensor. The float64 quotient
// rounded to float32 equals the correctly rounded float32 quotient: amax has
// at most 24 significant bits and 2688 = 21 * 2^7, so the exact quotient is
// either a float32 rounding midpoint itself or at least 2^-5 of a float32
// half-step away from one, far more than the float64 rounding error.
__device__ __forceinline__ float tensor_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.f ? (float)((double)amax / 2688.0) : 1.0f;
}

// E4M3 value of a positive finite code 1..126 (exact in float64)
__device__ __forceinline__ double e4m3_pos_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e ? ldexp(1.0 + m * 0.125, e - 7) : ldexp((double)m, -9);
}

// One thread per block of 16 weights: every E4M3 scale 1..126 is tried with
// S = e4m3 * g; each |w| rounds to the nearest E2M1 magnitude of |w| / S
// (ties to the even code, saturating at 6) by comparing |w| with S times the
// midpoints, all exact in float64; the error sum runs in element order with
// separate multiply and add (no contraction), so the choice is reproducible.
// The least error wins, the smallest code on equal errors.
__global__ __launch_bounds__(256) void k_quant_nvfp4(const bf16* __restrict__ W, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ s, const uint32_t* __restrict__ amax_bits,
                                                     int64_t nblocks) {
#pragma clang fp contract(off)
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const double g = (double)tensor_scale_of(*amax_bits);
  const u32x4* src = (const u32x4*)(W + b * 16);
  const u32x4 w0 = src[0], w1 = src[1];
  uint32_t raw[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  double a[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[2 * i] = (double)fabsf(bf_lo(raw[i]));
    a[2 * i + 1] = (double)fabsf(bf_hi(raw[i]));
  }
  constexpr double kMid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  constexpr double kMag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double best_err = 0.0;
  int best = 1;
  for (int c = 1; c <= 126; ++c) {
    const double S = e4m3_pos_value(c) * g;
    double T[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) T[j] = S * kMid[j];
    double err = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double m = 0.0;
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const bool up = (j & 1) ? (a[i] >= T[j]) : (a[i] > T[j]);  // ties go to the even index
        m = up ? kMag[j + 1] : m;
      }
      const double e = a[i] - m * S;
      const double e2 = e * e;
      err = err + e2;
    }
    if (c == 1 || err < best_err) {
      best_err = err;
      best = c;
    }
  }
  const double S = e4m3_pos_value(best) * g;
  uint32_t packed = 0, packed2 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t idx = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const double t = S * kMid[j];
      idx += (j & 1) ? (a[i] >= t) : (a[i] > t);
    }
    const uint32_t sign = ((i & 1) ? (raw[i >> 1] >> 31) : ((raw[i >> 1] >> 15) & 1u)) << 3;
    const uint32_t code = idx | sign;
    if (i < 8)
      packed |= code << (4 * i);
    else
      packed2 |= code << (4 * (i - 8));
  }
  uint32_t* dst = (uint32_t*)(q + b * 8);
  dst[0] = packed;
  dst[1] = packed2;
  s[b] = (uint8_t)best;
}

__global__ void k_tensor_scale(uint32_t* amax_bits) { *(float*)amax_bits = tensor_scale_of(*amax_bits); }

// ---------------------------------------------------------------------------
// Expansion to bfloat16 for the prefill GEMM
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_mxfp8(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                       bf16* __restrict__ W, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16 codes per chunk
  if (c >= nchunks) return;
  const u32x4 v = ((const u32x4*)q)[c];
  const float sc = e8m0_value(s[c >> 1]);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v[i], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v[i], true);
    const uint32_t a = __float_as_uint(f01[0] * sc), b2 = __float_as_uint(f01[1] * sc);
    const uint32_t c2 = __float_as_uint(f23[0] * sc), d = __float_as_uint(f23[1] * sc);
    out[i >> 1][(i & 1) * 2] = (a >> 16) | (b2 & 0xffff0000u);
    out[i >> 1][(i & 1) * 2 + 1] = (c2 >> 16) | (d & 0xffff0000u);
  }
  u32x4* dst = (u32x4*)(W + c * 16);
  dst[0] = out[0];
  dst[1] = out[1];
}

// E2M1 pairs of byte `sel` of w as bfloat16 pairs (exact)
#define DORY_FP4_PAIR(w, sel) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((w), 1.0f, (sel)))

__global__ __launch_bounds__(256) void k_dequant_nvfp4(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                       bf16* __restrict__ W, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16 codes (8 bytes) per block
  if (b >= nblocks) return;
  const uint32_t* src = (const uint32_t*)(q + b * 8);
  const float sc = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)s[b], false)[0];
  u32x4 out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t v = src[h];
    const uint32_t p[4] = {DORY_FP4_PAIR(v, 0), DORY_FP4_PAIR(v, 1), DORY_FP4_PAIR(v, 2), DORY_FP4_PAIR(v, 3)};
#pragma unroll
    for (int j = 0; j < 4; ++j)  // e2m1 * e4m3 has at most 6 significant bits: exact in bfloat16
      out[h][j] = (__float_as_uint(bf_lo(p[j]) * sc) >> 16) | (__float_as_uint(bf_hi(p[j]) * sc) & 0xffff0000u);
  }
  u32x4* dst = (u32x4*)(W + b * 16);
  dst[0] = out[0];
  dst[1] = out[1];
}

// ---------------------------------------------------------------------------
// Decode GEMVs
// ---------------------------------------------------------------------------
enum { LB_MX = 1, LB_FP4 = 2 };  // the dory_weight_format values

template <int FMT> struct LowBit;

template <> struct LowBit<LB_MX> {
  static constexpr int kCodes = 16;  // weights per 16-byte chunk
  __device__ static size_t row_bytes(int K) { return (size_t)K; }
  // scale bits of chunk v of a row: its block's E8M0 byte
  __device__ static uint32_t scale_bits(const uint8_t* Ws, size_t row, int K, int v) {
    return Ws[row * (size_t)(K / 32) + v / 2];
  }
  static constexpr int kXV = 2;  // activation vectors (8 bfloat16) per chunk
  __device__ static void load_x(const u32x4* xm, int v, u32x4 (&x)[kXV]) {
    x[0] = xm[2 * v];
    x[1] = xm[2 * v + 1];
  }
  __device__ static float dot(const u32x4& w, const u32x4* xm, int v, uint32_t sb, float acc) {
    u32x4 x[kXV];
    load_x(xm, v, x);
    return dot_x(w, x, sb, acc);
  }
  // <16 E4M3 weights, 16 bfloat16 activations> * 2^X + acc
  __device__ static float dot_x(const u32x4& w, const u32x4 (&x)[kXV], uint32_t sb, float acc) {
    const u32x4 x0 = x[0], x1 = x[1];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      // high halves of the floats are their exact bfloat16 values
      const uint32_t p01 = __builtin_amdgcn_perm(__float_as_uint(f01[1]), __float_as_uint(f01[0]), 0x07060302u);
      const uint32_t p23 = __builtin_amdgcn_perm(__float_as_uint(f23[1]), __float_as_uint(f23[0]), 0x07060302u);
      const u32x4& xv = i < 2 ? x0 : x1;
      part = dot2bf(p01, xv[(i & 1) * 2], part);
      part = dot2bf(p23, xv[(i & 1) * 2 + 1], part);
    }
    return fmaf(part, e8m0_value(sb), acc);
  }
};

template <> struct LowBit<LB_FP4> {
  static constexpr int kCodes = 32;
  __device__ static size_t row_bytes(int K) { return (size_t)(K / 2); }
  // the two E4M3 scale bytes of the chunk's blocks 2v, 2v+1
  __device__ static uint32_t scale_bits(const uint8_t* Ws, size_t row, int K, int v) {
    return *(const uint16_t*)(Ws + row * (size_t)(K / 16) + 2 * v);
  }
  static constexpr int kXV = 4;
  __device__ static void load_x(const u32x4* xm, int v, u32x4 (&x)[kXV]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = xm[4 * v + i];
  }
  __device__ static float dot(const u32x4& w, const u32x4* xm, int v, uint32_t sb, float acc) {
    u32x4 x[kXV];
    load_x(xm, v, x);
    return dot_x(w, x, sb, acc);
  }
  // <32 E2M1 weights, 32 bfloat16 activations>, block by block scaled, + acc
  __device__ static float dot_x(const u32x4& w, const u32x4 (&x)[kXV], uint32_t sb, float acc) {
    const auto sc = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false);
    float p[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // word i: elements 8i..8i+7, block i / 2
      const u32x4 xv = x[i];
      float t = p[i >> 1];
      t = dot2bf(DORY_FP4_PAIR(w[i], 0), xv[0], t);
      t = dot2bf(DORY_FP4_PAIR(w[i], 1), xv[1], t);
      t = dot2bf(DORY_FP4_PAIR(w[i], 2), xv[2], t);
      t = dot2bf(DORY_FP4_PAIR(w[i], 3), xv[3], t);
      p[i >> 1] = t;
    }
    return fmaf(p[1], sc[1], fmaf(p[0], sc[0], acc));
  }
};

// One output (two rows for SwiGLU) per wave, activations staged in LDS, small
// loads (activations, scale bits) issued before the weights.
template <int FMT, int MB, int CQ, int EPI, int XM = 0, int NW = 8>
__global__ __launch_bounds__(NW * 64) void k_gemv_rows_lb(const bf16* __restrict__ x, int64_t ldx,
                                                         const uint8_t* __restrict__ Wq,
                                                         const uint8_t* __restrict__ Ws, void* __restrict__ y, int M,
                                                         int N, int K, float scale, AttnX ax) {
  using F = LowBit<FMT>;
  constexpr int NT = NW * 64;
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8, nq = K / F::kCodes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o = blockIdx.x * NW + wave;
  const bool live = o < nout;
  const int oc = live ? o : nout - 1;

  constexpr int XV = (MB * CQ * F::kCodes * 8 + NT - 1) / NT;  // M rows x nv <= 8*CQ*kCodes vectors over NT threads
  u32x4 xr[XV];
  AttnXRaw xa[XM ? XV : 1];
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + NT * q;
    const int ec = min(e, M * nv - 1);
    if (XM)
      attn_x_load(ax, ec / nv, 8 * (ec % nv), xa[XM ? q : 0]);
    else
      xr[q] = ((const u32x4*)(x + (size_t)(ec / nv) * ldx))[ec % nv];
  }
  uint32_t sb[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int row = j ? nout + oc : oc;
#pragma unroll
    for (int c = 0; c < CQ; ++c) sb[j][c] = F::scale_bits(Ws, row, K, min(lane + 64 * c, nq - 1));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  u32x4 wv[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const u32x4* wr = (const u32x4*)(Wq + (size_t)(j ? nout + oc : oc) * F::row_bytes(K));
#pragma unroll
    for (int c = 0; c < CQ; ++c) wv[j][c] = __builtin_nontemporal_load(wr + min(lane + 64 * c, nq - 1));
  }
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + NT * q;
    if (XM) xr[q] = attn_x_make(ax, xa[XM ? q : 0]);
    if (e / nv < M) ((u32x4*)xs)[e] = xr[q];
  }
  __syncthreads();
  if (!live) return;

  float acc[MB][NR];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[m][j] = 0.f;
#pragma unroll
  for (int c = 0; c < CQ; ++c) {
    const int v = lane + 64 * c;
    if (v < nq) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const u32x4* xm = (const u32x4*)(xs + (size_t)m * K);
#pragma unroll
          for (int j = 0; j < NR; ++j) acc[m][j] = F::dot(wv[j][c], xm, v, sb[j][c], acc[m][j]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= M) break;
    const float sum = wave_sum(acc[m][0]) * scale;
    if (EPI == EPI_SWIGLU) {
      const float g = wave_sum(acc[m][NR - 1]) * scale;
      if (lane == 0) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(sum * silu_(g));
    } else {
      if (lane == 0) ((float*)y)[(size_t)m * N + o] = sum;
    }
  }
}

// Batch 1, float32 out, long rows (the down projection): each output's K
// range on two waves of CQ chunks, 12 waves (6 outputs) per workgroup, the
// halves' wave sums added through LDS (as k_gemv_rows_k2 of k_linear.hip).
template <int FMT, int CQ>
__global__ __launch_bounds__(768) void k_gemv_rows_lb_k2(const bf16* __restrict__ x, const uint8_t* __restrict__ Wq,
                                                        const uint8_t* __restrict__ Ws, float* __restrict__ y, int N,
                                                        int K, float scale) {
  using F = LowBit<FMT>;
  constexpr int NW = 12, NT = NW * 64, OPW = NW / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float part[NW];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8, nq = K / F::kCodes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int o = blockIdx.x * OPW + (wave >> 1), half = wave & 1;
  const bool live = o < N;
  const int oc = live ? o : N - 1;
  constexpr int XV = (2 * CQ * F::kCodes * 8 + NT - 1) / NT;  // 8-element groups over the whole row
  u32x4 xr[XV];
#pragma unroll
  for (int q = 0; q < XV; ++q) xr[q] = ((const u32x4*)x)[min((int)threadIdx.x + NT * q, nv - 1)];
  uint32_t sb[CQ];
#pragma unroll
  for (int c = 0; c < CQ; ++c) sb[c] = F::scale_bits(Ws, oc, K, min(half * CQ * 64 + lane + 64 * c, nq - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  u32x4 wv[CQ];
  const u32x4* wr = (const u32x4*)(Wq + (size_t)oc * F::row_bytes(K));
#pragma unroll
  for (int c = 0; c < CQ; ++c) wv[c] = __builtin_nontemporal_load(wr + min(half * CQ * 64 + lane + 64 * c, nq - 1));
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + NT * q;
    if (e < nv) ((u32x4*)xs)[e] = xr[q];
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CQ; ++c) {
    const int v = half * CQ * 64 + lane + 64 * c;
    if (v < nq) acc = F::dot(wv[c], (const u32x4*)xs, v, sb[c], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (half == 0 && lane == 0 && live) y[o] = (part[wave] + part[wave + 1]) * scale;
}

// The GEMV with the nGPT update (and optional loop re-injection) in its
// prologue, as k_gemv_pro of k_linear.hip: 1024-thread workgroups, two
// outputs per wave, a rolling window of 8 weight chunks per lane.
constexpr int kLbThreads = 1024;
constexpr int kLbOut = 2;
constexpr int kLbWin = 8;

template <int FMT, int MB, int CQ, int EPI>
__global__ __launch_bounds__(kLbThreads) void k_gemv_pro_lb(GemvPro pr, const uint8_t* __restrict__ Wq,
                                                           const uint8_t* __restrict__ Ws, void* __restrict__ y,
                                                           int M, int N, int K, float scale) {
  using F = LowBit<FMT>;
  constexpr int R = kLbOut;
  constexpr int NR = (EPI == EPI_SWIGLU ? 2 : 1) * R;  // weight rows per wave
  constexpr int NC = NR * CQ;                          // chunk loads per wave
  constexpr int P = NC < kLbWin ? NC : kLbWin;
  constexpr int NW = kLbThreads / 64;
  constexpr int EPT = (CQ * F::kCodes * 64 + kLbThreads - 1) / kLbThreads;  // prologue elements per thread
  __shared__ float sh[3][NW];  // one slot per workgroup sum of a row: each reuse follows a barrier
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nq = K / F::kCodes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = (blockIdx.x * NW + wave) * R;
  const bool live = o0 < nout;

  // row j of this wave: output o0 + j % R; the u row (j < R) or the v row of SwiGLU.
  // Chunk c: with few rows M the order is position-major (c = cc * NR + j) so
  // that a position's activations are read from LDS once for all NR rows.
  constexpr bool kReuse = MB <= 2;
  auto cj = [](int c) { return kReuse ? c % NR : c / CQ; };
  auto ccq = [](int c) { return kReuse ? c / NR : c % CQ; };
  auto wrow = [&](int j) { const int oc = min(o0 + j % R, nout - 1); return j >= R ? nout + oc : oc; };
  auto chunk_ptr = [&](int c) -> const u32x4* {
    const int v = min(lane + 64 * ccq(c), nq - 1);  // clamped: chunks past the row are ignored below
    return (const u32x4*)(Wq + (size_t)wrow(cj(c)) * F::row_bytes(K)) + v;
  };

  // prologue inputs of row 0 and the scale bits first, then the weight window
  const float* ep = pr.e ? pr.e : pr.y;
  float yv[EPT], hv[EPT], ev[EPT], av[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) {
    const int i = min((int)threadIdx.x + kLbThreads * c, K - 1);
    yv[c] = pr.y[i];
    hv[c] = pr.h_in[i];
    ev[c] = ep[i];
    av[c] = pr.alpha[i];
  }
  if (pr.zero)
    for (int i = blockIdx.x * kLbThreads + threadIdx.x; i < pr.zero_n; i += gridDim.x * kLbThreads) pr.zero[i] = 0ull;
  uint32_t sb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) sb[c] = F::scale_bits(Ws, wrow(cj(c)), K, min(lane + 64 * ccq(c), nq - 1));
  __builtin_amdgcn_sched_barrier(0);
  u32x4 buf[P];
#pragma unroll
  for (int c = 0; c < P; ++c) buf[c] = __builtin_nontemporal_load(chunk_ptr(c));
  __builtin_amdgcn_sched_barrier(0);

  // one row: a single pass the compiler sees whole (a runtime trip count with
  // loads inside makes its wait counts at the loop joins wait for the weights)
  const int Mp = MB == 1 ? 1 : M;
  for (int m = 0; m < Mp; ++m) {
    const size_t ro = (size_t)m * K;
    if (m > 0) {
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        const int i = min((int)threadIdx.x + kLbThreads * c, K - 1);
        yv[c] = pr.y[ro + i];
        hv[c] = pr.h_in[ro + i];
        ev[c] = ep[ro + i];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      if ((int)threadIdx.x + kLbThreads * c >= K) yv[c] = 0.f, hv[c] = 0.f, ev[c] = 0.f;
      ss += yv[c] * yv[c];
    }
    const float iy = inv_norm(block_sum_slot<kLbThreads>(ss, sh[0]));
    float st = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const float al = (int)threadIdx.x + kLbThreads * c < K ? av[c] : 0.f;
      hv[c] = hv[c] + al * (yv[c] * iy - hv[c]);
      st += hv[c] * hv[c];
    }
    const float ih = inv_norm(block_sum_slot<kLbThreads>(st, sh[1]));
#pragma unroll
    for (int c = 0; c < EPT; ++c) hv[c] *= ih;  // u
    if (pr.e_out && blockIdx.x == 0) {
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        const int i = threadIdx.x + kLbThreads * c;
        if (i < K) pr.e_out[ro + i] = hv[c];
      }
    }
    if (pr.e) {
      float sv = 0.f;
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        yv[c] = pr.wh * hv[c] + pr.we * ev[c];
        sv += yv[c] * yv[c];
      }
      const float iv = inv_norm(block_sum_slot<kLbThreads>(sv, sh[2]));
#pragma unroll
      for (int c = 0; c < EPT; ++c) hv[c] = yv[c] * iv;
    }
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const int i = threadIdx.x + kLbThreads * c;
      if (i < K) {
        xs[ro + i] = from_f<bf16>(hv[c]);
        if (blockIdx.x == 0) pr.h_out[ro + i] = hv[c];
      }
    }
  }
  __syncthreads();
  if (!live) return;

  float acc[MB][NR];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[m][j] = 0.f;
  u32x4 xq[kReuse ? MB : 1][F::kXV];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const u32x4 w = buf[c % P];
    if (c + P < NC) buf[c % P] = __builtin_nontemporal_load(chunk_ptr(c + P));
    const int j = cj(c), v = lane + 64 * ccq(c);
    if (kReuse && j == 0) {
#pragma unroll
      for (int m = 0; m < (kReuse ? MB : 1); ++m)
        if (m < M) F::load_x((const u32x4*)(xs + (size_t)m * K), min(v, nq - 1), xq[m]);
    }
    if (v < nq) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          if (kReuse)
            acc[m][j] = F::dot_x(w, xq[kReuse ? m : 0], sb[c], acc[m][j]);
          else
            acc[m][j] = F::dot(w, (const u32x4*)(xs + (size_t)m * K), v, sb[c], acc[m][j]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= M) break;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int o = o0 + r;
      const float sum = wave_sum(acc[m][r]) * scale;
      if (EPI == EPI_SWIGLU) {
        const float g = wave_sum(acc[m][R + r]) * scale;
        if (lane == 0 && o < nout) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(sum * silu_(g));
      } else {
        if (lane == 0 && o < nout) ((float*)y)[(size_t)m * N + o] = sum;
      }
    }
  }
}

// Batch 1: the same GEMV and update (without re-injection, e_out or clearing)
// on the skeleton of k_gemv_rows_lb. One output per wave, 8 waves per
// workgroup; each thread takes the update of one group of 8 consecutive
// elements with 16-byte loads (K <= 8 * 512). A bare
// barrier after the small loads (inputs, scale bits) queues every wave's
// before any weight load, so the update does not wait behind the weight
// stream. The activations of a chunk position are read from LDS once for the
// u and v rows. Per element the update is computed as in k_gemv_pro_lb; only
// the order of the workgroup sums differs. 4-bit up/gate projection of the
// 36-layer shape: 9.1 us against 10.2 us for k_gemv_pro_lb; the single-row
// outputs and the 8-bit format measured slower on it, so only that case uses it.
constexpr int kLb1Waves = 8;

template <int FMT, int CQ, int EPI>
__global__ __launch_bounds__(kLb1Waves * 64) void k_gemv_pro1_lb(GemvPro pr, const uint8_t* __restrict__ Wq,
                                                                const uint8_t* __restrict__ Ws, void* __restrict__ y,
                                                                int N, int K, float scale) {
  using F = LowBit<FMT>;
  constexpr int NW = kLb1Waves, NT = NW * 64;
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  __shared__ float sh[2][NW];  // one slot per workgroup sum: each is used once
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8, nq = K / F::kCodes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o = blockIdx.x * NW + wave;
  const bool live = o < nout;
  const int oc = live ? o : nout - 1;
  const int g = threadIdx.x;  // this thread's group: elements 8g .. 8g+7
  const bool gv = g < nv;
  const int gc = gv ? g : nv - 1;

  // inputs first
  float4 y4[2], h4[2], a4[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    y4[i] = ((const float4*)pr.y)[2 * gc + i];
    h4[i] = ((const float4*)pr.h_in)[2 * gc + i];
    a4[i] = ((const float4*)pr.alpha)[2 * gc + i];
  }
  uint32_t sb[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int c = 0; c < CQ; ++c) sb[j][c] = F::scale_bits(Ws, j ? nout + oc : oc, K, min(lane + 64 * c, nq - 1));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wv[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const u32x4* wr = (const u32x4*)(Wq + (size_t)(j ? nout + oc : oc) * F::row_bytes(K));
#pragma unroll
    for (int c = 0; c < CQ; ++c) wv[j][c] = __builtin_nontemporal_load(wr + min(lane + 64 * c, nq - 1));
  }
  __builtin_amdgcn_sched_barrier(0);

  float yv[8], hv[8], av[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    yv[i] = gv ? y4[i >> 2][i & 3] : 0.f;
    hv[i] = gv ? h4[i >> 2][i & 3] : 0.f;
    av[i] = gv ? a4[i >> 2][i & 3] : 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += yv[i] * yv[i];
  const float iy = inv_norm(block_sum_slot<NT>(ss, sh[0]));
  float st = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hv[i] = hv[i] + av[i] * (yv[i] * iy - hv[i]);
    st += hv[i] * hv[i];
  }
  const float ih = inv_norm(block_sum_slot<NT>(st, sh[1]));
#pragma unroll
  for (int i = 0; i < 8; ++i) hv[i] *= ih;  // u
  if (gv) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)from_f<bf16>(hv[2 * i]) | ((uint32_t)from_f<bf16>(hv[2 * i + 1]) << 16);
    ((u32x4*)xs)[g] = w;
    if (blockIdx.x == 0) {
      ((float4*)pr.h_out)[2 * g] = make_float4(hv[0], hv[1], hv[2], hv[3]);
      ((float4*)pr.h_out)[2 * g + 1] = make_float4(hv[4], hv[5], hv[6], hv[7]);
    }
  }
  __syncthreads();
  if (!live) return;

  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
#pragma unroll
  for (int c = 0; c < CQ; ++c) {
    const int v = lane + 64 * c;
    if (v < nq) {
      u32x4 xq[F::kXV];
      F::load_x((const u32x4*)xs, v, xq);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = F::dot_x(wv[j][c], xq, sb[j][c], acc[j]);
    }
  }
  const float sum = wave_sum(acc[0]) * scale;
  if (EPI == EPI_SWIGLU) {
    const float gt = wave_sum(acc[NR - 1]) * scale;
    if (lane == 0) ((bf16*)y)[o] = from_f<bf16>(sum * silu_(gt));
  } else {
    if (lane == 0) ((float*)y)[o] = sum;
  }
}

int chunks_per_lane(int fmt, int K) { return (K / (fmt == LB_MX ? 16 : 32) + 63) / 64; }

// chunk counts per lane with an instantiation (rows: 1-6, 8, 12, 16; with the prologue: 1-6, 8)
bool cq_ok(int cq, bool pro) { return (cq >= 1 && cq <= 6) || cq == 8 || (!pro && (cq == 12 || cq == 16)); }

template <int FMT, int MB, int EPI, int XM, int NW>
hipError_t rows_lb_launch_nw(const bf16* x, int64_t ldx, const uint8_t* Wq, const uint8_t* Ws, void* y, int M, int N,
                             int K, float scale, hipStream_t st, const AttnX& ax) {
  const int cq = chunks_per_lane(FMT, K);
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const dim3 grid((nout + NW - 1) / NW);
  const size_t lds = (size_t)M * K * 2;
  // M * K * 2 <= 64 KiB bounds K, hence the chunk counts worth instantiating
  constexpr int kMaxCq = (32768 / MB / LowBit<FMT>::kCodes + 63) / 64;
#define DORY_RLB(C)                                                                                                 \
  case C:                                                                                                           \
    if constexpr (C <= kMaxCq) {                                                                                    \
      dory_launch((k_gemv_rows_lb<FMT, MB, C, EPI, XM, NW>), grid, dim3(NW * 64), (uint32_t)lds, st, x, ldx, Wq, Ws, \
                  y, M, N, K, scale, ax);                                                                           \
      break;                                                                                                        \
    } else {                                                                                                        \
      return hipErrorInvalidValue;                                                                                  \
    }
  switch (cq) {
    DORY_RLB(1) DORY_RLB(2) DORY_RLB(3) DORY_RLB(4) DORY_RLB(5) DORY_RLB(6) DORY_RLB(8) DORY_RLB(12) DORY_RLB(16)
    default: return hipErrorInvalidValue;
  }
#undef DORY_RLB
  return hipGetLastError();
}

template <int FMT, int MB, int EPI, int XM = 0>
hipError_t rows_lb_launch(const bf16* x, int64_t ldx, const uint8_t* Wq, const uint8_t* Ws, void* y, int M, int N,
                          int K, float scale, hipStream_t st, const AttnX& ax = AttnX{}) {
  switch (rows_waves(EPI == EPI_SWIGLU ? N / 2 : N)) {
    case 9: return rows_lb_launch_nw<FMT, MB, EPI, XM, 9>(x, ldx, Wq, Ws, y, M, N, K, scale, st, ax);
    case 12: return rows_lb_launch_nw<FMT, MB, EPI, XM, 12>(x, ldx, Wq, Ws, y, M, N, K, scale, st, ax);
    case 16: return rows_lb_launch_nw<FMT, MB, EPI, XM, 16>(x, ldx, Wq, Ws, y, M, N, K, scale, st, ax);
    default: return rows_lb_launch_nw<FMT, MB, EPI, XM, 8>(x, ldx, Wq, Ws, y, M, N, K, scale, st, ax);
  }
}

template <int FMT, int MB, int EPI>
hipError_t pro_lb_launch(const GemvPro& p, const uint8_t* Wq, const uint8_t* Ws, void* y, int M, int N, int K,
                         float scale, hipStream_t st) {
  const int cq = chunks_per_lane(FMT, K);
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int per_block = kLbThreads / 64 * kLbOut;
  const dim3 grid((nout + per_block - 1) / per_block);
  const size_t lds = (size_t)M * K * 2;
  constexpr int kMaxCq = (32768 / MB / LowBit<FMT>::kCodes + 63) / 64;
#define DORY_PLB(C)                                                                                                  \
  case C:                                                                                                            \
    if constexpr (C <= kMaxCq) {                                                                                     \
      dory_launch((k_gemv_pro_lb<FMT, MB, C, EPI>), grid, dim3(kLbThreads), (uint32_t)lds, st, p, Wq, Ws, y, M, N, K, \
                  scale);                                                                                            \
      break;                                                                                                         \
    } else {                                                                                                         \
      return hipErrorInvalidValue;                                                                                   \
    }
  switch (cq) {
    DORY_PLB(1) DORY_PLB(2) DORY_PLB(3) DORY_PLB(4) DORY_PLB(5) DORY_PLB(6) DORY_PLB(8)
    default: return hipErrorInvalidValue;
  }
#undef DORY_PLB
  return hipGetLastError();
}

bool lb_shape_ok(int fmt, int M, int K, const void* Wq, const void* Ws) {
  if (fmt != LB_MX && fmt != LB_FP4) return false;
  if (fmt == LB_FP4 && ((uintptr_t)Ws & 1)) return false;
  return M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 && ((uintptr_t)Wq & 15) == 0;
}

template <int FMT>
hipError_t linear_lb(const void* x, int64_t ldx, const void* Wq, const void* Ws, void* y, int M, int N, int K,
                     int epi, float scale, hipStream_t st) {
  const bf16* xb = (const bf16*)x;
  const uint8_t* q = (const uint8_t*)Wq;
  const uint8_t* s = (const uint8_t*)Ws;
  // batch 1, long rows (8 or 4 chunks per lane on one wave): two waves per row
  if (M == 1 && epi == EPI_F32 && (uintptr_t)xb % 16 == 0) {
    const int cq = chunks_per_lane(FMT, K);
    const dim3 grid((N + 5) / 6);
    if (cq == 8) {
      dory_launch((k_gemv_rows_lb_k2<FMT, 4>), grid, dim3(768), (uint32_t)K * 2, st, xb, q, s, (float*)y, N, K, scale);
      return hipGetLastError();
    }
    if (cq == 4 && K / LowBit<FMT>::kCodes > 192) {
      dory_launch((k_gemv_rows_lb_k2<FMT, 2>), grid, dim3(768), (uint32_t)K * 2, st, xb, q, s, (float*)y, N, K, scale);
      return hipGetLastError();
    }
  }
#define DORY_LBM(E)                                                                         \
  if (M == 1) return rows_lb_launch<FMT, 1, E>(xb, ldx, q, s, y, M, N, K, scale, st);       \
  if (M == 2) return rows_lb_launch<FMT, 2, E>(xb, ldx, q, s, y, M, N, K, scale, st);       \
  if (M <= 4) return rows_lb_launch<FMT, 4, E>(xb, ldx, q, s, y, M, N, K, scale, st);       \
  return rows_lb_launch<FMT, 8, E>(xb, ldx, q, s, y, M, N, K, scale, st);
  if (epi == EPI_SWIGLU) {
    DORY_LBM(EPI_SWIGLU)
  }
  DORY_LBM(EPI_F32)
#undef DORY_LBM
}

// k_gemv_pro1_lb covers the plain update (no re-injection, no e_out, nothing
// to clear) at K <= 8 x 512 (one element group per thread) with 16-byte
// aligned vectors; everything else takes k_gemv_pro_lb.
bool pro1_ok(int fmt, const GemvPro& p, int K) {
  auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  const int cq = chunks_per_lane(fmt, K);
  return !p.e && !p.e_out && !p.zero && K % 8 == 0 && K / 8 <= kLb1Waves * 64 && cq >= 1 && cq <= 4 && al(p.y) &&
         al(p.h_in) && al(p.alpha) && al(p.h_out);
}

template <int FMT, int EPI>
hipError_t pro1_lb_launch(const GemvPro& p, const uint8_t* Wq, const uint8_t* Ws, void* y, int N, int K, float scale,
                          hipStream_t st) {
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const dim3 grid((nout + kLb1Waves - 1) / kLb1Waves);
  const size_t lds = (size_t)K * 2;
  // chunk counts a K <= 4096 can take (the 4-bit format: 1 or 2)
  constexpr int kMaxCq = (8 * kLb1Waves * 64 / LowBit<FMT>::kCodes + 63) / 64;
#define DORY_P1(C)                                                                                              \
  case C:                                                                                                       \
    if constexpr (C <= kMaxCq) {                                                                                \
      dory_launch((k_gemv_pro1_lb<FMT, C, EPI>), grid, dim3(kLb1Waves * 64), (uint32_t)lds, st, p, Wq, Ws, y, N, \
                  K, scale);                                                                                    \
      break;                                                                                                    \
    } else {                                                                                                    \
      return hipErrorInvalidValue;                                                                              \
    }
  switch (chunks_per_lane(FMT, K)) {
    DORY_P1(1) DORY_P1(2) DORY_P1(3) DORY_P1(4)
    default: return hipErrorInvalidValue;
  }
#undef DORY_P1
  return hipGetLastError();
}

template <int FMT>
hipError_t linear_pro_lb(const GemvPro& p, const void* Wq, const void* Ws, void* y, int M, int N, int K, int epi,
                         float scale, hipStream_t st) {
  const uint8_t* q = (const uint8_t*)Wq;
  const uint8_t* s = (const uint8_t*)Ws;
  // measured faster only where a wave streams two 4-bit rows (the u and v
  // rows of up/gate); the 8-bit format and single-row outputs keep k_gemv_pro_lb
  if (FMT == LB_FP4 && epi == EPI_SWIGLU && M == 1 && pro1_ok(FMT, p, K))
    return pro1_lb_launch<FMT, EPI_SWIGLU>(p, q, s, y, N, K, scale, st);
#define DORY_PLM(E)                                                               \
  if (M == 1) return pro_lb_launch<FMT, 1, E>(p, q, s, y, M, N, K, scale, st);    \
  if (M == 2) return pro_lb_launch<FMT, 2, E>(p, q, s, y, M, N, K, scale, st);    \
  if (M <= 4) return pro_lb_launch<FMT, 4, E>(p, q, s, y, M, N, K, scale, st);    \
  return pro_lb_launch<FMT, 8, E>(p, q, s, y, M, N, K, scale, st);
  if (epi == EPI_SWIGLU) {
    DORY_PLM(EPI_SWIGLU)
  }
  DORY_PLM(EPI_F32)
#undef DORY_PLM
}

}  // namespace

hipError_t launch_quant_mxfp8(const void* W, int N, int K, void* q, void* s, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (K % 32 || ((uintptr_t)W & 15) || ((uintptr_t)q & 15)) return hipErrorInvalidValue;
  const int64_t nblocks = (int64_t)N * (K / 32);
  hipLaunchKernelGGL(k_quant_mxfp8, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, (const bf16*)W,
                     (uint8_t*)q, (uint8_t*)s, nblocks);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const void* W, int N, int K, void* q, void* s, float* tscale, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (K % 32 || ((uintptr_t)W & 15) || ((uintptr_t)q & 7) || ((uintptr_t)tscale & 3)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)N * K, nblocks = n / 16;
  uint32_t* amax = (uint32_t*)tscale;  // holds the amax bits until k_tensor_scale turns them into g
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(1), 0, st, amax);
  const int64_t groups = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_absmax, dim3((unsigned)groups), dim3(256), 0, st, (const bf16*)W, n, amax);
  hipLaunchKernelGGL(k_quant_nvfp4, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, (const bf16*)W,
                     (uint8_t*)q, (uint8_t*)s, (const uint32_t*)amax, nblocks);
  hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(1), 0, st, amax);
  return hipGetLastError();
}

hipError_t launch_dequant_lowbit(int fmt, const void* q, const void* s, int N, int K, void* W, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (K % 32 || ((uintptr_t)W & 15) || ((uintptr_t)q & 15)) return hipErrorInvalidValue;
  // not timed kernels: plain launches, so a pending timing pair goes to the GEMM that follows
  if (fmt == LB_MX) {
    const int64_t nchunks = (int64_t)N * (K / 16);
    hipLaunchKernelGGL(k_dequant_mxfp8, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st,
                       (const uint8_t*)q, (const uint8_t*)s, (bf16*)W, nchunks);
  } else if (fmt == LB_FP4) {
    const int64_t nblocks = (int64_t)N * (K / 16);
    hipLaunchKernelGGL(k_dequant_nvfp4, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st,
                       (const uint8_t*)q, (const uint8_t*)s, (bf16*)W, nblocks);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool linear_lowbit_supported(int fmt, int M, int K) {
  return (fmt == LB_MX || fmt == LB_FP4) && M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 &&
         cq_ok(chunks_per_lane(fmt, K), false);
}

bool linear_pro_lowbit_supported(int fmt, int M, int K) {
  return (fmt == LB_MX || fmt == LB_FP4) && M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 &&
         cq_ok(chunks_per_lane(fmt, K), true);
}

hipError_t launch_linear_lowbit(int fmt, const void* x, int64_t ldx, const void* Wq, const void* Ws, void* y, int M,
                                int N, int K, int epi, float scale, hipStream_t st) {
  if (!lb_shape_ok(fmt, M, K, Wq, Ws) || !linear_lowbit_supported(fmt, M, K) || ldx % 8 || ((uintptr_t)x & 15))
    return hipErrorInvalidValue;
  return fmt == LB_MX ? linear_lb<LB_MX>(x, ldx, Wq, Ws, y, M, N, K, epi, scale, st)
                      : linear_lb<LB_FP4>(x, ldx, Wq, Ws, y, M, N, K, epi, scale, st);
}

hipError_t launch_linear_lowbit_attn(int fmt, const AttnX& ax, const void* Wq, const void* Ws, float* y, int M, int N,
                                     int K, float scale, hipStream_t st) {
  if (!lb_shape_ok(fmt, M, K, Wq, Ws) || !linear_lowbit_supported(fmt, M, K) || ax.hd % 8 || K != ax.nq * ax.hd)
    return hipErrorInvalidValue;
  const uint8_t* q = (const uint8_t*)Wq;
  const uint8_t* s = (const uint8_t*)Ws;
#define DORY_ALB(F)                                                                                      \
  if (M == 1) return rows_lb_launch<F, 1, EPI_F32, 1>(nullptr, K, q, s, y, M, N, K, scale, st, ax);     \
  if (M == 2) return rows_lb_launch<F, 2, EPI_F32, 1>(nullptr, K, q, s, y, M, N, K, scale, st, ax);     \
  if (M <= 4) return rows_lb_launch<F, 4, EPI_F32, 1>(nullptr, K, q, s, y, M, N, K, scale, st, ax);     \
  return rows_lb_launch<F, 8, EPI_F32, 1>(nullptr, K, q, s, y, M, N, K, scale, st, ax);
  if (fmt == LB_MX) {
    DORY_ALB(LB_MX)
  }
  DORY_ALB(LB_FP4)
#undef DORY_ALB
}

hipError_t launch_linear_pro_lowbit(int fmt, const GemvPro& p, const void* Wq, const void* Ws, void* y, int M, int N,
                                    int K, int epi, float scale, hipStream_t st) {
  if (!lb_shape_ok(fmt, M, K, Wq, Ws) || !linear_pro_lowbit_supported(fmt, M, K)) return hipErrorInvalidValue;
  return fmt == LB_MX ? linear_pro_lb<LB_MX>(p, Wq, Ws, y, M, N, K, epi, scale, st)
                      : linear_pro_lb<LB_FP4>(p, Wq, Ws, y, M, N, K, epi, scale, st);
}

}  // namespace dory
