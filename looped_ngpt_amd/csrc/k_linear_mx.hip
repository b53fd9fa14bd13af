// MXFP8 weights for the projections: the OCP Microscaling (MX) v1.0 format
// with E4M3 elements, blocks of 32 consecutive weights of an output row along
// the contraction dimension K, one E8M0 scale byte per block (X + 127, the
// block standing for e4m3(q) * 2^X). The pages name MXFP8 checkpoints of the
// model ("Dory1.0-4B: A Looped Normalized-GPT", AI summary, Key Contributions
// 4) without defining the format; this is the published definition.
//
//  * k_quant_mxfp8: bfloat16 [N][K] -> codes [N][K] + scales [N][K/32];
//    X = floor(log2(max |w|)) - 8 (8: exponent of 448, the largest E4M3
//    normal), all-zero blocks X = -127; elements rounded to nearest, ties to
//    the even code, saturating at 448. One thread per block.
//  * k_dequant_mxfp8: codes + scales -> bfloat16 (exact: E4M3 values times a
//    power of two are bfloat16 values while X >= -124).
//  * k_gemv_rows_mx / k_gemv_pro_mx: the decode GEMVs of k_linear.hip for
//    these weights. A lane takes 16-byte chunks of 16 codes; the hardware
//    decode (v_cvt_pk_f32_fp8, OCP E4M3 on gfx950) gives pairs of floats,
//    which v_perm_b32 repacks into bfloat16 pairs exactly, and v_dot2_f32_bf16
//    multiplies them with the activations; the chunk's partial sum takes the
//    block scale once. Weight bytes per output are K + K/32 instead of 2K.
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

// <16 E4M3 weights, 16 bfloat16 activations> * 2^X + acc
__device__ __forceinline__ float dot_mx16(const u32x4& w, const u32x4& x0, const u32x4& x1, float sc, float acc) {
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
  return fmaf(part, sc, acc);
}

// Decode GEMV, one output (two rows for SwiGLU) per wave, activations staged
// in LDS, small loads (activations, scale bytes) issued before the weights.
template <int MB, int CQ, int EPI>
__global__ __launch_bounds__(512) void k_gemv_rows_mx(const bf16* __restrict__ x, int64_t ldx,
                                                     const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
                                                     void* __restrict__ y, int M, int N, int K, float scale) {
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8, nq = K / 16, nb = K / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o = blockIdx.x * 8 + wave;
  const bool live = o < nout;
  const int oc = live ? o : nout - 1;

  constexpr int XV = (MB * CQ * 2 + 7) / 8;  // MB rows x nv <= 128*CQ vectors over 512 threads
  u32x4 xr[XV];
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + 512 * q;
    const int ec = min(e, M * nv - 1);
    xr[q] = ((const u32x4*)(x + (size_t)(ec / nv) * ldx))[ec % nv];
  }
  uint32_t sb[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int row = j ? nout + oc : oc;
#pragma unroll
    for (int c = 0; c < CQ; ++c) sb[j][c] = Ws[(size_t)row * nb + min(lane + 64 * c, nq - 1) / 2];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  u32x4 wv[NR][CQ];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const u32x4* wr = (const u32x4*)(Wq + (size_t)(j ? nout + oc : oc) * K);
#pragma unroll
    for (int c = 0; c < CQ; ++c) wv[j][c] = __builtin_nontemporal_load(wr + min(lane + 64 * c, nq - 1));
  }
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + 512 * q;
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
          for (int j = 0; j < NR; ++j)
            acc[m][j] = dot_mx16(wv[j][c], xm[2 * v], xm[2 * v + 1], e8m0_value(sb[j][c]), acc[m][j]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= M) break;
    const float sum = wave_sum(acc[m][0]);
    if (EPI == EPI_SWIGLU) {
      const float g = wave_sum(acc[m][NR - 1]);
      if (lane == 0) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(sum * silu_(g));
    } else {
      if (lane == 0) ((float*)y)[(size_t)m * N + o] = sum * scale;
    }
  }
}

// The GEMV with the nGPT update (and optional loop re-injection) in its
// prologue, as k_gemv_pro of k_linear.hip: 1024-thread workgroups, two
// outputs per wave, a rolling window of 8 weight chunks per lane.
constexpr int kMxThreads = 1024;
constexpr int kMxOut = 2;
constexpr int kMxWin = 8;

template <int MB, int CQ, int EPI>
__global__ __launch_bounds__(kMxThreads) void k_gemv_pro_mx(GemvPro pr, const uint8_t* __restrict__ Wq,
                                                           const uint8_t* __restrict__ Ws, void* __restrict__ y,
                                                           int M, int N, int K, float scale) {
  constexpr int R = kMxOut;
  constexpr int NR = (EPI == EPI_SWIGLU ? 2 : 1) * R;  // weight rows per wave
  constexpr int NC = NR * CQ;                          // chunk loads per wave
  constexpr int P = NC < kMxWin ? NC : kMxWin;
  constexpr int NW = kMxThreads / 64;
  constexpr int EPT = (CQ * 1024 + kMxThreads - 1) / kMxThreads;  // prologue elements per thread (K <= 1024*CQ)
  __shared__ float sh[NW];
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nq = K / 16, nb = K / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = (blockIdx.x * NW + wave) * R;
  const bool live = o0 < nout;

  // row j of this wave: output o0 + j % R; the u row (j < R) or the v row of SwiGLU
  auto wrow = [&](int j) { const int oc = min(o0 + j % R, nout - 1); return j >= R ? nout + oc : oc; };
  auto chunk_ptr = [&](int c) -> const u32x4* {
    const int v = min(lane + 64 * (c % CQ), nq - 1);  // clamped: chunks past the row are ignored below
    return (const u32x4*)(Wq + (size_t)wrow(c / CQ) * K) + v;
  };

  // prologue inputs of row 0 and the scale bytes first, then the weight window
  const float* ep = pr.e ? pr.e : pr.y;
  float yv[EPT], hv[EPT], ev[EPT], av[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) {
    const int i = min((int)threadIdx.x + kMxThreads * c, K - 1);
    yv[c] = pr.y[i];
    hv[c] = pr.h_in[i];
    ev[c] = ep[i];
    av[c] = pr.alpha[i];
  }
  uint32_t sb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) sb[c] = Ws[(size_t)wrow(c / CQ) * nb + min(lane + 64 * (c % CQ), nq - 1) / 2];
  __builtin_amdgcn_sched_barrier(0);
  u32x4 buf[P];
#pragma unroll
  for (int c = 0; c < P; ++c) buf[c] = __builtin_nontemporal_load(chunk_ptr(c));
  __builtin_amdgcn_sched_barrier(0);

  for (int m = 0; m < M; ++m) {
    const size_t ro = (size_t)m * K;
    if (m > 0) {
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        const int i = min((int)threadIdx.x + kMxThreads * c, K - 1);
        yv[c] = pr.y[ro + i];
        hv[c] = pr.h_in[ro + i];
        ev[c] = ep[ro + i];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      if ((int)threadIdx.x + kMxThreads * c >= K) yv[c] = 0.f, hv[c] = 0.f, ev[c] = 0.f;
      ss += yv[c] * yv[c];
    }
    const float iy = inv_norm(block_sum<kMxThreads>(ss, sh));
    float st = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const float al = (int)threadIdx.x + kMxThreads * c < K ? av[c] : 0.f;
      hv[c] = hv[c] + al * (yv[c] * iy - hv[c]);
      st += hv[c] * hv[c];
    }
    const float ih = inv_norm(block_sum<kMxThreads>(st, sh));
#pragma unroll
    for (int c = 0; c < EPT; ++c) hv[c] *= ih;  // u
    if (pr.e_out && blockIdx.x == 0) {
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        const int i = threadIdx.x + kMxThreads * c;
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
      const float iv = inv_norm(block_sum<kMxThreads>(sv, sh));
#pragma unroll
      for (int c = 0; c < EPT; ++c) hv[c] = yv[c] * iv;
    }
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const int i = threadIdx.x + kMxThreads * c;
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
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const u32x4 w = buf[c % P];
    if (c + P < NC) buf[c % P] = __builtin_nontemporal_load(chunk_ptr(c + P));
    const int j = c / CQ, v = lane + 64 * (c % CQ);
    if (v < nq) {
      const float sc = e8m0_value(sb[c]);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const u32x4* xm = (const u32x4*)(xs + (size_t)m * K);
          acc[m][j] = dot_mx16(w, xm[2 * v], xm[2 * v + 1], sc, acc[m][j]);
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
      const float sum = wave_sum(acc[m][r]);
      if (EPI == EPI_SWIGLU) {
        const float g = wave_sum(acc[m][R + r]);
        if (lane == 0 && o < nout) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(sum * silu_(g));
      } else {
        if (lane == 0 && o < nout) ((float*)y)[(size_t)m * N + o] = sum * scale;
      }
    }
  }
}

template <int MB, int EPI>
hipError_t rows_mx_launch(const bf16* x, int64_t ldx, const uint8_t* Wq, const uint8_t* Ws, void* y, int M, int N,
                          int K, float scale, hipStream_t st) {
  const int cq = (K / 16 + 63) / 64;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const dim3 grid((nout + 7) / 8);
  const size_t lds = (size_t)M * K * 2;
#define DORY_RMX(C)                                                                                          \
  case C:                                                                                                    \
    dory_launch((k_gemv_rows_mx<MB, C, EPI>), grid, dim3(512), (uint32_t)lds, st, x, ldx, Wq, Ws, y, M, N, K, \
                scale);                                                                                      \
    break;
  switch (cq) {
    DORY_RMX(1) DORY_RMX(2) DORY_RMX(3) DORY_RMX(4) DORY_RMX(5) DORY_RMX(6) DORY_RMX(8) DORY_RMX(12) DORY_RMX(16)
    default: return hipErrorInvalidValue;
  }
#undef DORY_RMX
  return hipGetLastError();
}

template <int MB, int EPI>
hipError_t pro_mx_launch(const GemvPro& p, const uint8_t* Wq, const uint8_t* Ws, void* y, int M, int N, int K,
                         float scale, hipStream_t st) {
  const int cq = (K / 16 + 63) / 64;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int per_block = kMxThreads / 64 * kMxOut;
  const dim3 grid((nout + per_block - 1) / per_block);
  const size_t lds = (size_t)M * K * 2;
#define DORY_PMX(C)                                                                                            \
  case C:                                                                                                      \
    dory_launch((k_gemv_pro_mx<MB, C, EPI>), grid, dim3(kMxThreads), (uint32_t)lds, st, p, Wq, Ws, y, M, N, K, \
                scale);                                                                                        \
    break;
  switch (cq) {
    DORY_PMX(1) DORY_PMX(2) DORY_PMX(3) DORY_PMX(4) DORY_PMX(5) DORY_PMX(6) DORY_PMX(8)
    default: return hipErrorInvalidValue;
  }
#undef DORY_PMX
  return hipGetLastError();
}

bool mx_shape_ok(int M, int K, const void* Wq) {
  return M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 && ((uintptr_t)Wq & 15) == 0;
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

hipError_t launch_dequant_mxfp8(const void* q, const void* s, int N, int K, void* W, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (K % 32 || ((uintptr_t)W & 15) || ((uintptr_t)q & 15)) return hipErrorInvalidValue;
  const int64_t nchunks = (int64_t)N * (K / 16);
  // not a timed kernel: plain launch, so a pending timing pair goes to the GEMM that follows
  hipLaunchKernelGGL(k_dequant_mxfp8, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st, (const uint8_t*)q,
                     (const uint8_t*)s, (bf16*)W, nchunks);
  return hipGetLastError();
}

// chunk counts per lane that have an instantiation (rows: 1-6, 8, 12, 16; with the prologue: 1-6, 8)
static bool mx_cq_ok(int cq, bool pro) {
  return (cq >= 1 && cq <= 6) || cq == 8 || (!pro && (cq == 12 || cq == 16));
}

bool linear_mx_supported(int M, int K) {
  return M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 && mx_cq_ok((K / 16 + 63) / 64, false);
}

hipError_t launch_linear_mx(const void* x, int64_t ldx, const void* Wq, const void* Ws, void* y, int M, int N,
                            int K, int epi, float scale, hipStream_t st) {
  if (!mx_shape_ok(M, K, Wq) || !mx_cq_ok((K / 16 + 63) / 64, false) || ldx % 8 || ((uintptr_t)x & 15)) return hipErrorInvalidValue;
  const bf16* xb = (const bf16*)x;
  const uint8_t* q = (const uint8_t*)Wq;
  const uint8_t* s = (const uint8_t*)Ws;
#define DORY_MXM(E)                                                                   \
  if (M == 1) return rows_mx_launch<1, E>(xb, ldx, q, s, y, M, N, K, scale, st);      \
  if (M == 2) return rows_mx_launch<2, E>(xb, ldx, q, s, y, M, N, K, scale, st);      \
  if (M <= 4) return rows_mx_launch<4, E>(xb, ldx, q, s, y, M, N, K, scale, st);      \
  return rows_mx_launch<8, E>(xb, ldx, q, s, y, M, N, K, scale, st);
  if (epi == EPI_SWIGLU) {
    DORY_MXM(EPI_SWIGLU)
  }
  DORY_MXM(EPI_F32)
#undef DORY_MXM
}

bool linear_pro_mx_supported(int M, int K) {
  return M >= 1 && M <= 8 && K % 32 == 0 && (size_t)M * K * 2 <= 64 * 1024 && mx_cq_ok((K / 16 + 63) / 64, true);
}

hipError_t launch_linear_pro_mx(const GemvPro& p, const void* Wq, const void* Ws, void* y, int M, int N, int K,
                                int epi, float scale, hipStream_t st) {
  if (!mx_shape_ok(M, K, Wq) || !mx_cq_ok((K / 16 + 63) / 64, true)) return hipErrorInvalidValue;
  const uint8_t* q = (const uint8_t*)Wq;
  const uint8_t* s = (const uint8_t*)Ws;
#define DORY_PXM(E)                                                         \
  if (M == 1) return pro_mx_launch<1, E>(p, q, s, y, M, N, K, scale, st);   \
  if (M == 2) return pro_mx_launch<2, E>(p, q, s, y, M, N, K, scale, st);   \
  if (M <= 4) return pro_mx_launch<4, E>(p, q, s, y, M, N, K, scale, st);   \
  return pro_mx_launch<8, E>(p, q, s, y, M, N, K, scale, st);
  if (epi == EPI_SWIGLU) {
    DORY_PXM(EPI_SWIGLU)
  }
  DORY_PXM(EPI_F32)
#undef DORY_PXM
}

}  // namespace dory
