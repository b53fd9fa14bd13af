// Linear layers y = x . W^T of the looped nGPT (the fused q|k|v|gate
// projection, the attention output projection, the SwiGLU up/gate projection
// and the down projection, and the tied LM head).
//
//  * k_gemv_vec: decode (M <= 8 rows). HBM-bound weight streaming: each wave
//    owns ROWS weight rows, every lane loads 16 B per row per step, the
//    activations sit in LDS, and a wave reduction closes each dot product.
//  * k_gemm_mfma: prefill, bfloat16. 128x128x64 workgroup tiles, four waves
//    of 64x64, v_mfma_f32_32x32x16_bf16, LDS rows padded by 16 B, the next
//    K tile prefetched into registers while the current one is multiplied.
//  * k_gemm_simple / k_gemv_scalar: float32 models and ragged shapes.
//
// Epilogue 1 (SwiGLU) pairs row o of u with row F + o of v inside one wave
// and stores u * silu(v) in the model dtype.
#include "common.h"
#include "kernels.h"
#include "linear_common.h"

namespace dory {

// acc + <w, x> over 8 bfloat16 pairs
__device__ __forceinline__ float dot16(const u32x4& w, const u32x4& x, const bf16*, float acc) {
  acc = dot2bf(w.x, x.x, acc);
  acc = dot2bf(w.y, x.y, acc);
  acc = dot2bf(w.z, x.z, acc);
  return dot2bf(w.w, x.w, acc);
}

__device__ __forceinline__ float dot16(const u32x4& w, const u32x4& x, const float*, float acc) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  return fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
}

// ---------------------------------------------------------------------------
// GEMV, vector path (K a multiple of 16 B worth of elements, rows aligned)
// ---------------------------------------------------------------------------
template <typename T, int MB, int ROWS, int EPI>
__global__ __launch_bounds__(256) void k_gemv_vec(const T* __restrict__ x, int64_t ldx, const T* __restrict__ W,
                                                 void* __restrict__ y, int M, int N, int K, float scale) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NR = EPI == EPI_SWIGLU ? 2 * ROWS : ROWS;
  extern __shared__ __align__(16) unsigned char smem[];
  T* xs = (T*)smem;
  const int nv = K / VEC;
  for (int m = 0; m < M; ++m)
    for (int v = threadIdx.x; v < nv; v += 256)
      ((u32x4*)(xs + (size_t)m * K))[v] = ((const u32x4*)(x + (size_t)m * ldx))[v];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = (blockIdx.x * 4 + wave) * ROWS;
  if (o0 >= nout) return;
  const T* wr[NR];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int o = min(o0 + r, nout - 1);
    wr[r] = W + (size_t)o * K;
    if (EPI == EPI_SWIGLU) wr[ROWS + r] = W + (size_t)(nout + o) * K;
  }
  float acc[MB][NR];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[m][j] = 0.f;

#pragma unroll 2
  for (int v = lane; v < nv; v += 64) {
    u32x4 wv[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) wv[j] = __builtin_nontemporal_load(((const u32x4*)wr[j]) + v);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < M) {
        const u32x4 xv = ((const u32x4*)(xs + (size_t)m * K))[v];
#pragma unroll
        for (int j = 0; j < NR; ++j) acc[m][j] = dot16(wv[j], xv, (const T*)nullptr, acc[m][j]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= M) break;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = wave_sum(acc[m][r]);
      if (EPI == EPI_SWIGLU) {
        const float g = wave_sum(acc[m][ROWS + r]);
        if (lane == 0 && o0 + r < nout) ((T*)y)[(size_t)m * nout + o0 + r] = from_f<T>(s * scale * silu_(g * scale));
      } else {
        if (lane == 0 && o0 + r < nout) ((float*)y)[(size_t)m * N + o0 + r] = s * scale;
      }
    }
  }
}

// GEMV for bfloat16 decode, row loads first. Each of the 8 waves of a
// workgroup owns one output (two weight rows for SwiGLU). All CH 16-byte
// chunks of its rows are requested before the activations are staged in LDS,
// so the HBM latency of the weights overlaps the activation staging and the
// workgroup barrier; then each lane multiplies its chunks and a wave
// reduction closes the dot products.
// XM 1: the activations are built from decode attention accumulators (AttnX)
// instead of read from x.
// NW waves per workgroup (one output each): 8, or nout / 256 so that the
// grid is exactly one workgroup per CU (3072 outputs: 12 waves).
template <int MB, int CH, int EPI, int XM = 0, int NW = 8>
__global__ __launch_bounds__(NW * 64) void k_gemv_rows(const bf16* __restrict__ x, int64_t ldx,
                                                      const bf16* __restrict__ W, void* __restrict__ y, int M, int N,
                                                      int K, float scale, AttnX ax) {
  constexpr int NT = NW * 64;
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o = blockIdx.x * NW + wave;
  const bool live = o < nout;
  const int oc = live ? o : nout - 1;

  // activations first (vector loads complete in issue order), then weights
  constexpr int XV = (MB * CH * 64 + NT - 1) / NT;  // MB rows x nv <= 64*CH vectors over NT threads
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
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  u32x4 wv[NR][CH];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const u32x4* wr = (const u32x4*)(W + (size_t)(j ? nout + oc : oc) * K);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // clamped, unconditional: straight-line loads keep exact wait counts;
      // chunks past the row are ignored in the product below
      const int v = min(lane + 64 * c, nv - 1);
      wv[j][c] = __builtin_nontemporal_load(wr + v);
    }
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
  for (int c = 0; c < CH; ++c) {
    const int v = lane + 64 * c;
    if (v < nv) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const u32x4 xv = ((const u32x4*)(xs + (size_t)m * K))[v];
#pragma unroll
          for (int j = 0; j < NR; ++j) acc[m][j] = dot16(wv[j][c], xv, (const bf16*)nullptr, acc[m][j]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= M) break;
    const float s = wave_sum(acc[m][0]);
    if (EPI == EPI_SWIGLU) {
      const float g = wave_sum(acc[m][NR - 1]);
      if (lane == 0) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(s * scale * silu_(g * scale));
    } else {
      if (lane == 0) ((float*)y)[(size_t)m * N + o] = s * scale;
    }
  }
}

// Batch 1, float32 out, long rows (the down projection, K = d_ff): the K
// range of each output is split over two waves of CH chunks, 12 waves (6
// outputs) per workgroup, and the two halves' wave sums are added through
// LDS. Shorter load chains and twice the waves of k_gemv_rows: 9.6 us
// against 10.3 us on the 36-layer shape (3072 x 8192).
template <int CH>
__global__ __launch_bounds__(768) void k_gemv_rows_k2(const bf16* __restrict__ x, const bf16* __restrict__ W,
                                                     float* __restrict__ y, int N, int K, float scale) {
  constexpr int NW = 12, NT = NW * 64, OPW = NW / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float part[NW];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int o = blockIdx.x * OPW + (wave >> 1), half = wave & 1;
  const bool live = o < N;
  const int oc = live ? o : N - 1;
  constexpr int XV = (CH * 2 * 64 + NT - 1) / NT;
  u32x4 xr[XV];
#pragma unroll
  for (int q = 0; q < XV; ++q) xr[q] = ((const u32x4*)x)[min((int)threadIdx.x + NT * q, nv - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  u32x4 wv[CH];
  const u32x4* wr = (const u32x4*)(W + (size_t)oc * K);
#pragma unroll
  for (int c = 0; c < CH; ++c) wv[c] = __builtin_nontemporal_load(wr + min(half * CH * 64 + lane + 64 * c, nv - 1));
#pragma unroll
  for (int q = 0; q < XV; ++q) {
    const int e = threadIdx.x + NT * q;
    if (e < nv) ((u32x4*)xs)[e] = xr[q];
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int v = half * CH * 64 + lane + 64 * c;
    if (v < nv) acc = dot16(wv[c], ((const u32x4*)xs)[v], (const bf16*)nullptr, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (half == 0 && lane == 0 && live) y[o] = (part[wave] + part[wave + 1]) * scale;
}

// waves per workgroup of the rows kernels: one workgroup per CU when the
// outputs split evenly that way (12 for 3072 outputs, 9 for 2304), else 8
int rows_waves(int nout) {
  if (nout % kNumCUs == 0 && (nout / kNumCUs == 9 || nout / kNumCUs == 12 || nout / kNumCUs == 16))
    return nout / kNumCUs;
  return 8;
}

template <int MB, int EPI, int NW>
static bool gemv_rows_launch_nw(const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K, float scale,
                                hipStream_t st) {
  const int ch = (K / 8 + 63) / 64;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const dim3 grid((nout + NW - 1) / NW);
  const size_t lds = (size_t)M * K * 2;
#define DORY_ROWS(C)                                                                                          \
  case C:                                                                                                     \
    dory_launch((k_gemv_rows<MB, C, EPI, 0, NW>), grid, dim3(NW * 64), lds, st, x, ldx, W, y, M, N, K, scale, \
                AttnX{});                                                                                     \
    return true;
  switch (ch) {
    DORY_ROWS(1) DORY_ROWS(2) DORY_ROWS(3) DORY_ROWS(4) DORY_ROWS(5) DORY_ROWS(6) DORY_ROWS(8) DORY_ROWS(12)
    DORY_ROWS(16)
    default: return false;
  }
#undef DORY_ROWS
}

template <int MB, int EPI>
static bool gemv_rows_launch(const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K, float scale,
                             hipStream_t st) {
  if constexpr (MB == 1 && EPI == EPI_F32) {
    const int ch = (K / 8 + 63) / 64;  // chunks per lane of the one-wave-per-row kernel
    const dim3 grid((N + 5) / 6);
    if (ch == 16) {
      dory_launch(k_gemv_rows_k2<8>, grid, dim3(768), (uint32_t)K * 2, st, x, W, (float*)y, N, K, scale);
      return true;
    }
    if (ch == 12) {
      dory_launch(k_gemv_rows_k2<6>, grid, dim3(768), (uint32_t)K * 2, st, x, W, (float*)y, N, K, scale);
      return true;
    }
  }
  switch (rows_waves(EPI == EPI_SWIGLU ? N / 2 : N)) {
    case 9: return gemv_rows_launch_nw<MB, EPI, 9>(x, ldx, W, y, M, N, K, scale, st);
    case 12: return gemv_rows_launch_nw<MB, EPI, 12>(x, ldx, W, y, M, N, K, scale, st);
    case 16: return gemv_rows_launch_nw<MB, EPI, 16>(x, ldx, W, y, M, N, K, scale, st);
    default: return gemv_rows_launch_nw<MB, EPI, 8>(x, ldx, W, y, M, N, K, scale, st);
  }
}

// k_gemv_rows with the residual update in the prologue (see launch_linear_pro).
// 1024-thread workgroups (16 waves) with kProOut outputs per wave: the
// 36-layer shape's q|k|v|gate and up/gate projections become 256 workgroups,
// one per CU, all resident at once, and the prologue runs once per CU (the
// 72-layer shape's 6144 outputs take 12-wave workgroups for the same count). Each
// wave streams the chunks of its rows through a rolling window of kProWin
// 16-byte loads per lane: a CU keeps ~16 x kProWin KB in flight (enough to
// cover HBM latency at its share of the bandwidth) with few registers.
constexpr int kProThreads = 1024;
constexpr int kProOut = 2;  // outputs per wave
constexpr int kProWin = 8;  // chunk loads in flight per wave

template <int MB, int CH, int EPI, int NTH = kProThreads>
__global__ __launch_bounds__(NTH) void k_gemv_pro(GemvPro pr, const bf16* __restrict__ W,
                                                      void* __restrict__ y, int M, int N, int K, float scale) {
  constexpr int R = kProOut;
  constexpr int NR = (EPI == EPI_SWIGLU ? 2 : 1) * R;  // weight rows per wave
  constexpr int NC = NR * CH;                          // chunk loads per wave
  constexpr int P = NC < kProWin ? NC : kProWin;
  constexpr int NW = NTH / 64;
  constexpr int EPT = (CH * 512 + NTH - 1) / NTH;  // prologue elements per thread
  __shared__ float sh[3][NW];  // one slot per workgroup sum of a row: each reuse follows a barrier
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)smem;
  const int nv = K / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = (blockIdx.x * NW + wave) * R;  // outputs o0 .. o0+R-1
  const bool live = o0 < nout;

  // row j of this wave: output o0 + j % R; the u row (j < R) or the v row of SwiGLU.
  // Chunk c: with few rows M the order is position-major (c = cc * NR + j) so
  // that a position's activations are read from LDS once for all NR rows.
  constexpr bool kReuse = MB <= 2;
  auto cj = [](int c) { return kReuse ? c % NR : c / CH; };
  auto ccq = [](int c) { return kReuse ? c / NR : c % CH; };
  auto chunk_ptr = [&](int c) -> const u32x4* {
    const int j = cj(c), cc = ccq(c);
    const int oc = min(o0 + j % R, nout - 1);
    const int v = min(lane + 64 * cc, nv - 1);  // clamped: chunks past the row are ignored below
    return (const u32x4*)(W + (size_t)(j >= R ? nout + oc : oc) * K) + v;
  };

  // prologue inputs of row 0 first (vector loads complete in issue order),
  // then the first P weight chunks; element i = threadIdx.x + NTH*c.
  // e is read from y when there is no re-injection so no branch separates loads.
  const float* ep = pr.e ? pr.e : pr.y;
  float yv[EPT], hv[EPT], ev[EPT], av[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) {
    const int i = min((int)threadIdx.x + NTH * c, K - 1);
    yv[c] = pr.y[i];
    hv[c] = pr.h_in[i];
    ev[c] = ep[i];
    av[c] = pr.alpha[i];  // before the weights: the update must not wait behind them
  }
  if (pr.zero)
    for (int i = blockIdx.x * NTH + threadIdx.x; i < pr.zero_n; i += gridDim.x * NTH) pr.zero[i] = 0ull;
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
        const int i = min((int)threadIdx.x + NTH * c, K - 1);
        yv[c] = pr.y[ro + i];
        hv[c] = pr.h_in[ro + i];
        ev[c] = ep[ro + i];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      if ((int)threadIdx.x + NTH * c >= K) yv[c] = 0.f, hv[c] = 0.f, ev[c] = 0.f;
      ss += yv[c] * yv[c];
    }
    const float iy = inv_norm(block_sum_slot<NTH>(ss, sh[0]));
    float st = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const float al = (int)threadIdx.x + NTH * c < K ? av[c] : 0.f;
      hv[c] = hv[c] + al * (yv[c] * iy - hv[c]);
      st += hv[c] * hv[c];
    }
    const float ih = inv_norm(block_sum_slot<NTH>(st, sh[1]));
#pragma unroll
    for (int c = 0; c < EPT; ++c) hv[c] *= ih;  // u
    if (pr.e_out && blockIdx.x == 0) {
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        const int i = threadIdx.x + NTH * c;
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
      const float iv = inv_norm(block_sum_slot<NTH>(sv, sh[2]));
#pragma unroll
      for (int c = 0; c < EPT; ++c) hv[c] = yv[c] * iv;
    }
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
      const int i = threadIdx.x + NTH * c;
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
  u32x4 xq[kReuse ? MB : 1];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const u32x4 w = buf[c % P];
    if (c + P < NC) buf[c % P] = __builtin_nontemporal_load(chunk_ptr(c + P));
    const int j = cj(c), cc = ccq(c);
    if (kReuse && j == 0) {
#pragma unroll
      for (int m = 0; m < (kReuse ? MB : 1); ++m)
        if (m < M) xq[m] = ((const u32x4*)(xs + (size_t)m * K))[min(lane + 64 * cc, nv - 1)];
    }
    if (lane + 64 * cc < nv) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const u32x4 xv = kReuse ? xq[kReuse ? m : 0] : ((const u32x4*)(xs + (size_t)m * K))[lane + 64 * cc];
          acc[m][j] = dot16(w, xv, (const bf16*)nullptr, acc[m][j]);
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
      const float s = wave_sum(acc[m][r]);
      if (EPI == EPI_SWIGLU) {
        const float g = wave_sum(acc[m][R + r]);
        if (lane == 0 && o < nout) ((bf16*)y)[(size_t)m * nout + o] = from_f<bf16>(s * scale * silu_(g * scale));
      } else {
        if (lane == 0 && o < nout) ((float*)y)[(size_t)m * N + o] = s * scale;
      }
    }
  }
}

template <int MB, int EPI>
static hipError_t gemv_pro_launch(const GemvPro& p, const bf16* W, void* y, int M, int N, int K, float scale,
                                  hipStream_t st) {
  const int ch = (K / 8 + 63) / 64;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const size_t lds = (size_t)M * K * 2;
  // batch 1, 12 x 2 outputs per CU: 12-wave workgroups keep one per CU (16
  // waves would leave a quarter of the CUs idle)
  if (MB == 1 && nout == 12 * kProOut * kNumCUs && ch <= 8) {
    const dim3 grid12(kNumCUs);
#define DORY_PRO12(C)                                                                                          \
  case C:                                                                                                      \
    dory_launch((k_gemv_pro<MB, C, EPI, 768>), grid12, dim3(768), lds, st, p, W, y, M, N, K, scale); \
    return hipGetLastError();
    switch (ch) {
      DORY_PRO12(1) DORY_PRO12(2) DORY_PRO12(3) DORY_PRO12(4) DORY_PRO12(5) DORY_PRO12(6) DORY_PRO12(7)
      DORY_PRO12(8)
      default: break;
    }
#undef DORY_PRO12
  }
  const int per_block = kProThreads / 64 * kProOut;
  const dim3 grid((nout + per_block - 1) / per_block);
#define DORY_PRO(C) \
  case C: dory_launch((k_gemv_pro<MB, C, EPI>), grid, dim3(kProThreads), lds, st, p, W, y, M, N, K, scale); break;
  switch (ch) {
    DORY_PRO(1) DORY_PRO(2) DORY_PRO(3) DORY_PRO(4) DORY_PRO(5) DORY_PRO(6) DORY_PRO(7) DORY_PRO(8)
    DORY_PRO(12) DORY_PRO(16)
    default: return hipErrorInvalidValue;
  }
#undef DORY_PRO
  return hipGetLastError();
}

bool linear_pro_supported(int M, int K) {
  const int ch = (K / 8 + 63) / 64;
  return M >= 1 && M <= 8 && K % 8 == 0 && (size_t)M * K * 2 <= 64 * 1024 && (ch <= 8 || ch == 12 || ch == 16);
}

hipError_t launch_linear_pro(const GemvPro& p, const void* W, void* y, int M, int N, int K, int epi, float scale,
                             hipStream_t st) {
  if (M < 1 || M > 8 || K % 8 || (size_t)M * K * 2 > 64 * 1024 || ((uintptr_t)W & 15)) return hipErrorInvalidValue;
  const bf16* w = (const bf16*)W;
#define DORY_PRO_M(E)                                                                                    \
  if (M == 1) return gemv_pro_launch<1, E>(p, w, y, M, N, K, scale, st);                                  \
  if (M == 2) return gemv_pro_launch<2, E>(p, w, y, M, N, K, scale, st);                                  \
  if (M <= 4) return gemv_pro_launch<4, E>(p, w, y, M, N, K, scale, st);                                  \
  return gemv_pro_launch<8, E>(p, w, y, M, N, K, scale, st);
  if (epi == EPI_SWIGLU) {
    DORY_PRO_M(EPI_SWIGLU)
  }
  DORY_PRO_M(EPI_F32)
#undef DORY_PRO_M
}

// Scalar GEMV (any K, any alignment): one wave per output.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemv_scalar(const T* __restrict__ x, int64_t ldx, const T* __restrict__ W,
                                                    void* __restrict__ y, int M, int N, int K, float scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o = blockIdx.x * 4 + wave;
  const int m = blockIdx.y;
  if (o >= nout) return;
  const T* xr = x + (size_t)m * ldx;
  const T* w0 = W + (size_t)o * K;
  const T* w1 = W + (size_t)(nout + o) * K;
  float s0 = 0.f, s1 = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float xv = to_f(xr[k]);
    s0 = fmaf(to_f(w0[k]), xv, s0);
    if (EPI == EPI_SWIGLU) s1 = fmaf(to_f(w1[k]), xv, s1);
  }
  s0 = wave_sum(s0);
  if (EPI == EPI_SWIGLU) s1 = wave_sum(s1);
  if (lane == 0) {
    if (EPI == EPI_SWIGLU)
      ((T*)y)[(size_t)m * nout + o] = from_f<T>(s0 * scale * silu_(s1 * scale));
    else
      ((float*)y)[(size_t)m * N + o] = s0 * scale;
  }
}

// ---------------------------------------------------------------------------
// MFMA GEMM (bfloat16 in, float32 accumulate)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;  // 144-byte LDS rows

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_mfma(const bf16* __restrict__ A, int64_t lda,
                                                  const bf16* __restrict__ B, void* __restrict__ C, int M, int N,
                                                  int K, float scale) {
  __shared__ __align__(16) bf16 As[GBM * GLD];
  __shared__ __align__(16) bf16 Bs[GBN * GLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * GBM;
  const int F = N / 2;
  const int n0 = EPI == EPI_SWIGLU ? blockIdx.x * (GBN / 2) : blockIdx.x * GBN;

  // each thread moves 4 x 16 B of A and of B per K tile
  int arow[4], brow[4], col8[4];
  bool aok[4], bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3;
    col8[i] = (c & 7) * 8;
    arow[i] = m0 + r;
    aok[i] = arow[i] < M;
    int br;
    if (EPI == EPI_SWIGLU) {
      const int nb = r >> 5;
      const int o = n0 + (nb >> 1) * 32 + (r & 31);
      bok[i] = o < F;
      br = (nb & 1 ? F : 0) + o;
    } else {
      br = n0 + r;
      bok[i] = br < N;
    }
    brow[i] = br;
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + col8[i];
      const bool kin = k < K;
      ra[i] = (aok[i] && kin) ? *(const uint4*)(A + (size_t)arow[i] * lda + k) : make_uint4(0, 0, 0, 0);
      rb[i] = (bok[i] && kin) ? *(const uint4*)(B + (size_t)brow[i] * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + 256 * i) >> 3;
      *(uint4*)(As + r * GLD + col8[i]) = ra[i];
      *(uint4*)(Bs + r * GLD + col8[i]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  sstore();
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int k0 = 0; k0 < K; k0 += GBK) {
    const bool more = k0 + GBK < K;
    if (more) gload(k0 + GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8_t*)(As + (wm * 64 + i * 32 + lr) * GLD + ks * 16 + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8_t*)(Bs + (wn * 64 + j * 32 + lr) * GLD + ks * 16 + lk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      sstore();
      __syncthreads();
    }
  }

  // C layout of a 32x32 block: register r of lane l -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
        const int o = n0 + wn * 32 + lr;
        if (o < F) ((bf16*)C)[(size_t)row * F + o] = from_f<bf16>(acc[i][0][r] * scale * silu_(acc[i][1][r] * scale));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + lr;
          if (col < N) ((float*)C)[(size_t)row * N + col] = acc[i][j][r] * scale;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M prefill GEMM: 256 x BN workgroup tiles (BN = 256, or 192 where 256
// would leave the last round of workgroups half empty, e.g. N = 3072), four
// waves (one per SIMD) in a 2 x 2 grid of 128 x BN/2, so every LDS fragment
// feeds BN/64 (A) or 4 (B) matrix-core products. The 4 x BN/64 accumulator
// blocks of v_mfma_f32_32x32x16_bf16 (256 floats per lane at BN = 256) live
// in the accumulation registers.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4:
// lane l of a wave's load writes bytes 16l..16l+15 of a 1 KB block). A stage
// is 64 deep in K, so a load covers 8 tile rows x 128 B — whole cache lines
// (16 rows x 64 B per load, a 32-deep stage, streamed measurably slower).
// Inside a row the 16-byte chunks are XOR-swizzled by (row/2)%8, which makes
// the 16-lane groups of the fragment reads hit distinct banks (no bank
// conflicts by the counters). The 160 KB of LDS hold A in a three-slot ring
// and B in a two-slot ring: the loads of A for stage kt+2 go out in three
// pieces during stage kt, those of B for stage kt+2 right after the barrier
// that ends stage kt (the slot that stage kt's B used is then free: its last
// 16-deep slice is already in registers), so every load has one to two
// stages of matrix work to land. One workgroup barrier per stage, after an
// explicit vmcnt wait for stage kt+1 (A of stage kt+2 stays in flight).
// Within a stage the fragments of the next 16-deep slice are read while the
// current one is multiplied, one LDS read (or global load) issued after each
// product (sched_group_barrier), so neither unit sees bursts.
//
// Workgroups are spread over the 8 XCDs in contiguous runs of tiles, grouped
// four M tiles at a time, so the tiles that run together on one XCD share A
// and B rows in its L2. SwiGLU (BN = 256 only): B tile rows come in 32-row
// chunks u, v, u, v of the same outputs, and a wave's blocks (0, 1) and
// (2, 3) are (u, v) pairs. Requires K % 64 == 0 and 16-byte aligned rows.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding)
#define DORY_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// s_waitcnt lgkmcnt(0) and no wait on the other counters
#define DORY_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4))
// sched_group_barrier masks
#define DORY_SG_MFMA 0x008
#define DORY_SG_VMEM_RD 0x020
#define DORY_SG_DS_RD 0x100

constexpr int kBigBK = 64;      // K per stage
constexpr int kBigGroupM = 4;
constexpr int kBigLds = 160 * 1024;

// 16 bytes per lane from global memory straight into LDS (a wave fills dst ..
// dst + 1023). A plain device function: called directly from a lambda of a
// kernel template, the builtin made host compilation drop its callers.
__device__ __forceinline__ void lds_load16(const bf16* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

// byte offset of 16-byte chunk c (K elements 8c..8c+7) of tile row r in a stage
__device__ __forceinline__ int big_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int EPI, int BN>
__global__ __launch_bounds__(256) void k_gemm_big(const bf16* __restrict__ A, int64_t lda,
                                                  const bf16* __restrict__ B, void* __restrict__ C, int M, int N,
                                                  int K, float scale) {
  static_assert(BN == 256 || (BN == 192 && EPI == EPI_F32), "tile widths");
  constexpr int NJ = BN / 64;          // 32-column blocks per wave
  constexpr int kHA = 256 * 128;       // A bytes per stage (32 KB)
  constexpr int kHB = BN * 128;        // B bytes per stage (32 or 24 KB)
  constexpr int kLA = kHA / 4096;      // 1 KB loads per wave per stage: A 8, B 8 or 6
  constexpr int kLB = kHB / 4096;
  extern __shared__ __align__(1024) unsigned char smem[];
  unsigned char* const sA = smem;             // 3 x kHA
  unsigned char* const sB = smem + 3 * kHA;   // 2 x kHB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;  // rows wm*128, columns wn*BN/2 of the tile
  const int F = N / 2;
  const int nM = (M + 255) / 256;
  const int nN = EPI == EPI_SWIGLU ? (F + 127) / 128 : (N + BN - 1) / BN;
  const int nt = nM * nN;
  const int per = (nt + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= nt) return;
  const int grp = t / (kBigGroupM * nN);
  const int gs = min(kBigGroupM, nM - grp * kBigGroupM);
  const int loc = t - grp * kBigGroupM * nN;
  const int m0 = (grp * kBigGroupM + loc % gs) * 256;
  const int n0 = EPI == EPI_SWIGLU ? (loc / gs) * 128 : (loc / gs) * BN;

  // this lane's source rows (clamped: rows past M or N load a valid row and
  // are never stored); load i of a wave fills tile rows 8 (wave kL + i) + 0..7
  const int lr = lane >> 3, ls = lane & 7;
  const bf16* srcA[kLA];
  const bf16* srcB[kLB];
#pragma unroll
  for (int i = 0; i < kLA; ++i) {
    const int r = (wave * kLA + i) * 8 + lr;
    srcA[i] = A + (size_t)min(m0 + r, M - 1) * lda + (ls ^ ((r >> 1) & 7)) * 8;
  }
#pragma unroll
  for (int i = 0; i < kLB; ++i) {
    const int r = (wave * kLB + i) * 8 + lr;
    int wr;
    if (EPI == EPI_SWIGLU) {
      const int nb = r >> 5;
      const int o = min(n0 + (nb >> 1) * 32 + (r & 31), F - 1);
      wr = (nb & 1 ? F : 0) + o;
    } else {
      wr = min(n0 + r, N - 1);
    }
    srcB[i] = B + (size_t)wr * K + (ls ^ ((r >> 1) & 7)) * 8;
  }
  auto issueA = [&](int kt, int i0, int i1) {
    unsigned char* st = sA + (kt % 3) * kHA;
#pragma unroll
    for (int i = i0; i < i1; ++i) lds_load16(srcA[i] + kt * kBigBK, st + (wave * kLA + i) * 1024);
  };
  auto issueB = [&](int kt) {
    unsigned char* st = sB + (kt & 1) * kHB;
#pragma unroll
    for (int i = 0; i < kLB; ++i) lds_load16(srcB[i] + kt * kBigBK, st + (wave * kLB + i) * 1024);
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nK = K / kBigBK;
  const int l32 = lane & 31, lh = lane >> 5;
  // fragments of 16-deep K slice ks (0..3) of stage kt
  auto frag = [&](int kt, int ks, bf16x8_t (&fa)[4], bf16x8_t (&fb)[NJ]) {
    const unsigned char* a = sA + (kt % 3) * kHA;
    const unsigned char* b = sB + (kt & 1) * kHB;
    const int c = ks * 2 + lh;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8_t*)(a + big_off(wm * 128 + i * 32 + l32, c));
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = *(const bf16x8_t*)(b + big_off(wn * (BN / 2) + j * 32 + l32, c));
  };
  auto mma = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  bf16x8_t fa[2][4], fb[2][NJ];
  // prologue: A and B of stages 0 and 1
  issueA(0, 0, kLA);
  issueB(0);
  if (nK > 1) {
    issueA(1, 0, kLA);
    issueB(1);
    DORY_WAIT_VM(kLA + kLB);
  } else {
    DORY_WAIT_VM(0);
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  frag(0, 0, fa[0], fb[0]);
  DORY_WAIT_LGKM0();
  for (int kt = 0; kt < nK; ++kt) {
    const bool moreA = kt + 2 < nK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) {
        // a third of A(kt+2) into the A slot stage kt-1 used; fragments of slice s+1
        constexpr int c0[3] = {0, kLA / 3, 2 * kLA / 3}, c1[3] = {kLA / 3, 2 * kLA / 3, kLA};
        if (moreA) issueA(kt + 2, c0[s], c1[s]);
        frag(kt, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
        mma(fa[s & 1], fb[s & 1]);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_VMEM_RD, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 4 + NJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_DS_RD, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 4 * NJ - 7 - NJ, 0);
      } else {
        // stage kt+1 complete (A of stage kt+2 may stay in flight), then B of
        // stage kt+2 into the B slot stage kt used, fragments of stage kt+1
        if (moreA) DORY_WAIT_VM(kLA); else DORY_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 2 < nK) issueB(kt + 2);
        frag(kt + 1, 0, fa[0], fb[0]);  // unconditional (past the last stage: a stale slot, unused): exact waits
        mma(fa[1], fb[1]);
#pragma unroll
        for (int q = 0; q < kLB; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_VMEM_RD, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 4 + NJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_DS_RD, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // the fragment reads are done long before the products are: waiting
      // here lets the next slice's products start without a wait
      DORY_WAIT_LGKM0();
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // C layout of a 32x32 block: register r of lane l -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int jp = 0; jp < NJ / 2; ++jp) {
          const int o = n0 + wn * 64 + jp * 32 + l32;
          if (o < F)
            ((bf16*)C)[(size_t)row * F + o] =
                from_f<bf16>(acc[i][2 * jp][r] * scale * silu_(acc[i][2 * jp + 1][r] * scale));
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = n0 + wn * (BN / 2) + j * 32 + l32;
          if (col < N) ((float*)C)[(size_t)row * N + col] = acc[i][j][r] * scale;
        }
      }
    }
  }
}

// LDS bytes of k_gemm_big (three A slots and two B slots of one stage)
static constexpr uint32_t big_lds(int bn) { return 3 * 256 * 128 + 2 * bn * 128; }

// k_gemm_big<EPI, BN> with its dynamic LDS above the 64 KB default allowed
// (set once per process)
template <int EPI, int BN>
static void big_launch(dim3 grid, const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K, float scale,
                       hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_gemm_big<EPI, BN>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)big_lds(BN));
  (void)attr;
  dory_launch((k_gemm_big<EPI, BN>), grid, dim3(256), big_lds(BN), st, x, ldx, W, y, M, N, K, scale);
}

// tile width for a large-M GEMM with N outputs: 192 when 256-wide tiles would
// leave the last round of workgroups (one per CU) at most half full and
// 192-wide ones do better
static int big_tile_n(int M, int N) {
  auto eff = [&](int bn) {
    const long tiles = (long)((M + 255) / 256) * ((N + bn - 1) / bn);
    const long rounds = (tiles + kNumCUs - 1) / kNumCUs;
    return (double)tiles / (double)(rounds * kNumCUs) * (bn == 256 ? 1.0 : 0.93);  // 192: more LDS reads per FLOP
  };
  return eff(192) > eff(256) ? 192 : 256;
}

// ---------------------------------------------------------------------------
// Batched-decode GEMM (9..64 rows): weight-stream bound. A workgroup owns 16
// outputs (16 weight rows; SwiGLU: those 16 u rows and the 16 matching v
// rows) and all M rows; its four waves split K in quarters. With
// v_mfma_f32_16x16x32_bf16 lane l supplies row l%16 of a 16-row block and K
// elements 8(l/16)..8(l/16)+7 of each 32-deep step, so every operand
// fragment is one 16-byte load straight from global memory (the weights
// stream once, the activations come from L2); four steps of loads are issued
// before their products. The quarters are summed through LDS. Rows past M
// and outputs past N are clamped loads whose results are dropped. Requires
// K % 128 == 0 and 16-byte aligned rows.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kSkU = 4;  // K steps of 32 whose loads are issued together

template <int MB, int EPI>
__global__ __launch_bounds__(256) void k_gemm_skinny(const bf16* __restrict__ X, int64_t ldx,
                                                     const bf16* __restrict__ W, void* __restrict__ C, int M, int N,
                                                     int K, float scale) {
  constexpr int NB = MB / 16;                  // 16-row blocks of X
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;  // weight blocks (u, v)
  __shared__ f32x4_t part[4][NR][NB][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = blockIdx.x * 16;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int kper = K / 4, kb = wave * kper;
  const bf16* wp[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) wp[j] = W + (size_t)((j ? nout : 0) + min(o0 + r16, nout - 1)) * K + kb + kq;
  const bf16* xp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) xp[b] = X + (size_t)min(b * 16 + r16, M - 1) * ldx + kb + kq;
  f32x4_t acc[NR][NB];
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kper; k += 32 * kSkU) {
    bf16x8_t wf[kSkU][NR], xf[kSkU][NB];
#pragma unroll
    for (int u = 0; u < kSkU; ++u) {
      const int kk = min(k + 32 * u, kper - 32);  // past the quarter: a re-read, not multiplied
#pragma unroll
      for (int j = 0; j < NR; ++j) wf[u][j] = __builtin_nontemporal_load((const bf16x8_t*)(wp[j] + kk));
#pragma unroll
      for (int b = 0; b < NB; ++b) xf[u][b] = *(const bf16x8_t*)(xp[b] + kk);
    }
#pragma unroll
    for (int u = 0; u < kSkU; ++u) {
      if (k + 32 * u >= kper) break;
#pragma unroll
      for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u][b], wf[u][j], acc[j][b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b) part[wave][j][b][lane] = acc[j][b];
  __syncthreads();
  // output (row m, column n) of block b: lane n + 16 (m%16 / 4), register m % 4
  for (int e = tid; e < MB * 16; e += 256) {
    const int m = e >> 4, n = e & 15;
    const int b = m >> 4, ln = n + 16 * ((m & 15) >> 2), r = m & 3;
    float s[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) s[j] = part[0][j][b][ln][r] + part[1][j][b][ln][r] + part[2][j][b][ln][r] +
                                        part[3][j][b][ln][r];
    if (m >= M || o0 + n >= nout) continue;
    if (EPI == EPI_SWIGLU)
      ((bf16*)C)[(size_t)m * nout + o0 + n] = from_f<bf16>(s[0] * scale * silu_(s[1] * scale));
    else
      ((float*)C)[(size_t)m * N + o0 + n] = s[0] * scale;
  }
}

// ---------------------------------------------------------------------------
// Simple tiled GEMM for float32 models and ragged shapes: 64x64 tiles, each
// thread a 4x4 block, K in steps of 16 through LDS.
// ---------------------------------------------------------------------------
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemm_simple(const T* __restrict__ A, int64_t lda, const T* __restrict__ B,
                                                    void* __restrict__ C, int M, int N, int K, float scale) {
  __shared__ float As[16][65];
  __shared__ float Bs[2][16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  float acc[2][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int rr = e >> 4, kk = e & 15;
      const int gm = m0 + rr, gn = n0 + rr, gk = k0 + kk;
      As[kk][rr] = (gm < M && gk < K) ? to_f(A[(size_t)gm * lda + gk]) : 0.f;
      Bs[0][kk][rr] = (gn < nout && gk < K) ? to_f(B[(size_t)gn * K + gk]) : 0.f;
      if (EPI == EPI_SWIGLU) Bs[1][kk][rr] = (gn < nout && gk < K) ? to_f(B[(size_t)(nout + gn) * K + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs[0][kk][tx * 4 + j];
        b1[j] = EPI == EPI_SWIGLU ? Bs[1][kk][tx * 4 + j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][i][j] = fmaf(a[i], b0[j], acc[0][i][j]);
          if (EPI == EPI_SWIGLU) acc[1][i][j] = fmaf(a[i], b1[j], acc[1][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= nout) continue;
      if (EPI == EPI_SWIGLU)
        ((T*)C)[(size_t)row * nout + col] = from_f<T>(acc[0][i][j] * scale * silu_(acc[1][i][j] * scale));
      else
        ((float*)C)[(size_t)row * N + col] = acc[0][i][j] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename T, int EPI>
static hipError_t gemv_dispatch(const T* x, int64_t ldx, const T* W, void* y, int M, int N, int K, float scale,
                                hipStream_t st) {
  constexpr int VEC = 16 / sizeof(T);
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const bool vec_ok = (K % VEC == 0) && (ldx % VEC == 0) && (((uintptr_t)x & 15) == 0) &&
                      (((uintptr_t)W & 15) == 0);
  const size_t osz = EPI == EPI_SWIGLU ? sizeof(T) : sizeof(float);
  const int ostride = EPI == EPI_SWIGLU ? nout : N;
  if (!vec_ok) {
    dim3 grid((nout + 3) / 4, M);
    dory_launch((k_gemv_scalar<T, EPI>), grid, dim3(256), 0, st, x, ldx, W, y, M, N, K, scale);
    return hipGetLastError();
  }
  if (sizeof(T) == 2) {
    // row-loads-first kernel: up to 8 rows per launch, staged rows within 64 KB
    int mb = (int)((64 * 1024) / ((size_t)K * 2));
    mb = mb > 8 ? 8 : mb;
    bool ok = mb >= 1;
    for (int m0 = 0; ok && m0 < M; m0 += mb) {
      const int mm = M - m0 < mb ? M - m0 : mb;
      const bf16* xm = (const bf16*)x + (size_t)m0 * ldx;
      void* ym = (char*)y + (size_t)m0 * ostride * osz;
      if (mm == 1) ok = gemv_rows_launch<1, EPI>(xm, ldx, (const bf16*)W, ym, mm, N, K, scale, st);
      else if (mm == 2) ok = gemv_rows_launch<2, EPI>(xm, ldx, (const bf16*)W, ym, mm, N, K, scale, st);
      else if (mm <= 4) ok = gemv_rows_launch<4, EPI>(xm, ldx, (const bf16*)W, ym, mm, N, K, scale, st);
      else ok = gemv_rows_launch<8, EPI>(xm, ldx, (const bf16*)W, ym, mm, N, K, scale, st);
      if (ok) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      } else if (m0 != 0) {
        return hipErrorInvalidValue;  // chunk count is a property of K: never changes mid-way
      }
    }
    if (ok) return hipSuccess;
  }
  // rows per launch limited by LDS (64 KB of staged activations)
  int mb = (int)((64 * 1024) / ((size_t)K * sizeof(T)));
  mb = mb < 1 ? 1 : (mb > 8 ? 8 : mb);
  for (int m0 = 0; m0 < M; m0 += mb) {
    const int mm = M - m0 < mb ? M - m0 : mb;
    const T* xm = x + (size_t)m0 * ldx;
    void* ym = (char*)y + (size_t)m0 * ostride * osz;
    const size_t lds = (size_t)mm * K * sizeof(T);
    // two rows per wave unless that leaves too few workgroups to fill 256 CUs
    const int rows = (nout >= 4096) ? 2 : 1;
    const int grid = (nout + 4 * rows - 1) / (4 * rows);
#define DORY_GEMV(MBV, RV) \
  dory_launch((k_gemv_vec<T, MBV, RV, EPI>), dim3(grid), dim3(256), lds, st, xm, ldx, W, ym, mm, N, K, scale)
    if (rows == 2) {
      if (mm == 1) DORY_GEMV(1, 2); else if (mm == 2) DORY_GEMV(2, 2); else if (mm <= 4) DORY_GEMV(4, 2); else DORY_GEMV(8, 2);
    } else {
      if (mm == 1) DORY_GEMV(1, 1); else if (mm == 2) DORY_GEMV(2, 1); else if (mm <= 4) DORY_GEMV(4, 1); else DORY_GEMV(8, 1);
    }
#undef DORY_GEMV
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int EPI>
static hipError_t gemm_dispatch(const T* x, int64_t ldx, const T* W, void* y, int M, int N, int K, float scale,
                                hipStream_t st) {
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const bool al16 = ldx % 8 == 0 && (((uintptr_t)x & 15) == 0) && (((uintptr_t)W & 15) == 0);
  if (sizeof(T) == 2 && al16 && K % kBigBK == 0 && M >= 1024) {
    const int bn = EPI == EPI_SWIGLU ? 256 : big_tile_n(M, N);
    const int tiles = ((M + 255) / 256) * (EPI == EPI_SWIGLU ? (nout + 127) / 128 : (N + bn - 1) / bn);
    if (bn == 192)
      big_launch<EPI_F32, 192>(dim3((tiles + 7) / 8 * 8), (const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st);
    else
      big_launch<EPI, 256>(dim3((tiles + 7) / 8 * 8), (const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st);
  } else if (sizeof(T) == 2 && al16 && K % 128 == 0 && M <= 64) {
    const dim3 grid((nout + 15) / 16);
    if (M <= 16)
      dory_launch((k_gemm_skinny<16, EPI>), grid, dim3(256), 0, st, (const bf16*)x, ldx, (const bf16*)W, y, M, N, K,
                  scale);
    else if (M <= 32)
      dory_launch((k_gemm_skinny<32, EPI>), grid, dim3(256), 0, st, (const bf16*)x, ldx, (const bf16*)W, y, M, N, K,
                  scale);
    else
      dory_launch((k_gemm_skinny<64, EPI>), grid, dim3(256), 0, st, (const bf16*)x, ldx, (const bf16*)W, y, M, N, K,
                  scale);
  } else if (sizeof(T) == 2 && K % 8 == 0 && al16) {
    const int nt = EPI == EPI_SWIGLU ? (nout + GBN / 2 - 1) / (GBN / 2) : (N + GBN - 1) / GBN;
    dim3 grid(nt, (M + GBM - 1) / GBM);
    dory_launch((k_gemm_mfma<EPI>), grid, dim3(256), 0, st, (const bf16*)x, ldx, (const bf16*)W, y, M, N, K,
                       scale);
  } else {
    dim3 grid((nout + 63) / 64, (M + 63) / 64);
    dory_launch((k_gemm_simple<T, EPI>), grid, dim3(256), 0, st, x, ldx, W, y, M, N, K, scale);
  }
  return hipGetLastError();
}

bool linear_attn_supported(int M, int K) {
  const int ch = (K / 8 + 63) / 64;
  return M >= 1 && M <= 8 && K % 8 == 0 && (size_t)M * K * 2 <= 64 * 1024 &&
         ((ch >= 1 && ch <= 6) || ch == 8 || ch == 12 || ch == 16);
}

template <int MB, int NW>
static hipError_t linear_attn_nw(const AttnX& ax, const bf16* W, float* y, int M, int N, int K, float scale,
                                 hipStream_t st) {
  const int ch = (K / 8 + 63) / 64;
  const dim3 grid((N + NW - 1) / NW);
  const size_t lds = (size_t)M * K * 2;
#define DORY_AROWS(C)                                                                                       \
  case C:                                                                                                   \
    dory_launch((k_gemv_rows<MB, C, EPI_F32, 1, NW>), grid, dim3(NW * 64), lds, st, (const bf16*)nullptr,   \
                (int64_t)K, W, (void*)y, M, N, K, scale, ax);                                               \
    break;
  switch (ch) {
    DORY_AROWS(1) DORY_AROWS(2) DORY_AROWS(3) DORY_AROWS(4) DORY_AROWS(5) DORY_AROWS(6) DORY_AROWS(8)
    DORY_AROWS(12) DORY_AROWS(16)
    default: return hipErrorInvalidValue;
  }
#undef DORY_AROWS
  return hipGetLastError();
}

template <int MB>
static hipError_t linear_attn_mb(const AttnX& ax, const bf16* W, float* y, int M, int N, int K, float scale,
                                 hipStream_t st) {
  switch (rows_waves(N)) {
    case 9: return linear_attn_nw<MB, 9>(ax, W, y, M, N, K, scale, st);
    case 12: return linear_attn_nw<MB, 12>(ax, W, y, M, N, K, scale, st);
    case 16: return linear_attn_nw<MB, 16>(ax, W, y, M, N, K, scale, st);
    default: return linear_attn_nw<MB, 8>(ax, W, y, M, N, K, scale, st);
  }
}

hipError_t launch_linear_attn(const AttnX& ax, const void* W, float* y, int M, int N, int K, float scale,
                              hipStream_t st) {
  if (!linear_attn_supported(M, K) || ax.hd % 8 || K != ax.nq * ax.hd || ((uintptr_t)W & 15)) return hipErrorInvalidValue;
  const bf16* w = (const bf16*)W;
  if (M == 1) return linear_attn_mb<1>(ax, w, y, M, N, K, scale, st);
  if (M == 2) return linear_attn_mb<2>(ax, w, y, M, N, K, scale, st);
  if (M <= 4) return linear_attn_mb<4>(ax, w, y, M, N, K, scale, st);
  return linear_attn_mb<8>(ax, w, y, M, N, K, scale, st);
}

hipError_t launch_linear(int dtype, const void* x, int64_t ldx, const void* W, void* y, int M, int N, int K, int epi,
                         float scale, int algo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const bool gemv = algo == 1 || (algo == 0 && M <= 8);
#define DORY_LIN(T)                                                                                       \
  do {                                                                                                    \
    if (epi == EPI_SWIGLU)                                                                                \
      return gemv ? gemv_dispatch<T, EPI_SWIGLU>((const T*)x, ldx, (const T*)W, y, M, N, K, scale, st)   \
                  : gemm_dispatch<T, EPI_SWIGLU>((const T*)x, ldx, (const T*)W, y, M, N, K, scale, st);  \
    return gemv ? gemv_dispatch<T, EPI_F32>((const T*)x, ldx, (const T*)W, y, M, N, K, scale, st)        \
                : gemm_dispatch<T, EPI_F32>((const T*)x, ldx, (const T*)W, y, M, N, K, scale, st);       \
  } while (0)
  if (dtype == 0) DORY_LIN(float);
  DORY_LIN(bf16);
#undef DORY_LIN
}

}  // namespace dory
