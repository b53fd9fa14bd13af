// Decode linear layers y = x . W^T of the looped nGPT at 1..8 rows (the
// fused q|k|v|gate projection, the attention output projection, the SwiGLU
// up/gate projection, the down projection and the tied LM head): HBM-bound
// weight streaming, every weight byte read once per step.
//
//  * k_gemv_pro: the q|k|v|gate and up/gate projections with the nGPT update
//    (or the loop re-injection) of the previous sub-layer fused in front.
//  * k_gemv_rows / k_gemv_rows_k2: row-loads-first GEMVs (k2: each weight
//    row's K range on two waves); k_gemv_rows with XM = 1 stages its input
//    from the decode attention's fixed-point sums.
//  * k_gemv_vec / k_gemv_scalar: the remaining shapes and float32 models.
//
// Epilogue 1 (SwiGLU) pairs row o of u with row F + o of v inside one wave
// and stores u * silu(v) in the model dtype. More than 8 rows go to the
// matrix-core GEMMs.
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
constexpr int kProWin = 12;  // chunk loads in flight per wave

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
  if (!gemv) return launch_gemm(dtype, x, ldx, W, y, M, N, K, epi, scale, st);
  if (dtype == 0)
    return epi == EPI_SWIGLU ? gemv_dispatch<float, EPI_SWIGLU>((const float*)x, ldx, (const float*)W, y, M, N, K, scale, st)
                             : gemv_dispatch<float, EPI_F32>((const float*)x, ldx, (const float*)W, y, M, N, K, scale, st);
  return epi == EPI_SWIGLU ? gemv_dispatch<bf16, EPI_SWIGLU>((const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st)
                           : gemv_dispatch<bf16, EPI_F32>((const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st);
}

}  // namespace dory
