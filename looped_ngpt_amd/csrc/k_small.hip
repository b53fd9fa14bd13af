// Row-wise kernels of the looped nGPT forward: embedding + norm, the nGPT
// hypersphere update, the loop re-injection, RoPE tables, RoPE with per-head
// q/k normalisation, the KV-cache writer and the greedy argmax.
//
// Row kernels use one 256-thread workgroup per row of d_model elements, each
// thread holding EPT elements in registers, so a row is read from memory once
// and the two L2 norms are workgroup reductions.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "dory.h"
#include "kernels.h"

namespace dory {

static thread_local LaunchEvents g_next_events{nullptr, nullptr};
void set_next_launch_events(hipEvent_t start, hipEvent_t stop) { g_next_events = LaunchEvents{start, stop}; }
LaunchEvents take_next_launch_events() {
  const LaunchEvents e = g_next_events;
  g_next_events = LaunchEvents{nullptr, nullptr};
  return e;
}

constexpr int kRowThreads = 256;

// ---------------------------------------------------------------------------
// embedding: h = norm(E[tok])
// ---------------------------------------------------------------------------
template <typename T, int EPT>
__global__ __launch_bounds__(kRowThreads) void k_embed(const int32_t* __restrict__ tok, const T* __restrict__ E,
                                                      float* __restrict__ h, float* __restrict__ h2,
                                                      T* __restrict__ xb, int d, int vocab, int* err) {
  __shared__ float sh[kRowThreads / 64];
  const int r = blockIdx.x;
  int t = tok[r];
  if (t < 0 || t >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    t = t < 0 ? 0 : vocab - 1;
  }
  const T* e = E + (size_t)t * d;
  float v[EPT];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    v[j] = i < d ? to_f(e[i]) : 0.f;
    ss += v[j] * v[j];
  }
  const float inv = inv_norm(block_sum_slot<kRowThreads>(ss, sh));  // first use of sh
  const size_t o = (size_t)r * d;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    if (i < d) {
      const float x = v[j] * inv;
      h[o + i] = x;
      xb[o + i] = from_f<T>(x);
      if (h2) h2[o + i] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// nGPT update: h = norm(h + alpha * (norm(y) - h))
// ---------------------------------------------------------------------------
template <typename T, int EPT>
__global__ __launch_bounds__(kRowThreads) void k_update(float* __restrict__ h, const float* __restrict__ y,
                                                       const float* __restrict__ alpha, T* __restrict__ xb,
                                                       float* __restrict__ h2, int d, RowGate gate,
                                                       const float* __restrict__ y1) {
  __shared__ float sh[2][kRowThreads / 64];  // one slot per sum: no barrier before either
  if (gate.loops && gate.loop > gate.loops[blockIdx.x / gate.n]) return;  // row past its loop count
  const size_t o = (size_t)blockIdx.x * d;
  float yv[EPT], hv[EPT];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    yv[j] = i < d ? y[o + i] : 0.f;
    if (y1 && i < d) yv[j] += y1[o + i];  // the two halves of a split product, in order
    hv[j] = i < d ? h[o + i] : 0.f;
    ss += yv[j] * yv[j];
  }
  const float iy = inv_norm(block_sum_slot<kRowThreads>(ss, sh[0]));
  float st = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    const float a = i < d ? alpha[i] : 0.f;
    hv[j] = hv[j] + a * (yv[j] * iy - hv[j]);
    st += hv[j] * hv[j];
  }
  const float ih = inv_norm(block_sum_slot<kRowThreads>(st, sh[1]));
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    if (i < d) {
      const float x = hv[j] * ih;
      h[o + i] = x;
      xb[o + i] = from_f<T>(x);
      if (h2) h2[o + i] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// loop re-injection: h = norm(wh * h + we * e)
// ---------------------------------------------------------------------------
template <typename T, int EPT>
__global__ __launch_bounds__(kRowThreads) void k_combine(float* __restrict__ h, const float* __restrict__ e,
                                                        float wh, float we, T* __restrict__ xb, int d,
                                                        RowGate gate) {
  __shared__ float sh[kRowThreads / 64];
  if (gate.loops && gate.loop > gate.loops[blockIdx.x / gate.n]) return;  // row past its loop count
  const size_t o = (size_t)blockIdx.x * d;
  float v[EPT];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    v[j] = i < d ? wh * h[o + i] + we * e[o + i] : 0.f;
    ss += v[j] * v[j];
  }
  const float inv = inv_norm(block_sum_slot<kRowThreads>(ss, sh));  // first use of sh
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = threadIdx.x + j * kRowThreads;
    if (i < d) {
      const float x = v[j] * inv;
      h[o + i] = x;
      xb[o + i] = from_f<T>(x);
    }
  }
}

template <template <typename, int> class K, typename T>
struct RowDispatch;

#define DORY_ROW_LAUNCH(KERNEL, T, d, rows, st, ...)                                                   \
  do {                                                                                                 \
    if ((d) <= 4 * kRowThreads)                                                                        \
      hipLaunchKernelGGL((KERNEL<T, 4>), dim3(rows), dim3(kRowThreads), 0, st, __VA_ARGS__);           \
    else if ((d) <= 8 * kRowThreads)                                                                   \
      hipLaunchKernelGGL((KERNEL<T, 8>), dim3(rows), dim3(kRowThreads), 0, st, __VA_ARGS__);           \
    else if ((d) <= 16 * kRowThreads)                                                                  \
      hipLaunchKernelGGL((KERNEL<T, 16>), dim3(rows), dim3(kRowThreads), 0, st, __VA_ARGS__);          \
    else                                                                                               \
      hipLaunchKernelGGL((KERNEL<T, 32>), dim3(rows), dim3(kRowThreads), 0, st, __VA_ARGS__);          \
  } while (0)

hipError_t launch_embed(int dtype, const int32_t* tok, const void* E, float* h, float* h2, void* xb, int rows,
                        int d, int vocab, int* err, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 0)
    DORY_ROW_LAUNCH(k_embed, float, d, rows, st, tok, (const float*)E, h, h2, (float*)xb, d, vocab, err);
  else
    DORY_ROW_LAUNCH(k_embed, bf16, d, rows, st, tok, (const bf16*)E, h, h2, (bf16*)xb, d, vocab, err);
  return hipGetLastError();
}

hipError_t launch_update(int dtype, float* h, const float* y, const float* alpha, void* xb, float* h2, int rows,
                         int d, hipStream_t st, RowGate gate, const float* y1) {
  if (rows <= 0) return hipSuccess;
  if (gate.loops && gate.n < 1) return hipErrorInvalidValue;
  if (dtype == 0)
    DORY_ROW_LAUNCH(k_update, float, d, rows, st, h, y, alpha, (float*)xb, h2, d, gate, y1);
  else
    DORY_ROW_LAUNCH(k_update, bf16, d, rows, st, h, y, alpha, (bf16*)xb, h2, d, gate, y1);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, float* h, const float* e, float wh, float we, void* xb, int rows, int d,
                          hipStream_t st, RowGate gate) {
  if (rows <= 0) return hipSuccess;
  if (gate.loops && gate.n < 1) return hipErrorInvalidValue;
  if (dtype == 0)
    DORY_ROW_LAUNCH(k_combine, float, d, rows, st, h, e, wh, we, (float*)xb, d, gate);
  else
    DORY_ROW_LAUNCH(k_combine, bf16, d, rows, st, h, e, wh, we, (bf16*)xb, d, gate);
  return hipGetLastError();
}

__global__ void k_set_rows(int* __restrict__ dst, RowLoops a) {
  if ((int)threadIdx.x < a.n) dst[threadIdx.x] = a.k[threadIdx.x];
}

hipError_t launch_set_rows(int* dst, const RowLoops& a, hipStream_t st) {
  if (a.n < 1 || a.n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_set_rows, dim3(1), dim3(64), 0, st, dst, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RoPE tables: angle = pos * base^(-2i/hd) in float64 (an fp32 product of a
// position near 262144 with theta loses ~1e-2 rad), stored as float (cos, sin)
// ---------------------------------------------------------------------------
__global__ void k_rope_table(float2* __restrict__ tab, int max_ctx, int hd, double base) {
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_ctx * half) return;
  const int pos = (int)(idx / half);
  const int i = (int)(idx % half);
  const double theta = pow(base, -2.0 * (double)i / (double)hd);
  const double ang = (double)pos * theta;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2* tab, int max_ctx, int hd, double base, hipStream_t st) {
  const int64_t n = (int64_t)max_ctx * (hd / 2);
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(k_rope_table, dim3(blocks), dim3(256), 0, st, tab, max_ctx, hd, base);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RoPE + per-head L2 norm of q and k. One wave per (head, kRopeRows
// consecutive rows); lane l owns the rotation pair (l, l + hd/2).
// ---------------------------------------------------------------------------
constexpr int kRopeRows = 4;  // rows (positions) per wave of k_rope_qk

template <typename T>
__global__ __launch_bounds__(256) void k_rope_qk(RopeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + wave;
  if (head >= a.nq + a.nkv) return;  // wave-uniform
  const int half = a.hd / 2;
  const int r0 = blockIdx.y * kRopeRows;
  // every row's loads first (rows past the end and lanes past half read a
  // clamped address and are masked below), so each lane keeps 3 x kRopeRows
  // loads in flight
  const int ln = min(lane, half - 1);
  float x1[kRopeRows], x2[kRopeRows];
  float2 cs[kRopeRows];
#pragma unroll
  for (int i = 0; i < kRopeRows; ++i) {
    const int r = min(r0 + i, a.rows - 1);
    const float* src = a.qkvg + (size_t)r * a.ld + (size_t)head * a.hd;
    x1[i] = src[ln];
    x2[i] = src[ln + half];
    cs[i] = a.tab[(size_t)(a.p0 + r % a.n) * half + ln];
  }
#pragma unroll
  for (int i = 0; i < kRopeRows; ++i) {
    const int r = r0 + i;
    if (r >= a.rows) break;  // wave-uniform
    const bool on = lane < half;
    const float r1 = on ? x1[i] * cs[i].x - x2[i] * cs[i].y : 0.f;
    const float r2 = on ? x2[i] * cs[i].x + x1[i] * cs[i].y : 0.f;
    // lanes past half add zeros: the same sums as a butterfly over the active lanes
    const float inv = inv_norm(wave_sum(r1 * r1 + r2 * r2));
    if (on) {
      T* dst = head < a.nq ? (T*)a.q_out + ((size_t)r * a.nq + head) * a.hd
                           : (T*)a.k_out + ((size_t)r * a.nkv + head - a.nq) * a.hd;
      dst[lane] = from_f<T>(r1 * inv);
      dst[lane + half] = from_f<T>(r2 * inv);
    }
  }
}

// The call's values transposed per kv head, [B][n_kv][hd][vld] with position
// i at column i (zeros from n to vld): a workgroup takes 64 positions of one
// kv head, reads them as rows through LDS and writes each dimension's run of
// positions contiguously.
constexpr int kVtPos = 64;

template <typename T>
__global__ __launch_bounds__(256) void k_v_transpose(RopeArgs a) {
  __shared__ float tile[kVtPos][129];
  const int i0 = blockIdx.x * kVtPos, kvh = blockIdx.y, b = blockIdx.z;
  const int hd = a.hd;  // <= 128
  const size_t col = (size_t)(a.nq + a.nkv + kvh) * hd;
  for (int e = threadIdx.x; e < kVtPos * hd; e += 256) {
    const int p = e / hd, d = e % hd, i = i0 + p;
    tile[p][d] = i < a.n ? a.qkvg[(size_t)(b * a.n + i) * a.ld + col + d] : 0.f;
  }
  __syncthreads();
  T* out = (T*)a.v_out + ((size_t)b * a.nkv + kvh) * hd * a.vld;
  for (int e = threadIdx.x; e < kVtPos * hd; e += 256) {
    const int d = e / kVtPos, p = e % kVtPos, i = i0 + p;
    if (i < a.vld) out[(size_t)d * a.vld + i] = from_f<T>(tile[p][d]);
  }
}

// Same transpose for head sizes 64 / 128 with 16-byte reads (4 dimensions of
// a position) and 4-position stores (one group of a dimension's run), no
// integer division by a runtime size: the generic kernel moved 2-4 bytes per
// instruction and divided by hd for every element.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_v_transpose4(RopeArgs a) {
  __shared__ float tile[kVtPos][HD + 1];
  constexpr int D4 = HD / 4, G = kVtPos / 4;
  const int i0 = blockIdx.x * kVtPos, kvh = blockIdx.y, b = blockIdx.z;
  const size_t col = (size_t)(a.nq + a.nkv + kvh) * HD;
  for (int e = threadIdx.x; e < kVtPos * D4; e += 256) {
    const int p = e / D4, d = 4 * (e % D4), i = i0 + p;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < a.n) v = *(const float4*)(a.qkvg + (size_t)(b * a.n + i) * a.ld + col + d);
    tile[p][d] = v.x;
    tile[p][d + 1] = v.y;
    tile[p][d + 2] = v.z;
    tile[p][d + 3] = v.w;
  }
  __syncthreads();
  T* out = (T*)a.v_out + ((size_t)b * a.nkv + kvh) * HD * a.vld;
  for (int e = threadIdx.x; e < HD * G; e += 256) {
    const int d = e / G, g = e % G, i = i0 + 4 * g;
    if (i >= a.vld) continue;  // vld % 4 == 0: a group is wholly inside or outside
    const float v0 = tile[4 * g][d], v1 = tile[4 * g + 1][d], v2 = tile[4 * g + 2][d], v3 = tile[4 * g + 3][d];
    if constexpr (sizeof(T) == 2) {
      *(uint2*)(out + (size_t)d * a.vld + i) =
          make_uint2((uint32_t)from_f<bf16>(v0) | ((uint32_t)from_f<bf16>(v1) << 16),
                     (uint32_t)from_f<bf16>(v2) | ((uint32_t)from_f<bf16>(v3) << 16));
    } else {
      *(float4*)(out + (size_t)d * a.vld + i) = make_float4(v0, v1, v2, v3);
    }
  }
}

template <typename T>
static void launch_v_transpose(const RopeArgs& a, dim3 vgrid, hipStream_t st) {
  const bool vec = a.ld % 4 == 0 && a.vld % 4 == 0 && ((uintptr_t)a.qkvg & 15) == 0 &&
                   ((uintptr_t)a.v_out & (sizeof(T) == 2 ? 7 : 15)) == 0;
  if (vec && a.hd == 128)
    hipLaunchKernelGGL((k_v_transpose4<T, 128>), vgrid, dim3(256), 0, st, a);
  else if (vec && a.hd == 64)
    hipLaunchKernelGGL((k_v_transpose4<T, 64>), vgrid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_v_transpose<T>, vgrid, dim3(256), 0, st, a);
}

hipError_t launch_rope_qk(int dtype, const RopeArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.hd > 128 || a.rows != a.B * a.n) return hipErrorInvalidValue;
  const dim3 grid((a.nq + a.nkv + 3) / 4, (a.rows + kRopeRows - 1) / kRopeRows);
  const dim3 vgrid((a.vld + kVtPos - 1) / kVtPos, a.nkv, a.B);
  if (dtype == 0) {
    hipLaunchKernelGGL(k_rope_qk<float>, grid, dim3(256), 0, st, a);
    launch_v_transpose<float>(a, vgrid, st);
  } else {
    hipLaunchKernelGGL(k_rope_qk<bf16>, grid, dim3(256), 0, st, a);
    launch_v_transpose<bf16>(a, vgrid, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV writer after a multi-position call (attention has already read the old
// ring contents): every position of a full layer, the last min(n, slots)
// positions of a sliding-window ring. A workgroup takes 32 consecutive
// positions of one (sequence, kv head): keys row by row, values as runs of
// positions (the call's V^T rows and the cache's 32-slot blocks both keep a
// dimension's positions contiguous), 16 bytes at a time where a run of 8
// positions lands on 8 consecutive slots of one block, else one by one.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_kv_write(const T* __restrict__ kw, const T* __restrict__ vw, int vld,
                                                 T* __restrict__ kc, T* __restrict__ vc, int n, int p0, int nkv,
                                                 int hd, int slots, int window, int is_full,
                                                 const int* __restrict__ wloops, int loop) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte vector
  const int i0 = blockIdx.x * 32, kvh = blockIdx.y, b = blockIdx.z;
  if (wloops && wloops[b] != loop) return;  // not this sequence's last pass
  const int i_first = is_full ? 0 : max(0, n - slots);  // earlier positions are overwritten later in this call
  auto slot_of = [&](int i) { return is_full ? p0 + i : (p0 + i) % window; };
  const size_t head = (size_t)b * nkv + kvh;
  // keys: 32 rows of hd, E elements per thread and step
  const int kv_per_row = hd / E;
  for (int e = threadIdx.x; e < 32 * kv_per_row; e += 256) {
    const int p = e / kv_per_row, c = e % kv_per_row, i = i0 + p;
    if (i < n && i >= i_first)
      *(u32x4*)(kc + (head * slots + slot_of(i)) * hd + c * E) =
          *(const u32x4*)(kw + ((size_t)(b * n + i) * nkv + kvh) * hd + c * E);
  }
  // values: per dimension, runs of E positions
  const T* vsrc = vw + head * hd * vld;
  T* vdst = vc + head * hd * vslots_of(slots);
  for (int e = threadIdx.x; e < hd * (32 / E); e += 256) {
    const int d = e / (32 / E), ia = i0 + E * (e % (32 / E));
    const int sa = slot_of(ia);
    const bool vec = ia >= i_first && ia + E <= n && (sa % E) == 0 && (sa % 32) + E <= 32 &&
                     slot_of(ia + E - 1) == sa + E - 1 && ((size_t)d * vld + ia) % E == 0;
    if (vec) {
      *(u32x4*)(vdst + vt_off(sa, d, hd)) = *(const u32x4*)(vsrc + (size_t)d * vld + ia);
    } else {
      for (int q = 0; q < E; ++q) {
        const int i = ia + q;
        if (i < n && i >= i_first) vdst[vt_off(slot_of(i), d, hd)] = vsrc[(size_t)d * vld + i];
      }
    }
  }
}

hipError_t launch_kv_write(int dtype, const void* kw, const void* vw, int vld, void* kc, void* vc, int B, int n,
                           int p0, int nkv, int hd, int slots, int window, int is_full, hipStream_t st,
                           const int* wloops, int loop) {
  if (B * n <= 0) return hipSuccess;
  if (hd % 8) return hipErrorInvalidValue;
  const dim3 grid((n + 31) / 32, nkv, B);
  if (dtype == 0)
    hipLaunchKernelGGL(k_kv_write<float>, grid, dim3(256), 0, st, (const float*)kw, (const float*)vw, vld,
                       (float*)kc, (float*)vc, n, p0, nkv, hd, slots, window, is_full, wloops, loop);
  else
    hipLaunchKernelGGL(k_kv_write<bf16>, grid, dim3(256), 0, st, (const bf16*)kw, (const bf16*)vw, vld,
                       (bf16*)kc, (bf16*)vc, n, p0, nkv, hd, slots, window, is_full, wloops, loop);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// greedy argmax, lowest index on ties, two passes
// ---------------------------------------------------------------------------
constexpr int kArgBlock = 1024;  // logits per partial (matches the plan)

__device__ __forceinline__ void arg_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__device__ __forceinline__ void block_argmax(float& bv, int& bi) {
  __shared__ float sv[4];
  __shared__ int si[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    arg_better(bv, bi, ov, oi);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  for (int k = 1; k < (int)(blockDim.x >> 6); ++k) arg_better(bv, bi, sv[k], si[k]);
}

__global__ __launch_bounds__(256) void k_argmax_part(const float* __restrict__ logits, int V, int nblk,
                                                    float2* __restrict__ part) {
  const int b = blockIdx.y, blk = blockIdx.x;
  const float* row = logits + (size_t)b * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const int lo = blk * kArgBlock;
  const int hi = min(V, lo + kArgBlock);
  for (int i = lo + threadIdx.x; i < hi; i += 256) arg_better(bv, bi, row[i], i);
  block_argmax(bv, bi);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blk] = make_float2(bv, __int_as_float(bi));
}

__global__ __launch_bounds__(256) void k_argmax_final(const float2* __restrict__ part, int nblk,
                                                     int32_t* __restrict__ out, int* __restrict__ pos_dev) {
  const int b = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int k = threadIdx.x; k < nblk; k += 256) {
    const float2 p = part[(size_t)b * nblk + k];
    arg_better(bv, bi, p.x, __float_as_int(p.y));
  }
  block_argmax(bv, bi);
  if (threadIdx.x == 0) out[b] = bi == 0x7fffffff ? 0 : bi;
  if (pos_dev && b == 0 && threadIdx.x == 0) pos_dev[0] += 1;  // this step's position is done
}

__global__ void k_set_pos(int* pos_dev, int value) { pos_dev[0] = value; }

hipError_t launch_set_pos(int* pos_dev, int value, hipStream_t st) {
  hipLaunchKernelGGL(k_set_pos, dim3(1), dim3(1), 0, st, pos_dev, value);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int B, int V, int32_t* out, void* scratch, hipStream_t st,
                         int* pos_dev) {
  if (B <= 0) return hipSuccess;
  const int nblk = (V + kArgBlock - 1) / kArgBlock;
  hipLaunchKernelGGL(k_argmax_part, dim3(nblk, B), dim3(256), 0, st, logits, V, nblk, (float2*)scratch);
  hipLaunchKernelGGL(k_argmax_final, dim3(B), dim3(256), 0, st, (const float2*)scratch, nblk, out, pos_dev);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// argmax with library-held partials (dory_op_argmax_noalloc): for callers
// that cannot allocate. The partials live in a fixed device array, one copy
// per GPU; its address on a device is looked up once, with that device
// current, and kept. Pass 1 writes every partial pass 2 reads, so nothing
// needs clearing between calls; calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float2 scratch[kArgmaxNoAllocPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float2* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t argmax_noalloc_scratch(float2** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float2*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dory

extern "C" dory_status dory_op_argmax_noalloc(const float* logits, int32_t B, int32_t V, int32_t* out,
                                              void* stream) {
  if (!logits || !out || B < 1 || V < 1) return DORY_E_ARG;
  const int64_t nblk = ((int64_t)V + dory::kArgBlock - 1) / dory::kArgBlock;
  if ((int64_t)B * nblk > dory::kArgmaxNoAllocPartials) return DORY_E_CAPACITY;
  float2* part = nullptr;
  if (dory::argmax_noalloc_scratch(&part) != hipSuccess) return DORY_E_HIP;
  const hipError_t e = dory::launch_argmax(logits, B, V, out, part, (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

namespace dory {

// ---------------------------------------------------------------------------
// clearing of 64-bit words (a kernel, so that recorded graphs hold no memset)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_zero_u64(unsigned long long* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0ull;
}

hipError_t launch_zero_u64(unsigned long long* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_u64, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU of a bfloat16 projection [M][2F] (u then v per row): a[M][F] =
// (scale u) silu(scale v), 8 outputs per thread (16-byte loads and stores).
// silu(v) = v / (1 + e^-v) with the hardware exp2 and reciprocal (each about
// 1 ulp; the precise expf and division had made the kernel VALU-bound): for
// v -> -inf e^-v overflows to inf and the reciprocal to 0, for v -> +inf the
// quotient tends to v, as it should.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_hw(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

__global__ __launch_bounds__(256) void k_swiglu_rows(const bf16* __restrict__ p, int F, float scale,
                                                     bf16* __restrict__ a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 8 outputs
  if (i >= n8) return;
  const int64_t e = i * 8, r = e / F, c = e % F;
  const u32x4 u = *(const u32x4*)(p + r * 2 * F + c);
  const u32x4 v = *(const u32x4*)(p + r * 2 * F + F + c);
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float u0 = bf_lo(u[k]) * scale, u1 = bf_hi(u[k]) * scale;
    const float v0 = bf_lo(v[k]) * scale, v1 = bf_hi(v[k]) * scale;
    o[k] = (uint32_t)from_f<bf16>(u0 * silu_hw(v0)) | ((uint32_t)from_f<bf16>(u1 * silu_hw(v1)) << 16);
  }
  *(u32x4*)(a + e) = o;
}

hipError_t launch_swiglu_rows(const void* p, int M, int F, float scale, void* a, hipStream_t st) {
  if (F % 8) return hipErrorInvalidValue;
  const int64_t n8 = (int64_t)M * F / 8;
  if (n8 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_rows, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, (const bf16*)p, F, scale,
                     (bf16*)a, n8);
  return hipGetLastError();
}

}  // namespace dory
