// Attention of the looped nGPT: softmax(scale * q.k) v over the allowed keys
// of a sliding-window (t - W < s <= t) or full (s <= t) layer, grouped-query
// heads, and the sigmoid output gate.
//
// k_attn_split is split-K flash decoding: one workgroup per (key split,
// batch row x kv head, query). It stages tiles of keys and values in LDS,
// scores them against all G query heads of the kv head at once (so each K/V
// byte is read once per group), keeps a running max / sum per head, and
// writes an unnormalised partial (m, l, acc). Keys at positions >= p0 (this
// call) come from the call's own K/V rows, earlier ones from the cache (ring
// slot pos mod W for sliding layers). k_attn_combine merges the partials with
// a log-sum-exp, applies the gate and stores the gated output.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace dory {

template <typename T, int HD, int G>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a) {
  constexpr int TK = sizeof(T) == 2 ? 64 : 32;   // keys per tile (LDS budget)
  constexpr int VEC = 16 / sizeof(T);
  constexpr int VPK = HD / VEC;                  // 16-byte vectors per key row
  constexpr int NPART = 256 / TK;                // threads per key in the score step
  constexpr int DP = HD / NPART;                 // dims per thread in the score step
  constexpr int KP = 256 / HD;                   // key partitions in the PV step
  constexpr int KPT = TK / KP;                   // keys per partition
  constexpr int KLD = HD + VEC;                  // padded K row

  __shared__ __align__(16) T Ks[TK * KLD];
  __shared__ __align__(16) T Vs[TK * HD];
  __shared__ float qs[G][HD];
  __shared__ float ps[G][TK];
  __shared__ float redm[4][G];
  __shared__ float reds[4][G];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int split = blockIdx.x;
  const int b = blockIdx.y / a.nkv, kvh = blockIdx.y % a.nkv;
  const int i = blockIdx.z;
  const int r = b * a.n + i;
  const int t = a.p0 + i;
  const int lo = a.is_full ? 0 : max(0, t - a.window + 1);
  const int L = t - lo + 1;
  int per = (L + a.n_split - 1) / a.n_split;
  per = (per + TK - 1) / TK * TK;
  const int s_lo = lo + split * per;
  const int s_hi = min(t + 1, s_lo + per);

  const T* q = (const T*)a.q;
  for (int e = tid; e < G * HD; e += 256) {
    const int g = e / HD, d = e % HD;
    qs[g][d] = to_f(q[((size_t)r * a.nq + kvh * G + g) * HD + d]);
  }

  const T* kw = (const T*)a.kw;
  const T* vw = (const T*)a.vw;
  const T* kc = (const T*)a.kc;
  const T* vc = (const T*)a.vc;

  float m[G], l[G], acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    acc[g] = 0.f;
  }
  const int key = tid / NPART, part = tid % NPART;
  const int pd = tid % HD, pk = tid / HD;

  for (int s0 = s_lo; s0 < s_hi; s0 += TK) {
    const int nk = min(TK, s_hi - s0);
    __syncthreads();  // previous tile fully consumed (and q staged on the first pass)
    for (int e = tid; e < TK * VPK; e += 256) {
      const int kk = e / VPK, c = e % VPK;
      uint4 kv4 = make_uint4(0, 0, 0, 0);
      const int s = s0 + kk;
      if (kk < nk) {
        if (s >= a.p0) {
          const size_t o = ((size_t)(b * a.n + (s - a.p0)) * a.nkv + kvh) * HD;
          kv4 = ((const uint4*)(kw + o))[c];
        } else {
          const int slot = a.is_full ? s : s % a.window;
          kv4 = ((const uint4*)(kc + (((size_t)b * a.nkv + kvh) * a.slots + slot) * HD))[c];
        }
      }
      *(uint4*)(Ks + kk * KLD + c * VEC) = kv4;
    }
    // values are stored transposed (blocks of [hd][32] in the cache, [hd][vld]
    // for this call): consecutive threads take consecutive keys of one dimension
    const size_t vhead = ((size_t)b * a.nkv + kvh) * HD * vslots_of(a.slots);
    const size_t vchunk = ((size_t)b * a.nkv + kvh) * HD * a.vld;
    for (int e = tid; e < TK * HD; e += 256) {
      const int d = e / TK, kk = e % TK;
      const int s = s0 + kk;
      T v = from_f<T>(0.f);
      if (kk < nk) {
        if (s < a.p0) {
          const int slot = a.is_full ? s : s % a.window;
          v = vc[vhead + vt_off(slot, d, HD)];
        } else {
          v = vw[vchunk + (size_t)d * a.vld + (s - a.p0)];
        }
      }
      Vs[kk * HD + d] = v;
    }
    __syncthreads();

    // scores of this thread's key for every head of the group
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dsum = 0.f;
#pragma unroll
      for (int d = 0; d < DP; ++d) dsum = fmaf(qs[g][part * DP + d], to_f(Ks[key * KLD + part * DP + d]), dsum);
      if constexpr (NPART > 1) dsum = xsum<1>(dsum);
      if constexpr (NPART > 2) dsum = xsum<2>(dsum);
      if constexpr (NPART > 4) dsum = xsum<4>(dsum);
      if constexpr (NPART > 8) dsum = xsum<8>(dsum);
      if constexpr (NPART > 16) dsum = xsum<16>(dsum);
      if constexpr (NPART > 32) dsum = xsum<32>(dsum);
      sc[g] = key < nk ? a.scale * dsum : -INFINITY;
    }
    // tile max per head
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float wm = wave_max(sc[g]);
      if (lane == 0) redm[wave][g] = wm;
    }
    __syncthreads();
    float mn[G], alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mt = fmaxf(fmaxf(redm[0][g], redm[1][g]), fmaxf(redm[2][g], redm[3][g]));
      mn[g] = fmaxf(m[g], mt);
      alpha[g] = (m[g] == -INFINITY) ? 0.f : expf(m[g] - mn[g]);
      const float p = key < nk ? expf(sc[g] - mn[g]) : 0.f;
      if (part == 0) ps[g][key] = p;
      const float wsum = wave_sum(part == 0 ? p : 0.f);
      if (lane == 0) reds[wave][g] = wsum;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] = l[g] * alpha[g] + ((reds[0][g] + reds[1][g]) + (reds[2][g] + reds[3][g]));
      m[g] = mn[g];
      acc[g] *= alpha[g];
    }
    // P.V for this thread's (dim, key partition)
#pragma unroll 4
    for (int kk = pk * KPT; kk < (pk + 1) * KPT; ++kk) {
      const float v = to_f(Vs[kk * HD + pd]);
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fmaf(ps[g][kk], v, acc[g]);
    }
  }

  // reduce the KP key partitions and write the partial
  __syncthreads();
  float* red = (float*)Ks;  // reuse: KP * G * HD floats fit in the K tile
  static_assert(KP * G * HD * 4 <= TK * KLD * (int)sizeof(T), "partition buffer");
#pragma unroll
  for (int g = 0; g < G; ++g) red[(pk * G + g) * HD + pd] = acc[g];
  __syncthreads();
  if (pk == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < KP; ++k) s += red[(k * G + g) * HD + pd];
      float* out = a.part + (((size_t)r * a.nq + kvh * G + g) * a.n_split + split) * (HD + 2);
      out[2 + pd] = s;
      if (pd == 0) {
        out[0] = m[g];
        out[1] = l[g];
      }
    }
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part, const float* __restrict__ qkvg,
                                                     int64_t ld, int gate_off, int gate, T* __restrict__ ob, int rows,
                                                     int nq, int n_split) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hq = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (hq >= nq) return;
  const float* p = part + ((size_t)r * nq + hq) * n_split * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, p[(size_t)s * (HD + 2)]);
  float L = 0.f;
  float o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float* ps = p + (size_t)s * (HD + 2);
    const float ms = ps[0];
    const float w = ms == -INFINITY ? 0.f : expf(ms - M);
    L = fmaf(ps[1], w, L);
    if (lane < HD) o0 = fmaf(ps[2 + lane], w, o0);
    if (lane + 64 < HD) o1 = fmaf(ps[2 + lane + 64], w, o1);
  }
  const float inv = 1.0f / L;
  const float* gr = qkvg + (size_t)r * ld + gate_off;
  T* dst = ob + ((size_t)r * nq + hq) * HD;
  if (lane < HD) {
    const float g = gate == 1 ? sigmoidf_(gr[hq * HD + lane]) : (gate == 2 ? sigmoidf_(gr[hq]) : 1.f);
    dst[lane] = from_f<T>(o0 * inv * g);
  }
  if (lane + 64 < HD) {
    const float g = gate == 1 ? sigmoidf_(gr[hq * HD + lane + 64]) : (gate == 2 ? sigmoidf_(gr[hq]) : 1.f);
    dst[lane + 64] = from_f<T>(o1 * inv * g);
  }
}

template <typename T, int HD>
static hipError_t attn_hd(const AttnArgs& a, hipStream_t st) {
  const int G = a.nq / a.nkv;
  dim3 grid(a.n_split, a.B * a.nkv, a.n);
  switch (G) {
    case 1: dory_launch((k_attn_split<T, HD, 1>), grid, dim3(256), 0, st, a); break;
    case 2: dory_launch((k_attn_split<T, HD, 2>), grid, dim3(256), 0, st, a); break;
    case 3: dory_launch((k_attn_split<T, HD, 3>), grid, dim3(256), 0, st, a); break;
    case 4: dory_launch((k_attn_split<T, HD, 4>), grid, dim3(256), 0, st, a); break;
    case 6: dory_launch((k_attn_split<T, HD, 6>), grid, dim3(256), 0, st, a); break;
    case 8: dory_launch((k_attn_split<T, HD, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_split(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.B * a.n <= 0) return hipSuccess;
  if (dtype == 0) {
    if (a.hd == 64) return attn_hd<float, 64>(a, st);
    if (a.hd == 128) return attn_hd<float, 128>(a, st);
  } else {
    if (a.hd == 64) return attn_hd<bf16, 64>(a, st);
    if (a.hd == 128) return attn_hd<bf16, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(int dtype, const float* part, const float* qkvg, int64_t ld, int gate_off, int gate,
                               void* ob, int rows, int nq, int hd, int n_split, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((nq + 3) / 4, rows);
#define DORY_CMB(T, HDV)                                                                                   \
  dory_launch((k_attn_combine<T, HDV>), grid, dim3(256), 0, st, part, qkvg, ld, gate_off, gate, (T*)ob, \
                     rows, nq, n_split)
  if (dtype == 0) {
    if (hd == 64) DORY_CMB(float, 64); else if (hd == 128) DORY_CMB(float, 128); else return hipErrorInvalidValue;
  } else {
    if (hd == 64) DORY_CMB(bf16, 64); else if (hd == 128) DORY_CMB(bf16, 128); else return hipErrorInvalidValue;
  }
#undef DORY_CMB
  return hipGetLastError();
}

}  // namespace dory

namespace dory {

// ---------------------------------------------------------------------------
// Fused decode attention. Each wave streams its own keys (8 keys per step,
// 8 lanes per key) with its own running max / sum, so the key loop has no
// workgroup barrier; the four waves are merged once at the end through LDS.
// Load order matters because vector loads complete in issue order: the few
// projection values that q and the new key need (L2-resident) are requested
// first, then the cache rows of the wave's first U steps (HBM), and RoPE /
// normalisation run while the cache rows are in flight. Lane `sub` of a key
// holds 16-byte chunks sub, sub + 8, ... of the row, so every load
// instruction reads 128 contiguous bytes per key.
// ---------------------------------------------------------------------------
template <typename T, int HD, int G>
__global__ __launch_bounds__(256) void k_attn_decode(AttnDecArgs a) {
  constexpr int KG = 8;              // keys per wave step
  constexpr int LPK = 8;             // lanes per key
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = HD / (LPK * VEC);  // 16-byte chunks per lane per key row
  constexpr int DPL = NV * VEC;         // dims per lane
  constexpr int U = 4;               // key steps whose loads are in flight together
  constexpr int NI = (G + 2 + 3) / 4;  // setup items per wave (q heads, new key, new value)
  constexpr float LOG2E = 1.4426950408889634f;

  __shared__ float qs[G][HD];
  __shared__ __align__(16) T selfk[HD];
  __shared__ __align__(16) T selfv[HD];
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wacc[4][G][HD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int split = blockIdx.x;
  const int b = blockIdx.y / a.nkv, kvh = blockIdx.y % a.nkv;
  const int t = *a.t_dev;  // position of the new key (device counter: graph-replayable)
  const int lo = a.is_full ? 0 : max(0, t - a.window + 1);
  const int L = t - lo + 1;
  int per = (L + a.n_split - 1) / a.n_split;
  per = (per + 4 * KG - 1) / (4 * KG) * (4 * KG);
  const int s_lo = lo + split * per;
  const int s_hi = min(t + 1, s_lo + per);
  const bool has_self = s_lo <= t && t < s_hi;
  const int half = HD / 2;

  // (1) projection values for q heads / new key / new value (L2). Loads are
  // unconditional from clamped addresses (straight-line code keeps the
  // wait counts exact); unused values are never stored.
  const float* row = a.qkvg + (size_t)b * a.ld;
  const int ln = min(lane, half - 1);
  float x1[NI], x2[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = min(wave + 4 * it, G + 1);
    const float* src = item < G ? row + (size_t)(kvh * G + item) * HD
                                : row + (size_t)a.nq * HD + (size_t)(item - G) * a.nkv * HD + (size_t)kvh * HD;
    x1[it] = src[ln];
    x2[it] = src[ln + half];
  }
  const float2 cs = a.tab[(size_t)t * half + ln];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the cache stream

  // (2) cache rows of the first U steps (HBM); out-of-range keys and the new
  // position load a valid slot and are masked when used
  const int kg = lane / LPK, sub = lane % LPK;
  const T* kc = (const T*)a.kc;
  const T* vc = (const T*)a.vc;
  const size_t head_base = ((size_t)b * a.nkv + kvh) * a.slots;
  u32x4 kv[U][NV], vv[U][NV];
  const T* vt = vc + ((size_t)b * a.nkv + kvh) * vslots_of(a.slots) * HD;  // this head's values (32-position blocks)
  auto issue = [&](int base0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base0 + u * 4 * KG + kg;
      const int sl = (s < s_hi && s != t) ? s : lo;
      const int slot = a.is_full ? sl : sl % a.window;
      const size_t o = (head_base + slot) * HD + sub * VEC;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        kv[u][i] = *(const u32x4*)(kc + o + i * LPK * VEC);
        T tmp[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) tmp[j] = vt[vt_off(slot, (i * LPK + sub) * VEC + j, HD)];
        vv[u][i] = *(const u32x4*)tmp;
      }
    }
  };
  const int first = s_lo + wave * KG;
  issue(first);

  // (3) RoPE at t, unit norm, storage rounding; q pre-scaled for exp2
  const float qscale = a.scale * LOG2E;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = wave + 4 * it;
    const float y1 = lane < half ? x1[it] : 0.f, y2 = lane < half ? x2[it] : 0.f;
    const float r1 = y1 * cs.x - y2 * cs.y;
    const float r2 = y2 * cs.x + y1 * cs.y;
    const float inv = inv_norm(wave_sum(r1 * r1 + r2 * r2));
    const bool rot = item <= G;  // q heads and the new key; the value is copied
    const T z1 = from_f<T>(rot ? r1 * inv : y1), z2 = from_f<T>(rot ? r2 * inv : y2);
    if (lane < half && item < G + 2) {
      if (item < G) {
        qs[item][lane] = to_f(z1) * qscale;
        qs[item][lane + half] = to_f(z2) * qscale;
      } else if (has_self) {
        T* dst = item == G ? selfk : selfv;
        dst[lane] = z1;
        dst[lane + half] = z2;
      }
    }
  }
  __syncthreads();
  if (has_self && a.write_kv && (!a.wloops || a.wloops[b] == a.loop) && tid < HD) {
    // the slot of t held t - W (outside every window of this call) or nothing
    const int slot = a.is_full ? t : t % a.window;
    ((T*)a.kc)[(head_base + slot) * HD + tid] = selfk[tid];
    ((T*)a.vc)[((size_t)b * a.nkv + kvh) * vslots_of(a.slots) * HD + vt_off(slot, tid, HD)] = selfv[tid];
  }

  // this lane's dims: chunks sub, sub + 8, ... of VEC elements
  float qr[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < VEC; ++j) qr[g][i * VEC + j] = qs[g][(i * LPK + sub) * VEC + j];

  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[g][i] = 0.f;
  }

  for (int base0 = first; base0 < s_hi; base0 += 4 * KG * U) {
    if (base0 != first) issue(base0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = base0 + u * 4 * KG;
      if (base >= s_hi) break;  // wave-uniform
      const int s = base + kg;
      const bool valid = s < s_hi;
      if (valid && s == t) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          kv[u][i] = *(const u32x4*)(selfk + (i * LPK + sub) * VEC);
          vv[u][i] = *(const u32x4*)(selfv + (i * LPK + sub) * VEC);
        }
      }
      float kf[DPL], vf[DPL];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (!valid) vv[u][i] = u32x4{0, 0, 0, 0};  // masked keys: p = 0 must not meet NaN
        const uint32_t* kw = (const uint32_t*)&kv[u][i];
        const uint32_t* vw = (const uint32_t*)&vv[u][i];
        if (sizeof(T) == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kf[i * 8 + 2 * j] = bf_lo(kw[j]);
            kf[i * 8 + 2 * j + 1] = bf_hi(kw[j]);
            vf[i * 8 + 2 * j] = bf_lo(vw[j]);
            vf[i * 8 + 2 * j + 1] = bf_hi(vw[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kf[i * 4 + j] = __uint_as_float(kw[j]);
            vf[i * 4 + j] = __uint_as_float(vw[j]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) d = fmaf(qr[g][i], kf[i], d);
        d = xsum<4>(xsum<2>(xsum<1>(d)));
        const float sc = valid ? d : -INFINITY;
        const float mt = xmax<32>(xmax<16>(xmax<8>(sc)));
        const float mn = fmaxf(m[g], mt);
        const float alpha = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mn);
        const float p = valid ? exp2f(sc - mn) : 0.f;
        const float ps = xsum<32>(xsum<16>(xsum<8>(p)));
        l[g] = l[g] * alpha + ps;
        m[g] = mn;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[g][i] = fmaf(p, vf[i], acc[g][i] * alpha);
      }
    }
  }

  // sum the 8 key groups of the wave (same running max across the wave)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float v = acc[g][i];
      acc[g][i] = xsum<32>(xsum<16>(xsum<8>(v)));
    }
  if (kg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < VEC; ++j) wacc[wave][g][(i * LPK + sub) * VEC + j] = acc[g][i * VEC + j];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      wm[wave][g] = m[g];
      wl[wave][g] = l[g];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * HD; e += 256) {
    const int g = e / HD, d = e % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float Ls = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (wm[w][g] == -INFINITY) continue;
        const float f = exp2f(wm[w][g] - M);
        Ls = fmaf(wl[w][g], f, Ls);
        A = fmaf(wacc[w][g][d], f, A);
      }
    }
    float* out = a.part + (((size_t)b * a.nq + kvh * G + g) * a.n_split + split) * (HD + 2);
    out[2 + d] = A;
    if (d == 0) {
      out[0] = M;
      out[1] = Ls;
    }
  }

}

// ---------------------------------------------------------------------------
// Decode attention on the matrix cores (bfloat16). Keys are taken in tiles of
// 32 positions; per tile a wave computes the scores as S^T = K . Q^T with
// v_mfma_f32_16x16x32_bf16 (rows = 16 keys, columns = the G query heads padded
// to 16, depth = head dims), so lane l ends up with the scores of head l%16
// for keys 4*(l/16)+i of each 16-key half. Those probabilities are exactly
// the B operand of O^T = V^T . P^T once the 32 keys are taken in the order
// {4g..4g+3, 16+4g..16+4g+3} for lane group g, so the P.V product needs no
// shuffles: the A operand reads the transposed cache values V^T[dim][keys]
// (two 8-byte runs per lane, inside one 32-position block of the value cache). Online softmax runs per head column; the only
// cross-lane steps are the 4-group max and sum (xor 16, 32).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// llrint(S * 2^e) in float32 and integer arithmetic (S * 2^e is exact in
// float32 here, so rounding it to the nearest integer, ties to even, then
// splitting off the high 32 bits gives the float64 route's result bit for bit)
__device__ __forceinline__ long long fixed_point(float S, int e) {
  const float r = rintf(ldexpf(S, e));
  const float mag = fabsf(r);
  const float hi = floorf(mag * 0x1p-32f);
  const float lo = mag - hi * 0x1p32f;  // exact: < 2^32, at most 24 significant bits
  const unsigned long long u = ((unsigned long long)(unsigned)hi << 32) | (unsigned long long)(unsigned)lo;
  return r < 0.f ? -(long long)u : (long long)u;
}

template <int HD, int G, bool FULL>
__global__ __launch_bounds__(256) void k_attn_decode_mfma(AttnDecArgs a) {
  constexpr int NKK = HD / 32;        // depth steps of the score product
  constexpr int NDD = HD / 16;        // 16-dim blocks of the output
  constexpr int NI = (G + 2 + 3) / 4;  // setup items per wave (q heads, new key, new value)
  constexpr float LOG2E = 1.4426950408889634f;

  __shared__ __align__(16) bf16 qs[16][HD];
  __shared__ __align__(16) bf16 selfk[HD];
  __shared__ __align__(16) bf16 selfv[HD];
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wacc[4][G][HD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int b = blockIdx.y / a.nkv, kvh = blockIdx.y % a.nkv;
  const int half = HD / 2;

  // (0) position of the new key: passed by value on eager calls; recorded
  // graphs read the device counter (every argument step-invariant)
  int t;
  if (a.t_now >= 0) {
    t = a.t_now;
  } else {
    const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc((void*)a.t_dev, (short)0, 4, 0x00020000);
    t = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(trs, 0, 0, 0));
  }

  // (1) projection values for q heads / new key / new value (L2), clamped and
  // unconditional so the waits stay exact; they do not depend on the position
  const float* row = a.qkvg + (size_t)b * a.ld;
  const int ln = min(lane, half - 1);
  float x1[NI], x2[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = min(wave + 4 * it, G + 1);
    const float* src = item < G ? row + (size_t)(kvh * G + item) * HD
                                : row + (size_t)a.nq * HD + (size_t)(item - G) * a.nkv * HD + (size_t)kvh * HD;
    x1[it] = src[ln];
    x2[it] = src[ln + half];
  }
  // gate values of this thread's entries of the sums (without a gate the
  // unused index points into q)
  constexpr int NE = (G * (HD + 1) + 255) / 256;
  float gx[NE];
  {
    const float* gp = a.gate ? row + a.gate_off : row;
#pragma unroll
    for (int it = 0; it < NE; ++it) {
      const int e = min(tid + 256 * it, G * (HD + 1) - 1);
      const int hq = kvh * G + e / (HD + 1), d = min(e % (HD + 1), HD - 1);
      gx[it] = gp[a.gate == 2 ? hq : hq * HD + d];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these small loads ahead of the cache stream

  // (2) cache operands. Tiles of 32 slots. Sliding layers (a ring of
  // `slots` slots, slot = pos mod window) walk the ring by slot, so a split's
  // tiles are fixed and their loads go out before the position is known;
  // which position a slot holds (and whether it is in the window) is worked
  // out afterwards. Full layers spread the tiles of positions 0..t over the
  // splits.
  const bf16* kc = (const bf16*)a.kc;
  const bf16* vt = (const bf16*)a.vc + ((size_t)b * a.nkv + kvh) * HD * vslots_of(a.slots);
  const size_t khead = ((size_t)b * a.nkv + kvh) * a.slots;
  // Key order inside a tile: A row r of 16-key half kb holds key 8 (r / 4) +
  // 4 kb + r % 4, so the score lane (head, g4) ends up with keys 8 g4 .. 8 g4
  // + 7 (half 0: +0..3, half 1: +4..7) — the k order of the P.V product,
  // whose V^T operand is then one 16-byte run of 8 slots.
  auto loadK = [&](int T, int smax, u32x4 (&ka)[2][NKK]) {
    const int s0t = T << 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int sl = min(s0t + 8 * (c16 >> 2) + 4 * kb + (c16 & 3), smax);  // past smax: masked later
      const bf16* kr = kc + (khead + sl) * HD + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) ka[kb][kk] = *(const u32x4*)(kr + kk * 32);
    }
  };
  // 8 consecutive slots, 8-aligned (slot and window counts are multiples of
  // 8), clamped in bounds
  auto loadV = [&](int T, u32x4 (&va)[NDD]) {
    const int s0 = min((T << 5) + 8 * g4, a.slots - 8);
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) va[dd] = *(const u32x4*)(vt + vt_off(s0, 16 * dd + c16, HD));
  };
  // rotation row at t, issued before the cache stream so that waiting for it
  // does not wait for the stream (vector loads return in order)
  const float2 cs = a.tab[(size_t)t * half + ln];
  __builtin_amdgcn_sched_barrier(0);
  int tb, te;
  if (!FULL) {
    const int ntiles = vslots_of(a.slots) >> 5;
    const int tps = (ntiles + a.n_split - 1) / a.n_split;
    tb = split * tps;
    te = min(ntiles, tb + tps);
  } else {
    const int ntiles = (t >> 5) + 1;
    const int tps = (ntiles + a.n_split - 1) / a.n_split;
    tb = split * tps;
    te = min(ntiles, tb + tps);
  }
  // issued unconditionally (a tile past te is clamped in bounds and never
  // processed): loads under a branch make the compiler wait for all of them
  // where the paths join
  const int smax = FULL ? t : a.slots - 1;
  const int T0 = FULL ? tb + wave : min(tb + wave, (vslots_of(a.slots) >> 5) - 1);
  u32x4 ka0[2][NKK];
  u32x4 va0[NDD];
  loadK(T0, smax, ka0);
  loadV(T0, va0);
  // position -> slot; ring: slot s holds position base + s (s <= tm) or
  // base + s - window (s > tm), base = t - tm, tm = t mod window
  const int tm = FULL ? t : t % a.window;
  const int base = t - tm;
  const int lo = FULL ? 0 : max(0, t - a.window + 1);
  const int tself = tm >> 5;  // tile holding the new key (by slot)
  const bool has_self = tb <= tself && tself < te;

  // (3) RoPE at t, unit norm, bfloat16 storage of q and of the new key/value
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = wave + 4 * it;
    const float y1 = lane < half ? x1[it] : 0.f, y2 = lane < half ? x2[it] : 0.f;
    const float r1 = y1 * cs.x - y2 * cs.y;
    const float r2 = y2 * cs.x + y1 * cs.y;
    const float inv = inv_norm(wave_sum(r1 * r1 + r2 * r2));
    const bool rot = item <= G;
    const bf16 z1 = from_f<bf16>(rot ? r1 * inv : y1), z2 = from_f<bf16>(rot ? r2 * inv : y2);
    if (lane < half && item < G + 2) {
      if (item < G) {
        qs[item][lane] = z1;
        qs[item][lane + half] = z2;
      } else if (has_self) {
        bf16* dst = item == G ? selfk : selfv;
        dst[lane] = z1;
        dst[lane + half] = z2;
      }
    }
  }
  for (int e = tid; e < (16 - G) * HD; e += 256) qs[G + e / HD][e % HD] = 0;  // padded head columns
  __syncthreads();
  // The new key and value go to the cache at the end of the kernel (nothing
  // in it reads that slot from memory): stores count in the same wait counter
  // as loads, so stores issued here would hold up every later wait for a tile.
  auto write_self = [&]() {
    if (has_self && a.write_kv && (!a.wloops || a.wloops[b] == a.loop) && tid < HD) {
      // the slot of t held t - window (outside every window of this call) or nothing
      ((bf16*)a.kc)[(khead + tm) * HD + tid] = selfk[tid];
      ((bf16*)a.vc)[((size_t)b * a.nkv + kvh) * HD * vslots_of(a.slots) + vt_off(tm, tid, HD)] = selfv[tid];
    }
  };

  bf16x8_t qb[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qb[kk] = *(const bf16x8_t*)&qs[c16][kk * 32 + 8 * g4];
  // the output gate's sigmoid, while the tiles are still arriving
  if (a.acc && a.gate) {
#pragma unroll
    for (int it = 0; it < NE; ++it) gx[it] = sigmoidf_(gx[it]);
  }

  // q and k are unit vectors, so no score exceeds the scale: while
  // sl2 = scale log2(e) is at most 40 the exponents are referenced to that
  // bound (no running max or rescale; 2^(-2 sl2) is still a normal float),
  // above it to a running max.
  const float sl2 = a.scale * LOG2E;
  const bool fixed_ref = sl2 <= 40.f;
  float m = fixed_ref ? sl2 : -INFINITY, l = 0.f;
  f32x4_t acc[NDD];
#pragma unroll
  for (int dd = 0; dd < NDD; ++dd) acc[dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // position held by slot s (ring) or slot = position (full); valid: in the
  // window and written
  auto pos_of = [&](int s) { return FULL ? s : (s <= tm ? base + s : base + s - a.window); };
  auto process = [&](int T, u32x4 (&ka)[2][NKK], u32x4 (&va)[NDD]) {
    const int s0t = T << 5;
    // wave-uniform: the tile needs masks (slots outside the window, past the
    // written ones or past the ring) or holds the new key
    const bool edge = FULL ? s0t + 31 >= t : (T == tself || t < a.window - 1 || s0t + 32 > a.slots);
    if (edge) {
      // branch-free: the new key's operands from LDS, selected per lane
      u32x4 sk[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) sk[kk] = *(const u32x4*)&selfk[kk * 32 + 8 * g4];
      uint32_t sv[NDD];
#pragma unroll
      for (int dd = 0; dd < NDD; ++dd) sv[dd] = (uint32_t)selfv[16 * dd + c16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool me = s0t + 8 * (c16 >> 2) + 4 * kb + (c16 & 3) == tm;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int q = 0; q < 4; ++q) ka[kb][kk][q] = me ? sk[kk][q] : ka[kb][kk][q];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = s0t + 8 * g4 + j;
        const int p = pos_of(s);
        const bool valid = s < a.slots && p >= lo && p <= t;
        const bool me = s == tm;
        const uint32_t sh = (j & 1) * 16;
#pragma unroll
        for (int dd = 0; dd < NDD; ++dd) {
          const uint32_t w = va[dd][j >> 1];
          const uint32_t v = me ? sv[dd] : (valid ? (w >> sh) & 0xffffu : 0u);
          va[dd][j >> 1] = (w & ~(0xffffu << sh)) | (v << sh);
        }
      }
    }
    // scores S^T[key][head] for both 16-key halves
    f32x4_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(bf16x8_t*)&ka[kb][kk], qb[kk], sc[kb], 0, 0, 0);
    }
    float v8[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0t + 8 * g4 + 4 * kb + i;
        bool valid = true;
        if (edge) {
          const int p = pos_of(s);
          valid = s < a.slots && p >= lo && p <= t;
        }
        const float v = valid ? sc[kb][i] * sl2 : -INFINITY;
        v8[kb * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    float mn = m, alpha = 1.f;
    if (!fixed_ref) {
      tmax = xmax<32>(xmax<16>(tmax));
      mn = fmaxf(m, tmax);
      alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
    }
    float ps = 0.f;
    bf16x8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // arguments >= -2 sl2 >= -80: the raw v_exp_f32 is exact enough
      const float p = v8[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v8[j] - mn);
      ps += p;
      pb[j] = (__bf16)p;
    }
    l = l * alpha + ps;  // this lane's keys; summed over the key groups after the loop
    m = mn;
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) {
      if (!fixed_ref) acc[dd] *= alpha;
      acc[dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)&va[dd], pb, acc[dd], 0, 0, 0);
    }
  };

  const int first = tb + wave;
  for (int T = first; T < te; T += 4) {
    if (T != first) {
      loadK(T, smax, ka0);
      loadV(T, va0);
    }
    process(T, ka0, va0);
  }

  l = xsum<32>(xsum<16>(l));  // the four key groups (g4) of head c16
  // this wave's result: head c16, dims 16*dd + 4*g4 + i
  if (c16 < G) {
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd)
#pragma unroll
      for (int i = 0; i < 4; ++i) wacc[wave][c16][16 * dd + 4 * g4 + i] = acc[dd][i];
    if (g4 == 0) {
      wm[wave][c16] = m;
      wl[wave][c16] = l;
    }
  }
  __syncthreads();
  if (a.acc) {
    // sums referenced to the largest possible score sl2 (unit q and k), the
    // value sums gated (linear in the sums), then fixed point in the bin that
    // this workgroup's sum p of the head selects; integer adds are
    // order-independent
    // per head, once: each wave's factor to the bound, the workgroup's sum p
    // L and its bin (L in [2^ex, 2^(ex+1)), normal: L >= 2^(-2 sl2) > 2^-126;
    // bin b keeps L 2^(16b) in [2^-15, 2))
    __shared__ float fw[4][16];
    __shared__ int binh[16];
    if (tid < G) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = wm[w][tid] == -INFINITY ? 0.f : exp2f(wm[w][tid] - sl2);
        fw[w][tid] = f;
        L = fmaf(wl[w][tid], f, L);
      }
      const int ex = (int)((__float_as_uint(L) >> 23) & 0xff) - 127;
      binh[tid] = ex < 0 ? min(-ex / kAttnAccBinBits, a.acc_nb - 1) : 0;
    }
    __syncthreads();
    const int stride = attn_acc_stride(HD, a.acc_nb);
#pragma unroll
    for (int it = 0; it < NE; ++it) {
      const int e = tid + 256 * it;
      if (e >= G * (HD + 1)) break;
      const int g = e / (HD + 1), d = e % (HD + 1);
      const int hq = kvh * G + g;
      float S = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) S = fmaf(d < HD ? wacc[w][g][d] : wl[w][g], fw[w][g], S);
      if (d < HD && a.gate) S *= gx[it];  // the sigmoid, taken during the set-up
      if (S == 0.f) continue;
      const int bin = binh[g];
      unsigned long long* ap = a.acc + ((size_t)b * a.nq + hq) * stride;
      atomicAdd(d < HD ? ap + bin * HD + d : ap + a.acc_nb * HD + bin,
                (unsigned long long)fixed_point(S, 36 + kAttnAccBinBits * bin));
    }
    write_self();
    return;
  }
  for (int e = tid; e < G * HD; e += 256) {
    const int g = e / HD, d = e % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float Ls = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (wm[w][g] == -INFINITY) continue;
        const float f = exp2f(wm[w][g] - M);
        Ls = fmaf(wl[w][g], f, Ls);
        A = fmaf(wacc[w][g][d], f, A);
      }
    }
    float* out = a.part + (((size_t)b * a.nq + kvh * G + g) * a.n_split + split) * (HD + 2);
    out[2 + d] = A;
    if (d == 0) {
      out[0] = M;
      out[1] = Ls;
    }
  }
  write_self();
}

// One workgroup of 512 threads per (q head, row): thread (d, group) takes
// dimension d of the splits group, group + NSG, ...; every load is issued at
// once from a clamped address (one round of L2 latency), the first wave
// turns the split maxima into weights meanwhile, and the groups are summed
// through LDS.
constexpr int kMergeThreads = 512;
constexpr int kMergeMaxSplits = 64;

template <typename T, int HD>
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge(const float* __restrict__ part,
                                                             const float* __restrict__ qkvg, int64_t ld, int gate_off,
                                                             int gate, T* __restrict__ ob, int nq, int n_split) {
  constexpr int NSG = kMergeThreads / HD;        // split groups
  constexpr int PER = kMergeMaxSplits / NSG;     // splits per group at most
  __shared__ float wsh[kMergeMaxSplits];
  __shared__ float lsh;
  __shared__ float red[NSG][HD];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = tid % HD, sg = tid / HD;
  const float* p = part + ((size_t)b * nq + hq) * n_split * (HD + 2);
  const int last = n_split - 1;
  // split maxima and sums first (they gate the weights), then the values
  float ms = 0.f, ls = 0.f;
  if (tid < kMergeMaxSplits) {
    const float* ps = p + (size_t)min(tid, last) * (HD + 2);
    ms = ps[0];
    ls = ps[1];
  }
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = p[(size_t)min(sg + NSG * i, last) * (HD + 2) + 2 + d];
  const float* gr = qkvg + (size_t)b * ld + gate_off;
  const float gx = gate == 1 ? gr[hq * HD + d] : (gate == 2 ? gr[hq] : 0.f);
  if (tid < kMergeMaxSplits) {  // wave 0: weights exp2(m_s - M), total sum
    const bool ok = tid < n_split && ms != -INFINITY;
    const float M = wave_max(ok ? ms : -INFINITY);
    const float w = ok ? exp2f(ms - M) : 0.f;
    wsh[tid] = w;
    const float L = wave_sum(ok ? ls * w : 0.f);
    if (tid == 0) lsh = L;
  }
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sp = sg + NSG * i;
    o = fmaf(v[i], sp < n_split ? wsh[sp] : 0.f, o);
  }
  red[sg][d] = o;
  __syncthreads();
  if (sg == 0) {
#pragma unroll
    for (int k = 1; k < NSG; ++k) o += red[k][d];
    const float g = gate == 0 ? 1.f : sigmoidf_(gx);
    ob[((size_t)b * nq + hq) * HD + d] = from_f<T>(o / lsh * g);
  }
}

template <typename T, int HD>
static hipError_t attn_dec_hd(const AttnDecArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.B * a.nkv);
  switch (a.nq / a.nkv) {
    case 1: dory_launch((k_attn_decode<T, HD, 1>), grid, dim3(256), 0, st, a); break;
    case 2: dory_launch((k_attn_decode<T, HD, 2>), grid, dim3(256), 0, st, a); break;
    case 3: dory_launch((k_attn_decode<T, HD, 3>), grid, dim3(256), 0, st, a); break;
    case 4: dory_launch((k_attn_decode<T, HD, 4>), grid, dim3(256), 0, st, a); break;
    case 6: dory_launch((k_attn_decode<T, HD, 6>), grid, dim3(256), 0, st, a); break;
    case 8: dory_launch((k_attn_decode<T, HD, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD, bool FULL>
static hipError_t attn_dec_mfma_f(const AttnDecArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.B * a.nkv);
  switch (a.nq / a.nkv) {
    case 1: dory_launch((k_attn_decode_mfma<HD, 1, FULL>), grid, dim3(256), 0, st, a); break;
    case 2: dory_launch((k_attn_decode_mfma<HD, 2, FULL>), grid, dim3(256), 0, st, a); break;
    case 3: dory_launch((k_attn_decode_mfma<HD, 3, FULL>), grid, dim3(256), 0, st, a); break;
    case 4: dory_launch((k_attn_decode_mfma<HD, 4, FULL>), grid, dim3(256), 0, st, a); break;
    case 6: dory_launch((k_attn_decode_mfma<HD, 6, FULL>), grid, dim3(256), 0, st, a); break;
    case 8: dory_launch((k_attn_decode_mfma<HD, 8, FULL>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
static hipError_t attn_dec_mfma(const AttnDecArgs& a, hipStream_t st) {
  return a.is_full ? attn_dec_mfma_f<HD, true>(a, st) : attn_dec_mfma_f<HD, false>(a, st);
}

bool attn_decode_uses_mfma(int dtype, int hd, int slots, int window, int is_full) {
  // 8-position runs of V^T must be contiguous and 16-byte aligned
  return dtype == 1 && (hd == 64 || hd == 128) && slots % 8 == 0 && slots >= 8 && (is_full || window % 8 == 0);
}

int attn_acc_bins(float scale) {
  const double sl2 = (double)scale * 1.4426950408889634;
  if (!(sl2 > 0.0)) return 0;
  const double nb = std::floor(2.0 * sl2 / kAttnAccBinBits) + 1.0;  // -log2(sum p) <= 2 sl2 < 16 nb
  return nb <= kAttnAccBinsMax ? (int)nb : 0;
}

hipError_t launch_attn_decode(int dtype, const AttnDecArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  const bool mfma = attn_decode_uses_mfma(dtype, a.hd, a.slots, a.window, a.is_full);
  // accumulators only from the matrix-core kernel, with enough bins for the scale
  if (a.acc && (!mfma || a.acc_nb < attn_acc_bins(a.scale) || a.acc_nb < 1 || a.acc_nb > kAttnAccBinsMax))
    return hipErrorInvalidValue;
  if (mfma)
    return a.hd == 64 ? attn_dec_mfma<64>(a, st) : attn_dec_mfma<128>(a, st);
  if (dtype == 0) {
    if (a.hd == 64) return attn_dec_hd<float, 64>(a, st);
    if (a.hd == 128) return attn_dec_hd<float, 128>(a, st);
  } else {
    if (a.hd == 64) return attn_dec_hd<bf16, 64>(a, st);
    if (a.hd == 128) return attn_dec_hd<bf16, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(int dtype, const float* part, const float* qkvg, int64_t ld, int gate_off, int gate,
                             void* ob, int B, int nq, int hd, int n_split, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (n_split < 1 || n_split > kMergeMaxSplits) return hipErrorInvalidValue;
  dim3 grid(nq, B);
#define DORY_MRG(T, HDV)                                                                                   \
  dory_launch((k_attn_merge<T, HDV>), grid, dim3(kMergeThreads), 0, st, part, qkvg, ld, gate_off, gate, (T*)ob, \
              nq, n_split)
  if (dtype == 0) {
    if (hd == 64) DORY_MRG(float, 64); else if (hd == 128) DORY_MRG(float, 128); else return hipErrorInvalidValue;
  } else {
    if (hd == 64) DORY_MRG(bf16, 64); else if (hd == 128) DORY_MRG(bf16, 128); else return hipErrorInvalidValue;
  }
#undef DORY_MRG
  return hipGetLastError();
}

}  // namespace dory
