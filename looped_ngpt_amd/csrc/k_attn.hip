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
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (kk < nk) {
        const int s = s0 + kk;
        const T* ks;
        const T* vs;
        if (s >= a.p0) {
          const size_t o = ((size_t)(b * a.n + (s - a.p0)) * a.nkv + kvh) * HD;
          ks = kw + o;
          vs = vw + o;
        } else {
          const int slot = a.is_full ? s : s % a.window;
          const size_t o = (((size_t)b * a.nkv + kvh) * a.slots + slot) * HD;
          ks = kc + o;
          vs = vc + o;
        }
        kv4 = ((const uint4*)ks)[c];
        vv4 = ((const uint4*)vs)[c];
      }
      *(uint4*)(Ks + kk * KLD + c * VEC) = kv4;
      *(uint4*)(Vs + kk * HD + c * VEC) = vv4;
    }
    __syncthreads();

    // scores of this thread's key for every head of the group
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dsum = 0.f;
#pragma unroll
      for (int d = 0; d < DP; ++d) dsum = fmaf(qs[g][part * DP + d], to_f(Ks[key * KLD + part * DP + d]), dsum);
#pragma unroll
      for (int o = 1; o < NPART; o <<= 1) dsum += __shfl_xor(dsum, o, 64);
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
    case 1: hipLaunchKernelGGL((k_attn_split<T, HD, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_attn_split<T, HD, 2>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_attn_split<T, HD, 3>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_attn_split<T, HD, 4>), grid, dim3(256), 0, st, a); break;
    case 6: hipLaunchKernelGGL((k_attn_split<T, HD, 6>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_attn_split<T, HD, 8>), grid, dim3(256), 0, st, a); break;
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
  hipLaunchKernelGGL((k_attn_combine<T, HDV>), grid, dim3(256), 0, st, part, qkvg, ld, gate_off, gate, (T*)ob, \
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
