// Depth-1 truncated backward of the last recurrent invocation: the pieces
// that are not projections. The pages say the looped stage trains with
// backpropagation truncated to depth one, only the final recurrent
// invocation receiving gradients ("Dory1.0-4B: A Looped Normalized-GPT", AI
// summary, Methodology in Plain English). The projections and their
// gradients (dX = dY W, dW = dY^T X) run on the matrix-core GEMM of
// k_linear.hip through transposed operands; everything here is float32.
//
// Row kernels take one 256-thread workgroup per row; the attention kernels
// one wave per (row, head): a wave walks the allowed keys (or, for the key
// gradient, the queries that see a key) in tiles of 64, one key per lane for
// the dot products, then one dimension per lane for the weighted sums.
#include "common.h"
#include "kernels.h"

namespace dory {
namespace {

__device__ __forceinline__ float guard_norm(float ss) { return sqrtf(fmaxf(ss, 1e-30f)); }

// ---------------------------------------------------------------------------
// copies and transposes
// ---------------------------------------------------------------------------
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_bw_cast(const TI* __restrict__ in, TO* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = from_f<TO>(to_f(in[i]));
}

// out [C][R] = in [R][C] (row stride ld), 32x32 tiles through LDS
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_bw_transpose(const TI* __restrict__ in, int64_t ld, TO* __restrict__ out,
                                                      int R, int C) {
  __shared__ float tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int j = ty; j < 32; j += 8) {
    const int r = r0 + j, c = c0 + tx;
    if (r < R && c < C) tile[j][tx] = to_f(in[(size_t)r * ld + c]);
  }
  __syncthreads();
#pragma unroll
  for (int j = ty; j < 32; j += 8) {
    const int c = c0 + j, r = r0 + tx;
    if (c < C && r < R) out[(size_t)c * R + r] = from_f<TO>(tile[tx][j]);
  }
}

// bfloat16 out [C][R] = in [R][C] (row stride ld) in 64 x 64 tiles: 16-byte
// loads of 8 consecutive columns, 2-byte scatter into an LDS tile (rows of 66
// elements: consecutive rows start 33 banks apart), 2-byte gathers of 8
// consecutive rows and 16-byte stores. vin / vout: the 16-byte accesses are
// aligned (ld a multiple of 8 and a 16-byte aligned base for the loads; R a
// multiple of 8 and an aligned base for the stores); chunks that run past the
// matrix edge, or any chunk without them, go element by element.
__global__ __launch_bounds__(256) void k_bw_transpose16(const bf16* __restrict__ in, int64_t ld,
                                                        bf16* __restrict__ out, int R, int C, int vin, int vout) {
  __shared__ uint16_t tile[64][66];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const uint16_t* src = (const uint16_t*)in;
  uint16_t* dst = (uint16_t*)out;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int rr = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    uint16_t v[8];
    if (vin && r < R && c + 8 <= C) {
      const uint4 u = *(const uint4*)(src + (size_t)r * ld + c);
      v[0] = u.x & 0xffff; v[1] = u.x >> 16; v[2] = u.y & 0xffff; v[3] = u.y >> 16;
      v[4] = u.z & 0xffff; v[5] = u.z >> 16; v[6] = u.w & 0xffff; v[7] = u.w >> 16;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (r < R && c + e < C) ? src[(size_t)r * ld + c + e] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[rr][cc + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int cc = q >> 3, rr = (q & 7) * 8;  // output row c0 + cc, columns r0 + rr ..
    const int c = c0 + cc, r = r0 + rr;
    if (c >= C) continue;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[rr + e][cc];
    if (vout && r + 8 <= R) {
      uint4 u;
      u.x = v[0] | ((uint32_t)v[1] << 16); u.y = v[2] | ((uint32_t)v[3] << 16);
      u.z = v[4] | ((uint32_t)v[5] << 16); u.w = v[6] | ((uint32_t)v[7] << 16);
      *(uint4*)(dst + (size_t)c * R + r) = u;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r + e < R) dst[(size_t)c * R + r + e] = v[e];
    }
  }
}

__global__ __launch_bounds__(256) void k_bw_add(const float* __restrict__ a, const float* __restrict__ b,
                                                const float* __restrict__ b2, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = a[i] + (b2 ? b[i] + b2[i] : b[i]);
}

// out[c][j] = sum of in[r][j] over the rows r of chunk c (blockIdx.y, rc rows
// each), in row order: a fixed summation order, so deterministic
constexpr int kColRows = 64;
__global__ __launch_bounds__(256) void k_bw_colsum(const float* __restrict__ in, int M, int d, int rc,
                                                   float* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int r0 = blockIdx.y * rc, r1 = min(M, r0 + rc);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += in[(size_t)r * d + j];
  out[(size_t)blockIdx.y * d + j] = s;
}

// ---------------------------------------------------------------------------
// forward with the values the backward needs
// ---------------------------------------------------------------------------
// h' = norm(h + alpha (norm(y) - h)); keeps norm(y), |y|, |z| and h'
// (y2: optional second partial sum of y)
template <typename T>
__global__ __launch_bounds__(256) void k_bw_update_fwd(const float* __restrict__ h, const float* __restrict__ y,
                                                       const float* __restrict__ y2,
                                                       const float* __restrict__ alpha, int d,
                                                       float* __restrict__ yh, float* __restrict__ ry,
                                                       float* __restrict__ rz, float* __restrict__ hout,
                                                       T* __restrict__ hout_t) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  const float* hr = h + r * d;
  const float* yr = y + r * d;
  const float* y2r = y2 ? y2 + r * d : nullptr;
  auto yv = [&](int j) { return y2r ? yr[j] + y2r[j] : yr[j]; };
  float ss = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float v = yv(j);
    ss += v * v;
  }
  const float ny = guard_norm(block_sum<256>(ss, sh));
  float sz = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float yn = yv(j) / ny;
    const float z = hr[j] + alpha[j] * (yn - hr[j]);
    yh[r * d + j] = yn;
    hout[r * d + j] = z;
    sz += z * z;
  }
  const float nz = guard_norm(block_sum<256>(sz, sh));
  for (int j = threadIdx.x; j < d; j += 256) {
    const float v = hout[r * d + j] / nz;
    hout[r * d + j] = v;
    if (hout_t) hout_t[r * d + j] = from_f<T>(v);
  }
  if (threadIdx.x == 0) {
    ry[r] = ny;
    rz[r] = nz;
  }
}

// RoPE + per-head norm of q and k from the fused projection; one wave per (row, head)
__global__ __launch_bounds__(256) void k_bw_rope_norm_fwd(const float* __restrict__ P1, int ldp,
                                                          const float2* __restrict__ tab, int n, int nq, int nkv,
                                                          int hd, int M, float* __restrict__ qn,
                                                          float* __restrict__ kn, float* __restrict__ rq,
                                                          float* __restrict__ rk) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (head >= nq + nkv || r >= M) return;
  const int half = hd / 2, pos = r % n;
  const float* src = P1 + (size_t)r * ldp + (size_t)head * hd;
  float r1 = 0.f, r2 = 0.f;
  if (lane < half) {
    const float x1 = src[lane], x2 = src[lane + half];
    const float2 cs = tab[(size_t)pos * half + lane];
    r1 = x1 * cs.x - x2 * cs.y;
    r2 = x2 * cs.x + x1 * cs.y;
  }
  const float nr = guard_norm(wave_sum(r1 * r1 + r2 * r2));
  const bool isq = head < nq;
  float* dst = isq ? qn + (size_t)r * nq * hd + (size_t)head * hd : kn + (size_t)r * nkv * hd + (size_t)(head - nq) * hd;
  if (lane < half) {
    dst[lane] = r1 / nr;
    dst[lane + half] = r2 / nr;
  }
  if (lane == 0) {
    if (isq)
      rq[(size_t)r * nq + head] = nr;
    else
      rk[(size_t)r * nkv + head - nq] = nr;
  }
}

// Causal (+ window) softmax attention of one sequence chunk; one wave per
// (row, q head); keeps the output and the softmax max / sum per (row, head).
template <int HD>
__global__ __launch_bounds__(256) void k_bw_attn_fwd(BwAttn a, float* __restrict__ o, float* __restrict__ mst,
                                                     float* __restrict__ lst) {
  constexpr int DL = HD / 64;  // dimensions per lane
  __shared__ float qs[4][HD];
  __shared__ float ps[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hq = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (hq >= a.nq) return;
  const int b = r / a.n, t = r % a.n;
  const int kvh = hq * a.nkv / a.nq;
  const int s_lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  const size_t rb = (size_t)b * a.n;
  const float* q = a.qn + (size_t)r * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int i = 0; i < DL; ++i) qs[wave][lane + 64 * i] = q[lane + 64 * i];
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) acc[i] = 0.f;
  for (int s0 = s_lo; s0 <= t; s0 += 64) {
    const int s = s0 + lane;
    float sc = -INFINITY;
    if (s <= t) {
      const float* k = a.kn + (rb + s) * a.nkv * HD + (size_t)kvh * HD;
      float dot = 0.f;
      for (int e = 0; e < HD; ++e) dot += qs[wave][e] * k[e];
      sc = a.scale * dot;
    }
    const float mn = fmaxf(m, wave_max(sc));
    const float p = s <= t ? expf(sc - mn) : 0.f;
    const float corr = expf(m - mn);
    l = l * corr + wave_sum(p);
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] *= corr;
    m = mn;
    ps[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const int cnt = min(64, t - s0 + 1);
    for (int j = 0; j < cnt; ++j) {
      const float* v = a.v + (rb + s0 + j) * a.ldv + (size_t)kvh * HD;
      const float pj = ps[wave][j];
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] += pj * v[lane + 64 * i];
    }
    __builtin_amdgcn_wave_barrier();
  }
  float* out = o + (size_t)r * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int i = 0; i < DL; ++i) out[lane + 64 * i] = acc[i] / l;
  if (lane == 0) {
    mst[(size_t)r * a.nq + hq] = m;
    lst[(size_t)r * a.nq + hq] = l;
  }
}

// c = o * sigmoid(gate); oh = c / |c| (float32 and the GEMM copy); keeps |c|
template <typename T>
__global__ __launch_bounds__(256) void k_bw_gate_fwd(const float* __restrict__ o, const float* __restrict__ P1,
                                                     int ldp, int goff, int mode, int hd, int qd,
                                                     float* __restrict__ oh, T* __restrict__ oh_t,
                                                     float* __restrict__ rc) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  const float* g = P1 + r * ldp + goff;
  float ss = 0.f;
  for (int j = threadIdx.x; j < qd; j += 256) {
    const float sg = mode == 1 ? sigmoidf_(g[j]) : mode == 2 ? sigmoidf_(g[j / hd]) : 1.f;
    const float c = o[r * qd + j] * sg;
    oh[r * qd + j] = c;
    ss += c * c;
  }
  const float nc = guard_norm(block_sum<256>(ss, sh));
  for (int j = threadIdx.x; j < qd; j += 256) {
    const float v = oh[r * qd + j] / nc;
    oh[r * qd + j] = v;
    oh_t[r * qd + j] = from_f<T>(v);
  }
  if (threadIdx.x == 0) rc[r] = nc;
}

// a = s / |s| with s = u * silu(v); keeps |s|
template <typename T>
__global__ __launch_bounds__(256) void k_bw_swiglu_fwd(const float* __restrict__ P2, int F, float* __restrict__ a32,
                                                       T* __restrict__ a_t, float* __restrict__ rs) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  const float* u = P2 + r * 2 * F;
  float ss = 0.f;
  for (int j = threadIdx.x; j < F; j += 256) {
    const float v = u[F + j];
    const float s = u[j] * v * sigmoidf_(v);
    a32[r * F + j] = s;
    ss += s * s;
  }
  const float ns = guard_norm(block_sum<256>(ss, sh));
  for (int j = threadIdx.x; j < F; j += 256) {
    const float v = a32[r * F + j] / ns;
    a32[r * F + j] = v;
    a_t[r * F + j] = from_f<T>(v);
  }
  if (threadIdx.x == 0) rs[r] = ns;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// dh = (G - hn (hn . G)) / |h|, hn = h / |h|: the block's closing norm
__global__ __launch_bounds__(256) void k_bw_final(const float* __restrict__ h, const float* __restrict__ G, int d,
                                                  float* __restrict__ dh) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  float ss = 0.f, sg = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    ss += h[r * d + j] * h[r * d + j];
    sg += h[r * d + j] * G[r * d + j];
  }
  const float nh = guard_norm(block_sum<256>(ss, sh));
  const float hg = block_sum<256>(sg, sh) / nh;  // hn . G
  for (int j = threadIdx.x; j < d; j += 256) dh[r * d + j] = (G[r * d + j] - h[r * d + j] / nh * hg) / nh;
}

// Update h' = norm(z), z = h + alpha (yh - h), yh = norm(y), given dL/dh':
// dz = (dh' - h' (h' . dh')) / |z|; dres = dz (1 - alpha); dyh = dz alpha;
// dy = (dyh - yh (yh . dyh)) / |y| (GEMM copy); contrib = dz (yh - h), whose
// column sums are dL/dalpha.
template <typename T>
__global__ __launch_bounds__(256) void k_bw_update_bwd(const float* __restrict__ dho, const float* __restrict__ ho,
                                                       const float* __restrict__ rz, const float* __restrict__ yh,
                                                       const float* __restrict__ ry, const float* __restrict__ h,
                                                       const float* __restrict__ alpha, int d,
                                                       float* __restrict__ dres, T* __restrict__ dy_t,
                                                       float* __restrict__ contrib) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  float s1 = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) s1 += ho[r * d + j] * dho[r * d + j];
  const float hd_ = block_sum<256>(s1, sh);
  const float iz = 1.f / rz[r];
  float s2 = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float dz = (dho[r * d + j] - ho[r * d + j] * hd_) * iz;
    const float yv = yh[r * d + j];
    dres[r * d + j] = dz * (1.f - alpha[j]);
    contrib[r * d + j] = dz * (yv - h[r * d + j]);
    s2 += yv * dz * alpha[j];
  }
  const float yd = block_sum<256>(s2, sh);
  const float iy = 1.f / ry[r];
  for (int j = threadIdx.x; j < d; j += 256) {
    const float dz = (dho[r * d + j] - ho[r * d + j] * hd_) * iz;
    dy_t[r * d + j] = from_f<T>((dz * alpha[j] - yh[r * d + j] * yd) * iy);
  }
}

// a = norm(u silu(v)): da -> [du | dv] (GEMM copy)
template <typename T>
__global__ __launch_bounds__(256) void k_bw_swiglu_bwd(const float* __restrict__ da, const float* __restrict__ a32,
                                                       const float* __restrict__ rs, const float* __restrict__ P2,
                                                       int F, T* __restrict__ dP2) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  float s = 0.f;
  for (int j = threadIdx.x; j < F; j += 256) s += a32[r * F + j] * da[r * F + j];
  const float ad = block_sum<256>(s, sh);
  const float is = 1.f / rs[r];
  for (int j = threadIdx.x; j < F; j += 256) {
    const float ds = (da[r * F + j] - a32[r * F + j] * ad) * is;
    const float u = P2[r * 2 * F + j], v = P2[r * 2 * F + F + j];
    const float sg = sigmoidf_(v);
    dP2[r * 2 * F + j] = from_f<T>(ds * v * sg);
    dP2[r * 2 * F + F + j] = from_f<T>(ds * u * sg * (1.f + v * (1.f - sg)));
  }
}

// oh = norm(o * sigmoid(g)): doh -> do (float32 [M][qd]) and dgate into the
// gate columns of dP1 (float32, row stride ldp)
__global__ __launch_bounds__(256) void k_bw_gate_bwd(const float* __restrict__ doh, const float* __restrict__ oh,
                                                     const float* __restrict__ rc, const float* __restrict__ o,
                                                     const float* __restrict__ P1, int ldp, int goff, int mode,
                                                     int hd, int qd, float* __restrict__ dO,
                                                     float* __restrict__ dP1, const float* __restrict__ doh2) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  auto dv = [&](int j) { return doh2 ? doh[r * qd + j] + doh2[r * qd + j] : doh[r * qd + j]; };
  float s = 0.f;
  for (int j = threadIdx.x; j < qd; j += 256) s += oh[r * qd + j] * dv(j);
  const float od = block_sum<256>(s, sh);
  const float ic = 1.f / rc[r];
  const float* g = P1 + r * ldp + goff;
  float* dg = dP1 + r * ldp + goff;
  for (int j = threadIdx.x; j < qd; j += 256) {
    const float dc = (dv(j) - oh[r * qd + j] * od) * ic;
    if (mode == 1) {
      const float sg = sigmoidf_(g[j]);
      dO[r * qd + j] = dc * sg;
      dg[j] = dc * o[r * qd + j] * sg * (1.f - sg);
    } else if (mode == 2) {
      dO[r * qd + j] = dc * sigmoidf_(g[j / hd]);
    } else {
      dO[r * qd + j] = dc;
    }
  }
  if (mode == 2) {  // one gate per head: dgate_h = sum over the head of dc * o, times sigmoid'
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nh = qd / hd;
    for (int hh = wave; hh < nh; hh += 4) {
      const float sg = sigmoidf_(g[hh]);
      float acc = 0.f;
      for (int e = lane; e < hd; e += 64) {
        const int j = hh * hd + e;
        acc += (dv(j) - oh[r * qd + j] * od) * ic * o[r * qd + j];
      }
      acc = wave_sum(acc);
      if (lane == 0) dg[hh] = acc * sg * (1.f - sg);
    }
  }
}

// D[r][h] = do . o (softmax backward term); one wave per (row, head)
template <int HD>
__global__ __launch_bounds__(256) void k_bw_attn_D(const float* __restrict__ dO, const float* __restrict__ o, int nq,
                                                   int M, float* __restrict__ D) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hq = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (hq >= nq || r >= M) return;
  const size_t off = (size_t)r * nq * HD + (size_t)hq * HD;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < HD / 64; ++i) s += dO[off + lane + 64 * i] * o[off + lane + 64 * i];
  s = wave_sum(s);
  if (lane == 0) D[(size_t)r * nq + hq] = s;
}

// dqn[t] = scale * sum_s dS[t][s] kn[s], dS = P (dP - D), dP = do . v
template <int HD>
__global__ __launch_bounds__(256) void k_bw_attn_dq(BwAttn a, const float* __restrict__ dO,
                                                    const float* __restrict__ mst, const float* __restrict__ lst,
                                                    const float* __restrict__ D, float* __restrict__ dqn) {
  constexpr int DL = HD / 64;
  __shared__ float qs[4][HD];
  __shared__ float ds_[4][HD];
  __shared__ float ps[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hq = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (hq >= a.nq) return;
  const int b = r / a.n, t = r % a.n;
  const int kvh = hq * a.nkv / a.nq;
  const int s_lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  const size_t rb = (size_t)b * a.n;
  const size_t qo = (size_t)r * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    qs[wave][lane + 64 * i] = a.qn[qo + lane + 64 * i];
    ds_[wave][lane + 64 * i] = dO[qo + lane + 64 * i];
  }
  __builtin_amdgcn_wave_barrier();
  const float m = mst[(size_t)r * a.nq + hq], il = 1.f / lst[(size_t)r * a.nq + hq];
  const float Dv = D[(size_t)r * a.nq + hq];
  float acc[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) acc[i] = 0.f;
  for (int s0 = s_lo; s0 <= t; s0 += 64) {
    const int s = s0 + lane;
    float dS = 0.f;
    if (s <= t) {
      const float* k = a.kn + (rb + s) * a.nkv * HD + (size_t)kvh * HD;
      const float* v = a.v + (rb + s) * a.ldv + (size_t)kvh * HD;
      float qk = 0.f, dv = 0.f;
      for (int e = 0; e < HD; ++e) {
        qk += qs[wave][e] * k[e];
        dv += ds_[wave][e] * v[e];
      }
      const float p = expf(a.scale * qk - m) * il;
      dS = p * (dv - Dv);
    }
    ps[wave][lane] = dS;
    __builtin_amdgcn_wave_barrier();
    const int cnt = min(64, t - s0 + 1);
    for (int j = 0; j < cnt; ++j) {
      const float* k = a.kn + (rb + s0 + j) * a.nkv * HD + (size_t)kvh * HD;
      const float w = ps[wave][j];
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] += w * k[lane + 64 * i];
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int i = 0; i < DL; ++i) dqn[qo + lane + 64 * i] = a.scale * acc[i];
}

// For key s of kv head kvh: dkn[s] = scale * sum_(t, h) dS[t][s] qn[t], dv[s] =
// sum_(t, h) P[t][s] do[t], over the queries t that see s and the q heads h
// of the group. One wave per (row s, kv head).
template <int HD>
__global__ __launch_bounds__(256) void k_bw_attn_dkv(BwAttn a, const float* __restrict__ dO,
                                                     const float* __restrict__ mst, const float* __restrict__ lst,
                                                     const float* __restrict__ D, float* __restrict__ dkn,
                                                     float* __restrict__ dv) {
  constexpr int DL = HD / 64;
  __shared__ float ks[4][HD];
  __shared__ float vs[4][HD];
  __shared__ float ps[4][64];
  __shared__ float dss[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kvh = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (kvh >= a.nkv) return;
  const int b = r / a.n, s = r % a.n;
  const int G = a.nq / a.nkv;
  const int t_hi = a.window > 0 ? min(a.n - 1, s + a.window - 1) : a.n - 1;
  const size_t rb = (size_t)b * a.n;
  const size_t ko = (size_t)r * a.nkv * HD + (size_t)kvh * HD;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    ks[wave][lane + 64 * i] = a.kn[ko + lane + 64 * i];
    vs[wave][lane + 64 * i] = a.v[(size_t)r * a.ldv + (size_t)kvh * HD + lane + 64 * i];
  }
  __builtin_amdgcn_wave_barrier();
  float ak[DL], av[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) ak[i] = av[i] = 0.f;
  const int items = (t_hi - s + 1) * G;  // (query, head in group) pairs
  for (int i0 = 0; i0 < items; i0 += 64) {
    const int it = i0 + lane;
    float p = 0.f, dS = 0.f;
    if (it < items) {
      const int t = s + it / G, hq = kvh * G + it % G;
      const size_t qo = (rb + t) * a.nq * HD + (size_t)hq * HD;
      float qk = 0.f, dvv = 0.f;
      for (int e = 0; e < HD; ++e) {
        qk += a.qn[qo + e] * ks[wave][e];
        dvv += dO[qo + e] * vs[wave][e];
      }
      const size_t si = (rb + t) * a.nq + hq;
      p = expf(a.scale * qk - mst[si]) / lst[si];
      dS = p * (dvv - D[si]);
    }
    ps[wave][lane] = p;
    dss[wave][lane] = dS;
    __builtin_amdgcn_wave_barrier();
    const int cnt = min(64, items - i0);
    for (int j = 0; j < cnt; ++j) {
      const int t = s + (i0 + j) / G, hq = kvh * G + (i0 + j) % G;
      const size_t qo = (rb + t) * a.nq * HD + (size_t)hq * HD;
      const float pj = ps[wave][j], dj = dss[wave][j];
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        ak[i] += dj * a.qn[qo + lane + 64 * i];
        av[i] += pj * dO[qo + lane + 64 * i];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    dkn[ko + lane + 64 * i] = a.scale * ak[i];
    dv[ko + lane + 64 * i] = av[i];
  }
}

// dqn, dkn -> through the per-head norm and RoPE^T into the q / k columns of
// dP1; dv into its v columns. One wave per (row, head of q | k | v).
__global__ __launch_bounds__(256) void k_bw_rope_norm_bwd(const float* __restrict__ dqn, const float* __restrict__ qn,
                                                          const float* __restrict__ rq,
                                                          const float* __restrict__ dkn, const float* __restrict__ kn,
                                                          const float* __restrict__ rk, const float* __restrict__ dv,
                                                          const float2* __restrict__ tab, int n, int nq, int nkv,
                                                          int hd, int M, float* __restrict__ dP1, int ldp) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + wave;
  const int r = blockIdx.y;
  if (head >= nq + 2 * nkv || r >= M) return;
  const int half = hd / 2, pos = r % n;
  float* dst = dP1 + (size_t)r * ldp + (size_t)head * hd;
  if (head >= nq + nkv) {  // v: straight copy
    const float* src = dv + (size_t)r * nkv * hd + (size_t)(head - nq - nkv) * hd;
    for (int e = lane; e < hd; e += 64) dst[e] = src[e];
    return;
  }
  const bool isq = head < nq;
  const size_t off = isq ? (size_t)r * nq * hd + (size_t)head * hd : (size_t)r * nkv * hd + (size_t)(head - nq) * hd;
  const float* xn = (isq ? qn : kn) + off;
  const float* dx = (isq ? dqn : dkn) + off;
  const float rn = isq ? rq[(size_t)r * nq + head] : rk[(size_t)r * nkv + head - nq];
  float x1 = 0.f, x2 = 0.f, d1 = 0.f, d2 = 0.f;
  if (lane < half) {
    x1 = xn[lane];
    x2 = xn[lane + half];
    d1 = dx[lane];
    d2 = dx[lane + half];
  }
  const float xd = wave_sum(x1 * d1 + x2 * d2);
  if (lane < half) {
    const float g1 = (d1 - x1 * xd) / rn, g2 = (d2 - x2 * xd) / rn;  // gradient of the rotated vector
    const float2 cs = tab[(size_t)pos * half + lane];
    dst[lane] = g1 * cs.x + g2 * cs.y;          // rotation transposed
    dst[lane + half] = g2 * cs.x - g1 * cs.y;
  }
}

// ---------------------------------------------------------------------------
// head-major operand copies of the matrix-core attention (k_bw_flash.hip)
// ---------------------------------------------------------------------------
// dst [B][H][n][hd] (model dtype) from src rows [B*n][ld] at column off + h*hd
// The same copy, one workgroup row per source row (blockIdx.x) and four
// consecutive elements per thread (ld, off, hd multiples of 4, src 16-byte
// aligned): no per-element index division.
template <typename T>
__global__ __launch_bounds__(256) void k_bw_to_heads4(const float* __restrict__ src, int64_t ld, int off, int H,
                                                      int hd, int n, T* __restrict__ dst) {
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H * hd) return;
  const int64_t row = blockIdx.x;  // b n + t
  const int64_t b = row / n;
  const int t = (int)(row - b * n);
  const int h = c / hd, d = c - h * hd;
  const float4 v = *(const float4*)(src + row * ld + off + c);
  T* o = dst + ((b * H + h) * n + t) * hd + d;
  o[0] = from_f<T>(v.x);
  o[1] = from_f<T>(v.y);
  o[2] = from_f<T>(v.z);
  o[3] = from_f<T>(v.w);
}

template <typename T>
__global__ __launch_bounds__(256) void k_bw_to_heads(const float* __restrict__ src, int64_t ld, int off, int H,
                                                     int hd, int n, int64_t total, T* __restrict__ dst) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int d = (int)(e % hd);
  const int64_t r = e / hd;  // (b, h, t)
  const int t = (int)(r % n);
  const int64_t bh = r / n;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  dst[e] = from_f<T>(src[(b * n + t) * ld + off + (int64_t)h * hd + d]);
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

// ---------------------------------------------------------------------------
// The same row kernels with the row held in registers (NPT elements per
// thread, rows up to 256 NPT): one read of each input instead of one per
// pass. Element for element the same operations in the same order as the
// streaming versions above, so the results are bit-identical.
// ---------------------------------------------------------------------------
template <typename T, int NPT>
__global__ __launch_bounds__(256) void k_bw_update_fwd_r(const float* __restrict__ h, const float* __restrict__ y,
                                                         const float* __restrict__ y2,
                                                         const float* __restrict__ alpha, int d,
                                                         float* __restrict__ yh, float* __restrict__ ry,
                                                         float* __restrict__ rz, float* __restrict__ hout,
                                                         T* __restrict__ hout_t) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  // loads from clamped indices, all issued before the first use; elements
  // past the row read as zero
  float yv[NPT], hv[NPT], av[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int jc = min((int)threadIdx.x + 256 * i, d - 1);
    yv[i] = y2 ? y[r * d + jc] + y2[r * d + jc] : y[r * d + jc];
    hv[i] = h[r * d + jc];
    av[i] = alpha[jc];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    if ((int)threadIdx.x + 256 * i >= d) yv[i] = hv[i] = 0.f;
    ss += yv[i] * yv[i];
  }
  const float ny = guard_norm(block_sum<256>(ss, sh));
  float sz = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {  // past the row: yv = hv = 0, so z = 0
    const int j = threadIdx.x + 256 * i;
    const float yn = yv[i] / ny;
    const float z = hv[i] + av[i] * (yn - hv[i]);
    if (j < d) yh[r * d + j] = yn;
    hv[i] = z;
    sz += z * z;
  }
  const float nz = guard_norm(block_sum<256>(sz, sh));
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < d) {
      const float v = hv[i] / nz;
      hout[r * d + j] = v;
      if (hout_t) hout_t[r * d + j] = from_f<T>(v);
    }
  }
  if (threadIdx.x == 0) {
    ry[r] = ny;
    rz[r] = nz;
  }
}

template <typename T, int NPT>
__global__ __launch_bounds__(256) void k_bw_swiglu_fwd_r(const float* __restrict__ P2, int F, float* __restrict__ a32,
                                                         T* __restrict__ a_t, float* __restrict__ rs) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  const float* u = P2 + r * 2 * F;
  float uv[NPT], vv[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int jc = min((int)threadIdx.x + 256 * i, F - 1);
    uv[i] = u[jc];
    vv[i] = u[F + jc];
  }
  float sv[NPT];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    sv[i] = (int)threadIdx.x + 256 * i < F ? uv[i] * vv[i] * sigmoidf_(vv[i]) : 0.f;
    ss += sv[i] * sv[i];
  }
  const float ns = guard_norm(block_sum<256>(ss, sh));
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < F) {
      const float v = sv[i] / ns;
      a32[r * F + j] = v;
      a_t[r * F + j] = from_f<T>(v);
    }
  }
  if (threadIdx.x == 0) rs[r] = ns;
}

template <typename T, int NPT>
__global__ __launch_bounds__(256) void k_bw_update_bwd_r(const float* __restrict__ dho, const float* __restrict__ ho,
                                                         const float* __restrict__ rz, const float* __restrict__ yh,
                                                         const float* __restrict__ ry, const float* __restrict__ h,
                                                         const float* __restrict__ alpha, int d,
                                                         float* __restrict__ dres, T* __restrict__ dy_t,
                                                         float* __restrict__ contrib) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  float gv[NPT], ov[NPT], yv[NPT], hv[NPT], av[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int jc = min((int)threadIdx.x + 256 * i, d - 1);
    gv[i] = dho[r * d + jc];
    ov[i] = ho[r * d + jc];
    yv[i] = yh[r * d + jc];
    hv[i] = h[r * d + jc];
    av[i] = alpha[jc];
  }
  float s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    if ((int)threadIdx.x + 256 * i >= d) gv[i] = ov[i] = yv[i] = 0.f;
    s1 += ov[i] * gv[i];
  }
  const float hd_ = block_sum<256>(s1, sh);
  const float iz = 1.f / rz[r];
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    const float dz = (gv[i] - ov[i] * hd_) * iz;
    if (j < d) {
      dres[r * d + j] = dz * (1.f - av[i]);
      contrib[r * d + j] = dz * (yv[i] - hv[i]);
    }
    s2 += yv[i] * dz * av[i];
    gv[i] = dz;
  }
  const float yd = block_sum<256>(s2, sh);
  const float iy = 1.f / ry[r];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < d) dy_t[r * d + j] = from_f<T>((gv[i] * av[i] - yv[i] * yd) * iy);
  }
}

template <typename T, int NPT>
__global__ __launch_bounds__(256) void k_bw_swiglu_bwd_r(const float* __restrict__ da, const float* __restrict__ a32,
                                                         const float* __restrict__ rs, const float* __restrict__ P2,
                                                         int F, T* __restrict__ dP2) {
  __shared__ float sh[4];
  const size_t r = blockIdx.x;
  float dv[NPT], av[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int jc = min((int)threadIdx.x + 256 * i, F - 1);
    dv[i] = da[r * F + jc];
    av[i] = a32[r * F + jc];
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) s += (int)threadIdx.x + 256 * i < F ? av[i] * dv[i] : 0.f;
  const float ad = block_sum<256>(s, sh);
  const float is = 1.f / rs[r];
  float uv[NPT], vv[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int jc = min((int)threadIdx.x + 256 * i, F - 1);
    uv[i] = P2[r * 2 * F + jc];
    vv[i] = P2[r * 2 * F + F + jc];
  }
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < F) {
      const float ds = (dv[i] - av[i] * ad) * is;
      const float u = uv[i], v = vv[i];
      const float sg = sigmoidf_(v);
      dP2[r * 2 * F + j] = from_f<T>(ds * v * sg);
      dP2[r * 2 * F + F + j] = from_f<T>(ds * u * sg * (1.f + v * (1.f - sg)));
    }
  }
}

// elements per thread of a register-held row of n, at most max_npt (0: too
// long, stream it). The update kernels hold two arrays and stop at 16: at 32
// the compiler left their arrays in scratch memory.
int row_npt(int n, int max_npt) {
  const int npt = n <= 1024 ? 4 : n <= 2048 ? 8 : n <= 4096 ? 16 : n <= 8192 ? 32 : 0;
  return npt <= max_npt ? npt : 0;
}

#define DORY_ROW_DISPATCH16(KERNEL, T, NPT, ...)                                             \
  switch (NPT) {                                                                              \
    case 4: hipLaunchKernelGGL((KERNEL<T, 4>), __VA_ARGS__); break;                          \
    case 8: hipLaunchKernelGGL((KERNEL<T, 8>), __VA_ARGS__); break;                          \
    default: hipLaunchKernelGGL((KERNEL<T, 16>), __VA_ARGS__); break;                        \
  }
#define DORY_ROW_DISPATCH(KERNEL, T, NPT, ...)                                               \
  if ((NPT) == 32) {                                                                          \
    hipLaunchKernelGGL((KERNEL<T, 32>), __VA_ARGS__);                                        \
  } else {                                                                                    \
    DORY_ROW_DISPATCH16(KERNEL, T, NPT, __VA_ARGS__)                                         \
  }

}  // namespace

hipError_t launch_bw_to_heads(int dt, const float* src, int64_t ld, int off, int H, int hd, int n, int B, void* dst,
                              hipStream_t st) {
  const int64_t total = (int64_t)B * H * n * hd;
  if (total <= 0) return hipSuccess;
  if (ld % 4 == 0 && off % 4 == 0 && hd % 4 == 0 && ((uintptr_t)src & 15) == 0 && (H * hd + 1023) / 1024 <= 65535) {
    const dim3 grid((unsigned)((int64_t)B * n), (unsigned)((H * hd + 1023) / 1024));
    if (dt == 1)
      hipLaunchKernelGGL((k_bw_to_heads4<bf16>), grid, dim3(256), 0, st, src, ld, off, H, hd, n, (bf16*)dst);
    else
      hipLaunchKernelGGL((k_bw_to_heads4<float>), grid, dim3(256), 0, st, src, ld, off, H, hd, n, (float*)dst);
    return hipGetLastError();
  }
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_to_heads<bf16>), dim3(blocks_for(total)), dim3(256), 0, st, src, ld, off, H, hd, n,
                       total, (bf16*)dst);
  else
    hipLaunchKernelGGL((k_bw_to_heads<float>), dim3(blocks_for(total)), dim3(256), 0, st, src, ld, off, H, hd, n,
                       total, (float*)dst);
  return hipGetLastError();
}

hipError_t launch_bw_attn_D(const float* dO, const float* o, int nq, int hd, int M, float* D, hipStream_t st) {
  const dim3 g((nq + 3) / 4, M);
  if (hd == 64)
    hipLaunchKernelGGL((k_bw_attn_D<64>), g, dim3(256), 0, st, dO, o, nq, M, D);
  else if (hd == 128)
    hipLaunchKernelGGL((k_bw_attn_D<128>), g, dim3(256), 0, st, dO, o, nq, M, D);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_bw_cast(int dt_out, const float* in, void* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (dt_out == 1)
    hipLaunchKernelGGL((k_bw_cast<float, bf16>), dim3(blocks_for(n)), dim3(256), 0, st, in, (bf16*)out, n);
  else
    hipLaunchKernelGGL((k_bw_cast<float, float>), dim3(blocks_for(n)), dim3(256), 0, st, in, (float*)out, n);
  return hipGetLastError();
}

hipError_t launch_bw_transpose(int dt, const void* in, int64_t ld, void* out, int R, int C, hipStream_t st) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if ((R + 31) / 32 > 65535) return hipErrorInvalidValue;
  const dim3 grid((C + 31) / 32, (R + 31) / 32);
  if (dt == 1) {
    const int vin = ld % 8 == 0 && ((uintptr_t)in & 15) == 0;
    const int vout = R % 8 == 0 && ((uintptr_t)out & 15) == 0;
    hipLaunchKernelGGL(k_bw_transpose16, dim3((C + 63) / 64, (R + 63) / 64), dim3(256), 0, st, (const bf16*)in, ld,
                       (bf16*)out, R, C, vin, vout);
  } else
    hipLaunchKernelGGL((k_bw_transpose<float, float>), grid, dim3(256), 0, st, (const float*)in, ld, (float*)out, R,
                       C);
  return hipGetLastError();
}

hipError_t launch_bw_add(const float* a, const float* b, float* out, int64_t n, hipStream_t st, const float* b2) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_add, dim3(blocks_for(n)), dim3(256), 0, st, a, b, b2, out, n);
  return hipGetLastError();
}

hipError_t launch_bw_colsum(const float* in, int M, int d, float* out, float* part, hipStream_t st) {
  if (M <= 0 || d <= 0) return hipSuccess;
  const int chunks = (M + kColRows - 1) / kColRows;
  if (chunks == 1) {
    hipLaunchKernelGGL(k_bw_colsum, dim3(blocks_for(d), 1), dim3(256), 0, st, in, M, d, M, out);
    return hipGetLastError();
  }
  // chunk sums into part [chunks][d], then the sum of the chunks in order
  hipLaunchKernelGGL(k_bw_colsum, dim3(blocks_for(d), chunks), dim3(256), 0, st, in, M, d, kColRows, part);
  hipLaunchKernelGGL(k_bw_colsum, dim3(blocks_for(d), 1), dim3(256), 0, st, (const float*)part, chunks, d, chunks,
                     out);
  return hipGetLastError();
}

hipError_t launch_bw_update_fwd(int dt, const float* h, const float* y, const float* alpha, int M, int d, float* yh,
                                float* ry, float* rz, float* hout, void* hout_t, hipStream_t st, const float* y2) {
  if (M <= 0) return hipSuccess;
  if (const int npt = row_npt(d, 16)) {
    if (dt == 1) {
      DORY_ROW_DISPATCH16(k_bw_update_fwd_r, bf16, npt, dim3(M), dim3(256), 0, st, h, y, y2, alpha, d, yh, ry, rz, hout,
                        (bf16*)hout_t)
    } else {
      DORY_ROW_DISPATCH16(k_bw_update_fwd_r, float, npt, dim3(M), dim3(256), 0, st, h, y, y2, alpha, d, yh, ry, rz, hout,
                        (float*)hout_t)
    }
    return hipGetLastError();
  }
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_update_fwd<bf16>), dim3(M), dim3(256), 0, st, h, y, y2, alpha, d, yh, ry, rz, hout,
                       (bf16*)hout_t);
  else
    hipLaunchKernelGGL((k_bw_update_fwd<float>), dim3(M), dim3(256), 0, st, h, y, y2, alpha, d, yh, ry, rz, hout,
                       (float*)hout_t);
  return hipGetLastError();
}

hipError_t launch_bw_rope_norm_fwd(const float* P1, int ldp, const float2* tab, int n, int nq, int nkv, int hd, int M,
                                   float* qn, float* kn, float* rq, float* rk, hipStream_t st) {
  if (hd > 128 || hd % 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bw_rope_norm_fwd, dim3((nq + nkv + 3) / 4, M), dim3(256), 0, st, P1, ldp, tab, n, nq, nkv, hd,
                     M, qn, kn, rq, rk);
  return hipGetLastError();
}

hipError_t launch_bw_attn_fwd(const BwAttn& a, int M, float* o, float* mst, float* lst, hipStream_t st) {
  const dim3 grid((a.nq + 3) / 4, M);
  if (a.hd == 64)
    hipLaunchKernelGGL((k_bw_attn_fwd<64>), grid, dim3(256), 0, st, a, o, mst, lst);
  else if (a.hd == 128)
    hipLaunchKernelGGL((k_bw_attn_fwd<128>), grid, dim3(256), 0, st, a, o, mst, lst);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bw_gate_fwd(int dt, const float* o, const float* P1, int ldp, int goff, int mode, int hd, int qd,
                              int M, float* oh, void* oh_t, float* rc, hipStream_t st) {
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_gate_fwd<bf16>), dim3(M), dim3(256), 0, st, o, P1, ldp, goff, mode, hd, qd, oh,
                       (bf16*)oh_t, rc);
  else
    hipLaunchKernelGGL((k_bw_gate_fwd<float>), dim3(M), dim3(256), 0, st, o, P1, ldp, goff, mode, hd, qd, oh,
                       (float*)oh_t, rc);
  return hipGetLastError();
}

hipError_t launch_bw_swiglu_fwd(int dt, const float* P2, int F, int M, float* a32, void* a_t, float* rs,
                                hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (const int npt = row_npt(F, 32)) {
    if (dt == 1) {
      DORY_ROW_DISPATCH(k_bw_swiglu_fwd_r, bf16, npt, dim3(M), dim3(256), 0, st, P2, F, a32, (bf16*)a_t, rs)
    } else {
      DORY_ROW_DISPATCH(k_bw_swiglu_fwd_r, float, npt, dim3(M), dim3(256), 0, st, P2, F, a32, (float*)a_t, rs)
    }
    return hipGetLastError();
  }
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_swiglu_fwd<bf16>), dim3(M), dim3(256), 0, st, P2, F, a32, (bf16*)a_t, rs);
  else
    hipLaunchKernelGGL((k_bw_swiglu_fwd<float>), dim3(M), dim3(256), 0, st, P2, F, a32, (float*)a_t, rs);
  return hipGetLastError();
}

hipError_t launch_bw_final(const float* h, const float* G, int M, int d, float* dh, hipStream_t st) {
  hipLaunchKernelGGL(k_bw_final, dim3(M), dim3(256), 0, st, h, G, d, dh);
  return hipGetLastError();
}

hipError_t launch_bw_update_bwd(int dt, const float* dho, const float* ho, const float* rz, const float* yh,
                                const float* ry, const float* h, const float* alpha, int M, int d, float* dres,
                                void* dy_t, float* contrib, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (const int npt = row_npt(d, 16)) {
    if (dt == 1) {
      DORY_ROW_DISPATCH16(k_bw_update_bwd_r, bf16, npt, dim3(M), dim3(256), 0, st, dho, ho, rz, yh, ry, h, alpha, d, dres,
                        (bf16*)dy_t, contrib)
    } else {
      DORY_ROW_DISPATCH16(k_bw_update_bwd_r, float, npt, dim3(M), dim3(256), 0, st, dho, ho, rz, yh, ry, h, alpha, d,
                        dres, (float*)dy_t, contrib)
    }
    return hipGetLastError();
  }
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_update_bwd<bf16>), dim3(M), dim3(256), 0, st, dho, ho, rz, yh, ry, h, alpha, d, dres,
                       (bf16*)dy_t, contrib);
  else
    hipLaunchKernelGGL((k_bw_update_bwd<float>), dim3(M), dim3(256), 0, st, dho, ho, rz, yh, ry, h, alpha, d, dres,
                       (float*)dy_t, contrib);
  return hipGetLastError();
}

hipError_t launch_bw_swiglu_bwd(int dt, const float* da, const float* a32, const float* rs, const float* P2, int F,
                                int M, void* dP2, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (const int npt = row_npt(F, 32)) {
    if (dt == 1) {
      DORY_ROW_DISPATCH(k_bw_swiglu_bwd_r, bf16, npt, dim3(M), dim3(256), 0, st, da, a32, rs, P2, F, (bf16*)dP2)
    } else {
      DORY_ROW_DISPATCH(k_bw_swiglu_bwd_r, float, npt, dim3(M), dim3(256), 0, st, da, a32, rs, P2, F, (float*)dP2)
    }
    return hipGetLastError();
  }
  if (dt == 1)
    hipLaunchKernelGGL((k_bw_swiglu_bwd<bf16>), dim3(M), dim3(256), 0, st, da, a32, rs, P2, F, (bf16*)dP2);
  else
    hipLaunchKernelGGL((k_bw_swiglu_bwd<float>), dim3(M), dim3(256), 0, st, da, a32, rs, P2, F, (float*)dP2);
  return hipGetLastError();
}

hipError_t launch_bw_gate_bwd(const float* doh, const float* oh, const float* rc, const float* o, const float* P1,
                              int ldp, int goff, int mode, int hd, int qd, int M, float* dO, float* dP1,
                              hipStream_t st, const float* doh2) {
  hipLaunchKernelGGL(k_bw_gate_bwd, dim3(M), dim3(256), 0, st, doh, oh, rc, o, P1, ldp, goff, mode, hd, qd, dO, dP1,
                     doh2);
  return hipGetLastError();
}

hipError_t launch_bw_attn_bwd(const BwAttn& a, int M, const float* dO, const float* o, const float* mst,
                              const float* lst, float* D, float* dqn, float* dkn, float* dv, hipStream_t st) {
  const dim3 gq((a.nq + 3) / 4, M), gk((a.nkv + 3) / 4, M);
  if (a.hd == 64) {
    hipLaunchKernelGGL((k_bw_attn_D<64>), gq, dim3(256), 0, st, dO, o, a.nq, M, D);
    hipLaunchKernelGGL((k_bw_attn_dq<64>), gq, dim3(256), 0, st, a, dO, mst, lst, D, dqn);
    hipLaunchKernelGGL((k_bw_attn_dkv<64>), gk, dim3(256), 0, st, a, dO, mst, lst, D, dkn, dv);
  } else if (a.hd == 128) {
    hipLaunchKernelGGL((k_bw_attn_D<128>), gq, dim3(256), 0, st, dO, o, a.nq, M, D);
    hipLaunchKernelGGL((k_bw_attn_dq<128>), gq, dim3(256), 0, st, a, dO, mst, lst, D, dqn);
    hipLaunchKernelGGL((k_bw_attn_dkv<128>), gk, dim3(256), 0, st, a, dO, mst, lst, D, dkn, dv);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bw_rope_norm_bwd(const float* dqn, const float* qn, const float* rq, const float* dkn,
                                   const float* kn, const float* rk, const float* dv, const float2* tab, int n, int nq,
                                   int nkv, int hd, int M, float* dP1, int ldp, hipStream_t st) {
  if (hd > 128 || hd % 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bw_rope_norm_bwd, dim3((nq + 2 * nkv + 3) / 4, M), dim3(256), 0, st, dqn, qn, rq, dkn, kn, rk,
                     dv, tab, n, nq, nkv, hd, M, dP1, ldp);
  return hipGetLastError();
}

}  // namespace dory
