// Attention of the depth-1 truncated backward on the matrix cores (bfloat16
// models, head dim 64 or 128): the forward with its softmax statistics, dQ,
// and dK / dV per query head, then summed over the query heads of each kv
// head. Scores are never
// stored: every kernel recomputes its score tiles from q and k, so the
// workspace stays O(n d) ("Dory1.0-4B: A Looped Normalized-GPT", ai.info AI
// summary, Methodology in Plain English: backpropagation is truncated to the
// last invocation of the recurrent block; the attention is the causal /
// sliding-window grouped-query attention of the forward).
//
// Math (one head, queries t, keys s, unit q and k): S = scale q.k,
// P = exp(S - m_t) / l_t over the allowed keys (s <= t, t - s < window),
// O = P V;  given dO:  D_t = dO_t . O_t,  dP = dO V^T,  dS = P (dP - D),
// dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// Operands are bfloat16 head-major copies [B][H][n][hd] and transposed ones
// [B][H][hd][nT] (nT = n rounded up to 8, zero past n), made once per layer.
// Matrix products use v_mfma_f32_32x32x16_bf16 as the prefill attention
// does: the product whose rows are the workgroup's own positions is taken
// transposed (S^T = K Q^T in the query kernels, S = Q K^T in the key kernel)
// so that each position's softmax terms sit in its two lanes, and the 16
// inner positions of every step are permuted identically on both operands
// (lane half g supplies positions 4g..4g+3 and 8+4g..8+4g+3), which lets
// the second product take P or dS straight from the score registers.
#include "common.h"
#include "kernels.h"

namespace dory {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kFR = 128;  // own positions per workgroup (4 waves x 32)
constexpr int kFT = 64;   // inner positions per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bool allowed(int t, int s, int window) {
  return s <= t && (window == 0 || t - s < window);
}

// Staging of a tile in two halves, so that the global loads of the next tile
// are in flight while the current one is multiplied: fetch_* loads into
// registers (every thread HD/32 16-byte pieces), put_* writes them to LDS.
//
// [kFT rows][HD] of a head-major array (rows r0.., clamped to n-1), LDS rows
// of ld elements
template <int HD>
__device__ __forceinline__ void fetch_rows(const bf16* __restrict__ src, int n, int r0, u32x4* v) {
  constexpr int CPK = HD / 8;
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) {
    const int e = threadIdx.x + 256 * i;
    v[i] = *(const u32x4*)(src + (size_t)min(r0 + e / CPK, n - 1) * HD + 8 * (e % CPK));
  }
}
template <int HD>
__device__ __forceinline__ void put_rows(const u32x4* v, bf16* dst, int ld) {
  constexpr int CPK = HD / 8;
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) {
    const int e = threadIdx.x + 256 * i;
    *(u32x4*)(dst + (e / CPK) * ld + 8 * (e % CPK)) = v[i];
  }
}

// [HD][kFT] of a transposed array (columns c0.., nT columns, zero past n;
// runs past nT clamped: their positions are masked), LDS rows of ld
// elements written as 8-byte pieces
template <int HD>
__device__ __forceinline__ void fetch_cols(const bf16* __restrict__ srcT, int nT, int c0, u32x4* v) {
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) {
    const int e = threadIdx.x + 256 * i;
    v[i] = *(const u32x4*)(srcT + (size_t)(e >> 3) * nT + min(c0 + 8 * (e & 7), nT - 8));
  }
}
template <int HD>
__device__ __forceinline__ void put_cols(const u32x4* v, bf16* dst, int ld) {
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) {
    const int e = threadIdx.x + 256 * i;
    u32x2_t* p = (u32x2_t*)(dst + (e >> 3) * ld + 8 * (e & 7));
    p[0] = u32x2_t{v[i][0], v[i][1]};
    p[1] = u32x2_t{v[i][2], v[i][3]};
  }
}

// A operand of the second product: rows = 32 dims of block mb, the 16 inner
// positions of step (kt, h) in the permuted order, from a transposed tile
template <int LD>
__device__ __forceinline__ bf16x8_t perm_frag(const bf16* tT, int mb, int kt, int h, int lr, int g) {
  const bf16* row = tT + (mb * 32 + lr) * LD + 32 * kt + 16 * h + 4 * g;
  const u32x2_t lo = *(const u32x2_t*)row;
  const u32x2_t hi = *(const u32x2_t*)(row + 8);
  const u32x4 v = u32x4{lo[0], lo[1], hi[0], hi[1]};
  return *(const bf16x8_t*)&v;
}

// ---------------------------------------------------------------------------
// forward: O and the softmax statistics (mst: the reference exponent m of
// p = 2^(scale log2(e) q.k - m), lst: the reciprocal of the row sum)
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256, 2) void k_bwf_fwd(BwFlash a) {
  constexpr int KLD = HD + 8, VLD = kFT + 4, NKS = HD / 16, NMB = HD / 32;
  __shared__ __align__(16) bf16 Ks[kFT * KLD];
  __shared__ __align__(16) bf16 Vt[HD * VLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, g = lane >> 5;
  const int nqb = (a.n + kFR - 1) / kFR;
  const int qb = nqb - 1 - (int)(blockIdx.x % nqb);  // most keys first
  const int bh = blockIdx.x / nqb, b = bh / a.nq, hq = bh % a.nq, kvh = hq * a.nkv / a.nq;
  const int i0 = qb * kFR, iw0 = i0 + 32 * wave;
  const int t = min(iw0 + lq, a.n - 1);
  const bf16* Q = a.Q + ((size_t)b * a.nq + hq) * a.n * HD;
  const bf16* K = a.K + ((size_t)b * a.nkv + kvh) * a.n * HD;
  const bf16* VT = a.VT + ((size_t)b * a.nkv + kvh) * HD * a.nT;
  bf16x8_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(Q + (size_t)t * HD + 16 * ks + 8 * g);

  const float sl2 = a.scale * kLog2e;
  const bool fixed_ref = sl2 <= 40.f;  // unit q, k: no score exceeds scale
  float m = fixed_ref ? sl2 : -1e30f, l = 0.f;
  f32x16_t acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const int hi = min(i0 + kFR - 1, a.n - 1);
  const int lo = a.window ? max(0, i0 - a.window + 1) : 0;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
  const int sfirst = lo / kFT * kFT, slast = hi / kFT * kFT;
  u32x4 kr[HD / 32], vr[HD / 32];
  fetch_rows<HD>(K, a.n, sfirst, kr);
  fetch_cols<HD>(VT, a.nT, sfirst, vr);
  for (int s0 = sfirst; s0 <= slast; s0 += kFT) {
    __syncthreads();  // the previous tile is consumed
    put_rows<HD>(kr, Ks, KLD);
    put_cols<HD>(vr, Vt, VLD);
    __syncthreads();
    const int s1 = min(s0 + kFT, slast);  // in flight during this tile (the last refetches itself)
    fetch_rows<HD>(K, a.n, s1, kr);
    fetch_cols<HD>(VT, a.nT, s1, vr);
    if (iw0 >= a.n || s0 > iw0 + 31) continue;
    f32x16_t sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8_t*)(Ks + (kt * 32 + lq) * KLD + 16 * ks + 8 * g), qf[ks], sc[kt], 0, 0, 0);
    }
    // masks only where some key of the tile is not allowed for some query of
    // the wave (a wave-uniform branch); a masked score is -inf, so p = 0
    const bool edge = s0 + kFT - 1 > iw0 || (a.window && min(iw0 + 31, a.n - 1) - s0 >= a.window);
    float tmax = -INFINITY;
    if (edge) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int s = s0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
          sc[kt][r] = allowed(t, s, a.window) && s < a.n ? sc[kt][r] : -INFINITY;
          tmax = fmaxf(tmax, sc[kt][r]);
        }
    } else if (!fixed_ref) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sc[kt][r]);
    }
    float mn = m;
    if (!fixed_ref) mn = fmaxf(m, fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ps = 0.f;
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        bf16x2_t pr;
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[kt][r], sl2, -mn));
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[kt][r + 1], sl2, -mn));
        ps = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ps, false);
        pb[kt][r >> 3][r & 7] = pr[0];
        pb[kt][r >> 3][(r & 7) + 1] = pr[1];
      }
    l = l * alpha + ps;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (alpha != 1.f) acc[mb] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(perm_frag<VLD>(Vt, mb, kt, h, lq, g), pb[kt][h],
                                                            acc[mb], 0, 0, 0);
    }
  }
  if (iw0 >= a.n || iw0 + lq >= a.n) return;
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.f / lt;
  const size_t row = (size_t)b * a.n + t;
  float* o = a.o + row * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)] = acc[mb][r] * inv;
  if (g == 0) {
    a.mst[row * a.nq + hq] = m;    // reference exponent, log2 units of the scaled score
    a.lst[row * a.nq + hq] = inv;  // 1 / row sum
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries of one (sequence, q head)
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256, 2) void k_bwf_dq(BwFlash a) {
  constexpr int KLD = HD + 8, VLD = kFT + 4, NKS = HD / 16, NMB = HD / 32;
  __shared__ __align__(16) bf16 Ks[kFT * KLD];
  __shared__ __align__(16) bf16 Vs[kFT * KLD];
  __shared__ __align__(16) bf16 KTs[HD * VLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, g = lane >> 5;
  const int nqb = (a.n + kFR - 1) / kFR;
  const int qb = nqb - 1 - (int)(blockIdx.x % nqb);
  const int bh = blockIdx.x / nqb, b = bh / a.nq, hq = bh % a.nq, kvh = hq * a.nkv / a.nq;
  const int i0 = qb * kFR, iw0 = i0 + 32 * wave;
  const int t = min(iw0 + lq, a.n - 1);
  const size_t qoff = ((size_t)b * a.nq + hq) * a.n * HD;
  const bf16* K = a.K + ((size_t)b * a.nkv + kvh) * a.n * HD;
  const bf16* V = a.V + ((size_t)b * a.nkv + kvh) * a.n * HD;
  const bf16* KT = a.KT + ((size_t)b * a.nkv + kvh) * HD * a.nT;
  bf16x8_t qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = *(const bf16x8_t*)(a.Q + qoff + (size_t)t * HD + 16 * ks + 8 * g);
    df[ks] = *(const bf16x8_t*)(a.dO + qoff + (size_t)t * HD + 16 * ks + 8 * g);
  }
  const size_t row = (size_t)b * a.n + t;
  const float sl2 = a.scale * kLog2e;
  const float m2 = a.mst[row * a.nq + hq], il = a.lst[row * a.nq + hq];
  const float Dt = a.D[row * a.nq + hq];
  f32x16_t acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const int hi = min(i0 + kFR - 1, a.n - 1);
  const int lo = a.window ? max(0, i0 - a.window + 1) : 0;
  const int sfirst = lo / kFT * kFT, slast = hi / kFT * kFT;
  // K and V rows of the next tile are prefetched; K^T is loaded at staging
  // (registers for two workgroups per CU)
  u32x4 kr[HD / 32], vr[HD / 32];
  fetch_rows<HD>(K, a.n, sfirst, kr);
  fetch_rows<HD>(V, a.n, sfirst, vr);
  for (int s0 = sfirst; s0 <= slast; s0 += kFT) {
    __syncthreads();
    {
      u32x4 ktr[HD / 32];
      fetch_cols<HD>(KT, a.nT, s0, ktr);
      put_rows<HD>(kr, Ks, KLD);
      put_rows<HD>(vr, Vs, KLD);
      put_cols<HD>(ktr, KTs, VLD);
    }
    __syncthreads();
    const int s1 = min(s0 + kFT, slast);
    fetch_rows<HD>(K, a.n, s1, kr);
    fetch_rows<HD>(V, a.n, s1, vr);
    if (iw0 >= a.n || s0 > iw0 + 31) continue;
    // one 32-key half at a time (fewer live registers): S^T, dP^T, dS, dQ
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16_t sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (kt * 32 + lq) * KLD + 16 * ks + 8 * g;
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(Ks + o), qf[ks], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(Vs + o), df[ks], dp, 0, 0, 0);
      }
      // p = 2^(s sl2 - m) / l (the exponent is at most 0 up to rounding)
      bf16x8_t db[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s = s0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
        const float e = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -m2)) * il;
        const float p = allowed(t, s, a.window) && s < a.n ? e : 0.f;
        db[r >> 3][r & 7] = (__bf16)(p * (dp[r] - Dt));
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(perm_frag<VLD>(KTs, mb, kt, h, lq, g), db[h], acc[mb],
                                                            0, 0, 0);
    }
  }
  if (iw0 >= a.n || iw0 + lq >= a.n) return;
  float* dq = a.dq + row * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)] = a.scale * acc[mb][r];
}

// ---------------------------------------------------------------------------
// dK, dV of one query head: one workgroup per 128 keys of one (sequence, q
// head), over every query that sees those keys; the G query heads of a kv
// head write separate partial sums (dkh, dvh [B n][nq][HD]) that
// k_bwf_sum_heads adds in head order. Workgroup ids: the eight XCDs take
// every eighth head, and inside an XCD the key blocks with the most queries
// start first.
//
// The query tiles (Q and dO rows, their transposed copies, the softmax
// terms) reach LDS by direct global->LDS loads into two alternating
// buffers: the next tile's loads are in flight while the current one is
// multiplied, without registers to hold them (a wave keeps its 32 keys' k,
// v fragments and two 32 x HD accumulators). Dense rows with the 16-byte
// chunk index XORed by (row mod 8): row tiles are read conflict-free,
// transposed ones with at most two lanes per bank.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
#define DORY_BWF_WAIT_VM0() __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8))

// byte offset of 16-byte chunk c of row r (rows of cpr chunks)
__device__ __forceinline__ int sw_off(int r, int c, int cpr) { return (r * cpr + (c ^ (r & 7))) * 16; }

template <int HD>
struct DkvStage {
  static constexpr int kRow = kFT * HD * 2;  // one row tile (Q or dO), bytes
  static constexpr int kCol = HD * kFT * 2;  // one transposed tile
  static constexpr int kBytes = 2 * kRow + 2 * kCol + 3 * kFT * 4;  // + m, 1/l, D of the 64 queries
};

template <int HD>
__global__ __launch_bounds__(256, 1) void k_bwf_dkv(BwFlash a) {
  constexpr int NKS = HD / 16, NMB = HD / 32, CPR = HD / 8;
  using S = DkvStage<HD>;
  __shared__ __align__(1024) unsigned char lds[2 * S::kBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lk = lane & 31, g = lane >> 5;
  const int nkb = (a.n + kFR - 1) / kFR;
  const int BH = a.B * a.nq, hpx = (BH + 7) / 8;
  const int j = (int)(blockIdx.x >> 3), bhq = (j % hpx) * 8 + (int)(blockIdx.x & 7);
  const int kb = j / hpx;
  if (bhq >= BH || kb >= nkb) return;
  const int b = bhq / a.nq, hq = bhq % a.nq, kvh = hq / (a.nq / a.nkv);
  const int k0 = kb * kFR, kw0 = k0 + 32 * wave;
  const int s = min(kw0 + lk, a.n - 1);
  const size_t koff = ((size_t)b * a.nkv + kvh) * a.n * HD;
  const int khi = min(k0 + kFR - 1, a.n - 1);
  const int qlo = k0, qhi = a.window ? min(a.n - 1, khi + a.window - 1) : a.n - 1;
  const int qfirst = qlo / kFT * kFT, qlast = qhi / kFT * kFT;
  const bf16* Qh = a.Q + ((size_t)b * a.nq + hq) * a.n * HD;
  const bf16* Dh = a.dO + ((size_t)b * a.nq + hq) * a.n * HD;
  const bf16* QT = a.QT + ((size_t)b * a.nq + hq) * HD * a.nT;
  const bf16* DT = a.dOT + ((size_t)b * a.nq + hq) * HD * a.nT;
  const size_t srow = (size_t)b * a.n;

  // direct loads of the tile at query q0 into buffer buf: every wave fills
  // CPR/4 1 KB blocks of each row tile and HD/32 of each transposed tile
  auto issue = [&](int q0, int buf) {
    unsigned char* st = lds + buf * S::kBytes;
#pragma unroll
    for (int i = 0; i < CPR / 4; ++i) {
      const int e = (wave * (CPR / 4) + i) * 64 + lane;
      const int r = e / CPR, c = (e % CPR) ^ (r & 7);
      const size_t go = (size_t)min(q0 + r, a.n - 1) * HD + 8 * c;
      unsigned char* d0 = st + (wave * (CPR / 4) + i) * 1024;
      __builtin_amdgcn_global_load_lds(Qh + go, (lds_void_t*)d0, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Dh + go, (lds_void_t*)(d0 + S::kRow), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < HD / 32; ++i) {
      const int e = (wave * (HD / 32) + i) * 64 + lane;
      const int d = e >> 3, c = (e & 7) ^ (d & 7);
      const size_t go = (size_t)d * a.nT + min(q0 + 8 * c, a.nT - 8);
      unsigned char* d0 = st + 2 * S::kRow + (wave * (HD / 32) + i) * 1024;
      __builtin_amdgcn_global_load_lds(QT + go, (lds_void_t*)d0, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(DT + go, (lds_void_t*)(d0 + S::kCol), 16, 0, 0);
    }
  };
  // softmax terms of a tile's 64 queries: threads 0..63 load one query's
  // into registers a tile ahead and write them to LDS before the barrier
  float st_m = 0.f, st_l = 0.f, st_d = 0.f;
  auto fetch_stats = [&](int q0) {
    if (tid < kFT) {
      const size_t r = (srow + min(q0 + tid, a.n - 1)) * a.nq + hq;
      st_m = a.mst[r];
      st_l = a.lst[r];
      st_d = a.D[r];
    }
  };
  // query tiles from the last down: the key blocks of one head then read the
  // same tile at the same step (one fetch from memory, the rest from L2)
  issue(qlast, 0);
  fetch_stats(qlast);

  bf16x8_t kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = *(const bf16x8_t*)(a.K + koff + (size_t)s * HD + 16 * ks + 8 * g);
    vf[ks] = *(const bf16x8_t*)(a.V + koff + (size_t)s * HD + 16 * ks + 8 * g);
  }
  const float sl2 = a.scale * kLog2e;
  f32x16_t ak[NMB], av[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ak[mb][r] = av[mb][r] = 0.f;

  // A operand of the second products from a transposed tile: rows = dims
  // 32 mb .., the 16 positions of step (qt, hh) in the permuted order
  auto tfrag = [&](const unsigned char* tT, int mb, int qt, int hh) {
    const int d = mb * 32 + lk, c = 4 * qt + 2 * hh;
    const u32x2_t lo = *(const u32x2_t*)(tT + sw_off(d, c, 8) + 8 * g);
    const u32x2_t hi = *(const u32x2_t*)(tT + sw_off(d, c + 1, 8) + 8 * g);
    const u32x4 v = u32x4{lo[0], lo[1], hi[0], hi[1]};
    return *(const bf16x8_t*)&v;
  };

  int buf = 0;
  for (int q0 = qlast; q0 >= qfirst; q0 -= kFT, buf ^= 1) {
    unsigned char* st = lds + buf * S::kBytes;
    DORY_BWF_WAIT_VM0();  // this wave's loads of the current buffer (and the k, v fragments, the terms) are done
    if (tid < kFT) {
      float* t3 = (float*)(st + 2 * S::kRow + 2 * S::kCol);
      t3[tid] = st_m;
      t3[kFT + tid] = st_l;
      t3[2 * kFT + tid] = st_d;
    }
    __syncthreads();  // everyone's are, and the other buffer is consumed
    if (q0 - kFT >= qfirst) {
      issue(q0 - kFT, buf ^ 1);
      fetch_stats(q0 - kFT);
    }
    const unsigned char* Qs = st;
    const unsigned char* Ds_ = st + S::kRow;
    const unsigned char* QTs = st + 2 * S::kRow;
    const unsigned char* DTs = QTs + S::kCol;
    const float* m2s = (const float*)(DTs + S::kCol);
    const float* ils = m2s + kFT;
    const float* Dq = ils + kFT;
    // queries of the tile that see some key of this wave
    if (kw0 >= a.n || q0 + kFT - 1 < kw0 || (a.window && q0 > kw0 + 31 + a.window - 1)) continue;
    // one 32-query half at a time: S^T, dP^T, P, dS, then dV, dK
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16_t sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = sw_off(qt * 32 + lk, 2 * ks + g, CPR);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(Qs + o), kf[ks], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(Ds_ + o), vf[ks], dp, 0, 0, 0);
      }
      // p = 2^(s sl2 - m) / l: the exponent is at most 0 up to rounding (m is
      // the row's reference), so the hardware exp2 needs no range handling
      bf16x8_t pb[2], db[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
        const int t = q0 + qi;
        const float e = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -m2s[qi])) * ils[qi];
        const float p = allowed(t, s, a.window) && t < a.n ? e : 0.f;
        pb[r >> 3][r & 7] = (__bf16)p;
        db[r >> 3][r & 7] = (__bf16)(p * (dp[r] - Dq[qi]));
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          av[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(DTs, mb, qt, hh), pb[hh], av[mb], 0, 0, 0);
          ak[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(QTs, mb, qt, hh), db[hh], ak[mb], 0, 0, 0);
        }
    }
  }
  if (kw0 >= a.n || kw0 + lk >= a.n) return;
  const size_t row = srow + s;
  float* dk = a.dkh + row * a.nq * HD + (size_t)hq * HD;
  float* dv = a.dvh + row * a.nq * HD + (size_t)hq * HD;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
      dk[d] = a.scale * ak[mb][r];
      dv[d] = av[mb][r];
    }
}

// dk [B n][nkv][hd] = sum over the G query heads h of kv head k, in head
// order, of dkh [B n][k G + h][hd] (the same for dv); one thread per output
__global__ __launch_bounds__(256) void k_bwf_sum_heads(const float* __restrict__ dkh, const float* __restrict__ dvh,
                                                       int G, int hd, int nkv, int64_t total, float* __restrict__ dk,
                                                       float* __restrict__ dv) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int kvd = nkv * hd;
  const int64_t row = e / kvd;
  const int c = (int)(e % kvd), kvh = c / hd, d = c % hd;
  const size_t src = (size_t)row * G * kvd + ((size_t)kvh * G) * hd + d;
  float sk = dkh[src], sv = dvh[src];
  for (int h = 1; h < G; ++h) {
    sk += dkh[src + (size_t)h * hd];
    sv += dvh[src + (size_t)h * hd];
  }
  dk[e] = sk;
  dv[e] = sv;
}

// bfloat16 transposed head copies: dst[b][h][d][t] (nT columns, zero past n)
// from float32 rows src[(b n + t) ld + off + h hd + d]; one thread per element,
// t fastest
__global__ __launch_bounds__(256) void k_bwf_heads_t(const float* __restrict__ src, int64_t ld, int off, int H,
                                                     int hd, int n, int nT, int64_t total, bf16* __restrict__ dst) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int t = (int)(e % nT);
  const int64_t r = e / nT;  // (b, h, d)
  const int d = (int)(r % hd);
  const int64_t bh = r / hd;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  dst[e] = t < n ? from_f<bf16>(src[(b * n + t) * ld + off + (int64_t)h * hd + d]) : (bf16)0;
}

// The same copies through a 64 x 64 LDS tile per (sequence, head): float4
// reads along the head dimension, 8-byte writes of four consecutive
// positions (ld, off, hd multiples of 4, src 16-byte aligned). Grid:
// (nT / 64 position tiles, hd / 64 dimension tiles, B H).
__global__ __launch_bounds__(256) void k_bwf_heads_t64(const float* __restrict__ src, int64_t ld, int off, int H,
                                                       int hd, int n, int nT, bf16* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, bh = blockIdx.z;
  const int64_t b = bh / H;
  const int h = bh - (int)b * H;
  const int rr = threadIdx.x >> 4, cc = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int t = t0 + 16 * p + rr, d = d0 + cc;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < n && d < hd) v = *(const float4*)(src + (b * n + t) * ld + off + (int64_t)h * hd + d);
    tile[16 * p + rr][cc] = v.x;
    tile[16 * p + rr][cc + 1] = v.y;
    tile[16 * p + rr][cc + 2] = v.z;
    tile[16 * p + rr][cc + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int dd = 16 * p + rr, d = d0 + dd, t = t0 + cc;
    if (d >= hd || t >= nT) continue;
    const uint32_t lo = (uint32_t)from_f<bf16>(tile[cc][dd]) | ((uint32_t)from_f<bf16>(tile[cc + 1][dd]) << 16);
    const uint32_t hi =
        (uint32_t)from_f<bf16>(tile[cc + 2][dd]) | ((uint32_t)from_f<bf16>(tile[cc + 3][dd]) << 16);
    *(u32x2_t*)(dst + ((size_t)bh * hd + d) * nT + t) = u32x2_t{lo, hi};
  }
}

}  // namespace

bool bw_flash_supported(int dtype, int hd, int nq, int nkv) {
  return dtype == 1 && (hd == 64 || hd == 128) && nkv > 0 && nq % nkv == 0;
}

hipError_t launch_bw_heads_t(const float* src, int64_t ld, int off, int H, int hd, int n, int B, int nT, void* dst,
                             hipStream_t st) {
  const int64_t total = (int64_t)B * H * hd * nT;
  if (total <= 0) return hipSuccess;
  if (nT < n || nT % 8) return hipErrorInvalidValue;
  if (ld % 4 == 0 && off % 4 == 0 && hd % 4 == 0 && ((uintptr_t)src & 15) == 0 && (hd + 63) / 64 <= 65535 &&
      (int64_t)B * H <= 65535) {
    const dim3 grid((unsigned)((nT + 63) / 64), (unsigned)((hd + 63) / 64), (unsigned)(B * H));
    hipLaunchKernelGGL(k_bwf_heads_t64, grid, dim3(256), 0, st, src, ld, off, H, hd, n, nT, (bf16*)dst);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_bwf_heads_t, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, ld, off, H, hd, n,
                     nT, total, (bf16*)dst);
  return hipGetLastError();
}

hipError_t launch_bw_flash_fwd(const BwFlash& a, hipStream_t st) {
  if (a.B * a.n <= 0) return hipSuccess;
  if (!bw_flash_supported(1, a.hd, a.nq, a.nkv) || a.nT < a.n || a.nT % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n + kFR - 1) / kFR * a.B * a.nq));
  if (a.hd == 64)
    hipLaunchKernelGGL(k_bwf_fwd<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_bwf_fwd<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bw_flash_bwd(const BwFlash& a, hipStream_t st) {
  if (a.B * a.n <= 0) return hipSuccess;
  if (!bw_flash_supported(1, a.hd, a.nq, a.nkv) || a.nT < a.n || a.nT % 8) return hipErrorInvalidValue;
  if (!a.dkh || !a.dvh) return hipErrorInvalidValue;
  const int nkb = (a.n + kFR - 1) / kFR, hpx = (a.B * a.nq + 7) / 8;
  const dim3 gq((unsigned)(nkb * a.B * a.nq)), gk((unsigned)((int64_t)nkb * hpx * 8));
  if (a.hd == 64) {
    hipLaunchKernelGGL(k_bwf_dq<64>, gq, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_bwf_dkv<64>, gk, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_bwf_dq<128>, gq, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_bwf_dkv<128>, gk, dim3(256), 0, st, a);
  }
  const int64_t total = (int64_t)a.B * a.n * a.nkv * a.hd;
  hipLaunchKernelGGL(k_bwf_sum_heads, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const float*)a.dkh,
                     (const float*)a.dvh, a.nq / a.nkv, a.hd, a.nkv, total, a.dk, a.dv);
  return hipGetLastError();
}

}  // namespace dory
