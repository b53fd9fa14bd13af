// Prefill attention of the looped nGPT on the matrix cores (bfloat16, head
// dim 64 or 128): softmax(scale * q.k) v over the allowed keys of a sliding
// window (t - W < s <= t) or full (s <= t) layer, grouped-query heads, then
// the sigmoid output gate — the attention sublayer of the nGPT block
// ("Dory1.0-4B: A Looped Normalized-GPT", ai.info AI summary, Methodology in
// Plain English).
//
// One workgroup of eight waves takes eight work items of one kv head; an
// item is 32 consecutive query positions of one query head, and the items of
// a kv head are ordered query block first, then head inside the GQA group, so
// the G query heads that read the same keys share the workgroup (for G = 3 a
// workgroup spans about three 32-position query blocks of all three heads).
// Keys are visited in tiles of 64 positions staged in LDS, K as rows
// [key][hd] and V transposed [hd][key] (the cache keeps values in 32-position
// blocks [hd][32], the call's own values as [hd][n]); every staged tile
// serves all eight waves. Two LDS tile buffers alternate: the global loads of
// tile T+2 are issued right after the barrier that publishes tile T+1, and
// tile T+1 is written to LDS after tile T has been multiplied, so one
// workgroup barrier per tile suffices.
// Per wave and 32-key half tile (v_mfma_f32_32x32x16_bf16):
//   S^T[key][query] = K . Q^T            hd/16 steps
//   online softmax per query column      a lane owns one query; the lane
//                                        32 apart holds the other key rows
//   O^T[d][query]  += V^T . P^T          P in bfloat16, 2 steps x hd/32 blocks
// so the running max, sum and rescale of a query stay inside its two lanes.
// The key order inside a 16-key step is permuted the same way on both
// operands (lane half g supplies keys 4g..4g+3 and 8+4g..8+4g+3), which lets
// P^T come straight from the score registers.
//
// Workgroup g takes kv head g mod (B x nkv), so with eight kv heads every XCD
// (workgroups are dealt to the XCDs round robin) streams the keys of one kv
// head through its own L2; the item blocks with the most keys start first.
#include "common.h"
#include "kernels.h"

namespace dory {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kNW = 8;    // waves (work items) per workgroup
constexpr int kNT = 64 * kNW;
constexpr int kKT = 64;   // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

// LDS of one tile buffer pair: K rows padded 16 B, V^T rows padded 8 B
template <int HD>
constexpr uint32_t attn_pf_lds() { return 2u * (kKT * (HD + 8) + HD * (kKT + 4)) * 2u; }

template <int HD>
__global__ __launch_bounds__(kNT, 1) void k_attn_prefill(AttnArgs a, const float* __restrict__ qkvg, int64_t ld,
                                                        int gate_off, int gate, bf16* __restrict__ ob) {
  constexpr int CPK = HD / 8;          // 16-byte chunks per key row
  constexpr int NL = HD / 64;          // K chunks (and V runs) per thread per tile
  constexpr int KLD = HD + 8;          // K tile row, padded 16 B (conflict-free 16-byte reads)
  constexpr int VLD = kKT + 4;         // V^T tile row, padded 8 B (conflict-free 8-byte reads)
  constexpr int NKS = HD / 16;         // S steps
  constexpr int NMB = HD / 32;         // O^T row blocks
  constexpr int KSZ = kKT * KLD, VSZ = HD * VLD;
  extern __shared__ __align__(16) bf16 lds[];  // [buffer][K tile | V^T tile]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: item bounds in scalar registers
  const int lq = lane & 31, g = lane >> 5;
  const int G = a.nq / a.nkv;

  // ---- work: item block (most keys first) and (sequence, kv head)
  const int p0 = a.p0, n = a.n, W = a.window, full = a.is_full;
  const int items = ((n + 31) / 32) * G;
  const int nwb = (items + kNW - 1) / kNW;
  const int BK = a.B * a.nkv;
  if ((int)blockIdx.x >= nwb * BK) return;
  const int wb = nwb - 1 - (int)blockIdx.x / BK;
  const int b = ((int)blockIdx.x % BK) / a.nkv, kvh = (int)blockIdx.x % a.nkv;
  const int item0 = wb * kNW, item1 = min(item0 + kNW, items) - 1;
  const int lo_blk = full ? 0 : max(0, p0 + (item0 / G) * 32 - W + 1);  // keys any item of the block may see
  const int hi_blk = p0 + min((item1 / G) * 32 + 31, n - 1);

  // ---- this wave's item (a wave past the last item stages tiles only)
  const bool wave_live = item0 + wave < items;
  const int item = min(item0 + wave, items - 1);
  const int hq = kvh * G + item % G;
  const int iw0 = (item / G) * 32;
  const int ta = p0 + iw0, tb = p0 + min(iw0 + 31, n - 1);
  const int wlo = full ? 0 : max(0, ta - W + 1);
  const int iq = min(iw0 + lq, n - 1);  // clamped: rows past n are computed and dropped
  const int t = p0 + iq;

  const bf16* q = (const bf16*)a.q;
  const bf16* kw = (const bf16*)a.kw;
  const bf16* vw = (const bf16*)a.vw;
  const bf16* kc = (const bf16*)a.kc;
  const bf16* vc = (const bf16*)a.vc;

  // Q^T operand: lane (query lq, half g) holds dims 16*ks + 8*g .. +7
  bf16x8_t qf[NKS];
  {
    const bf16* qr = q + ((size_t)(b * n + iq) * a.nq + hq) * HD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8_t*)(qr + 16 * ks);
  }

  // ---- tile loader: unconditional 16-byte loads from clamped addresses (so
  // the waits stay exact); what must read as zero, or needs a per-key gather,
  // is decided again when the registers go to LDS
  const size_t khead = ((size_t)b * a.nkv + kvh) * a.slots;
  const size_t vhead_c = ((size_t)b * a.nkv + kvh) * HD * vslots_of(a.slots);  // cache values (32-position blocks)
  const size_t vhead_w = ((size_t)b * a.nkv + kvh) * HD * a.vld;    // this call's V^T rows
  const bool vec_chunk = (p0 & 7) == 0;
  const bool vec_cache = full || (W & 7) == 0;  // 8-aligned runs stay inside one 32-position block
  auto slot_of = [&](int s) { return full ? s : s % W; };
  auto key_src = [&](int s) -> const bf16* {  // K row of key s (clamped into the block's range)
    s = min(max(s, lo_blk), hi_blk);
    return s >= p0 ? kw + ((size_t)(b * n + (s - p0)) * a.nkv + kvh) * HD : kc + (khead + slot_of(s)) * HD;
  };
  // V run mode: 0 = vector (one source, contiguous), 1 = zero, 2 = per-key gather
  auto run_mode = [&](int s) -> int {
    if (s + 7 < lo_blk || s > hi_blk) return 1;
    if (s < lo_blk || s + 7 > hi_blk) return 2;
    if (s >= p0) return vec_chunk ? 0 : 2;
    if (s + 7 < p0) return (vec_cache && (full || slot_of(s) + 8 <= W)) ? 0 : 2;
    return 2;
  };
  auto v_src = [&](int d, int s) -> const bf16* {  // vector path source (or any aligned address)
    if (run_mode(s) != 0) return vc;
    return s >= p0 ? vw + vhead_w + (size_t)d * a.vld + (s - p0) : vc + vhead_c + vt_off(slot_of(s), d, HD);
  };
  auto v_elem = [&](int d, int s) -> bf16 {  // one value of key s (zero outside the block's range)
    if (s < lo_blk || s > hi_blk) return 0;
    return s >= p0 ? vw[vhead_w + (size_t)d * a.vld + (s - p0)] : vc[vhead_c + vt_off(slot_of(s), d, HD)];
  };

  // A plain tile (every key inside the block's range, and all from the cache
  // without a ring wrap, or all from this call with 8-aligned value runs)
  // has every address as a wave-uniform base plus a per-thread constant.
  // fetch always issues those loads (clamped in bounds, no branch around
  // them, so the waits stay exact); stage writes them to LDS for a plain
  // tile and otherwise re-reads the tile through the per-key path above
  // (edge tiles only: the block's first and last, the one holding p0).
  const int slots = a.slots, vslots = vslots_of(a.slots);
  const bool cache_plain = vec_cache && (full || W % kKT == 0);
  auto plain = [&](int s0) {
    if (s0 < lo_blk || s0 + kKT - 1 > hi_blk) return false;
    if (s0 >= p0) return vec_chunk;
    return s0 + kKT - 1 < p0 && cache_plain;
  };
  u32x4 kr[NL], vr[NL];
  auto fetch = [&](int s0) {
    const bool chunk = s0 >= p0;
    const int r0 = s0 - p0;
    const int slot0 = slot_of(s0);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + kNT * i;
      const int kk = e / CPK, c = e % CPK, d = e >> 3, run = e & 7;
      const bf16* kp = chunk ? kw + ((size_t)(b * n + min(r0 + kk, n - 1)) * a.nkv + kvh) * HD + 8 * c
                             : kc + (khead + min(slot0 + kk, slots - 1)) * HD + 8 * c;
      // value runs rounded down to 8 positions: 16-byte aligned (they are
      // used as loaded only when already aligned, i.e. in a plain tile)
      const bf16* vp = chunk ? vw + vhead_w + (size_t)d * a.vld + (min(r0 + 8 * run, a.vld - 8) & ~7)
                             : vc + vhead_c + vt_off(min(slot0 + 8 * run, vslots - 8) & ~7, d, HD);
      kr[i] = *(const u32x4*)kp;
      vr[i] = *(const u32x4*)vp;
    }
  };
  auto stage = [&](int s0, int buf) {
    bf16* const Ks = lds + buf * (KSZ + VSZ);
    bf16* const Vt = Ks + KSZ;
    if (plain(s0)) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int e = tid + kNT * i;
        *(u32x4*)(Ks + (e / CPK) * KLD + 8 * (e % CPK)) = kr[i];
        u32x2_t* dst = (u32x2_t*)(Vt + (e >> 3) * VLD + 8 * (e & 7));
        dst[0] = u32x2_t{vr[i][0], vr[i][1]};
        dst[1] = u32x2_t{vr[i][2], vr[i][3]};
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + kNT * i;
      const int kk = e / CPK, c = e % CPK;
      const int s = s0 + kk;
      u32x4 kv = *(const u32x4*)(key_src(s) + 8 * c);
      if (s < lo_blk || s > hi_blk) kv = u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(Ks + kk * KLD + 8 * c) = kv;
      const int d = e >> 3, run = e & 7;
      const int sv = s0 + 8 * run;
      const int mode = run_mode(sv);
      u32x4 vv = *(const u32x4*)v_src(d, sv);
      if (mode == 1) {
        vv = u32x4{0u, 0u, 0u, 0u};
      } else if (mode == 2) {
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          vv[w2] = (uint32_t)v_elem(d, sv + 2 * w2) | ((uint32_t)v_elem(d, sv + 2 * w2 + 1) << 16);
      }
      u32x2_t* dst = (u32x2_t*)(Vt + d * VLD + 8 * run);
      dst[0] = u32x2_t{vv[0], vv[1]};
      dst[1] = u32x2_t{vv[2], vv[3]};
    }
  };

  // q and k are unit vectors, so no score exceeds the scale: with sl2 at most
  // 40 the exponents are referenced to that bound (softmax is unchanged by
  // the shift, and 2^(-2 sl2) is still a normal bfloat16), which needs no
  // running max and no rescaling; above it, the usual online max.
  const float sl2 = a.scale * kLog2e;
  const bool fixed_ref = sl2 <= 40.f;
  float m = fixed_ref ? sl2 : -1e30f, l = 0.f;
  f32x16_t acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  const int T0 = lo_blk / kKT, T1 = hi_blk / kKT;
  fetch(T0 * kKT);
  stage(T0 * kKT, 0);
  __syncthreads();
  fetch(min(T0 + 1, T1) * kKT);  // (a single tile refetches itself: exact waits)
  for (int T = T0; T <= T1; ++T) {
    const int s0 = T * kKT;
    const int buf = (T - T0) & 1;
    const bf16* const Ks = lds + buf * (KSZ + VSZ);
    const bf16* const Vt = Ks + KSZ;
    // the wave's work on this tile, then tile T+1 into the other buffer (last
    // read in iteration T-1, which every wave finished before the barrier
    // that ended it), then one barrier publishes it
    if (wave_live && s0 <= tb && s0 + kKT - 1 >= wlo) {
      // masks needed unless every key of the tile is allowed for every query of the wave
      const bool edge = s0 + kKT - 1 > ta || (!full && s0 < tb - W + 1);

      // the two halves' score products alternate (two independent chains)
      f32x16_t sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
      const bf16* kr0 = Ks + lq * KLD + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)(kr0 + kt * 32 * KLD + 16 * ks), qf[ks],
                                                           sc[kt], 0, 0, 0);
      // register r of half tile kt holds key s0 + 32 kt + 8 (r / 4) + 4 g + r % 4.
      // Masks only on edge tiles (a wave-uniform branch), as selects; a masked
      // score (-inf) gives p = 2^-inf = 0 since the reference m is finite (the
      // bound sl2, or a running max that starts at -1e30 and is taken on the
      // raw scores, sl2 > 0).
      float tmax = -INFINITY;
      if (edge) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = s0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool ok = (key <= t) & (full | (key > t - W));
            sc[kt][r] = ok ? sc[kt][r] : -INFINITY;
            tmax = fmaxf(tmax, sc[kt][r]);
          }
      } else if (!fixed_ref) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sc[kt][r]);
      }
      float mn = m;
      if (!fixed_ref) {
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        mn = fmaxf(m, tmax * sl2);
      }
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      // p = 2^(s sl2 - m) in bfloat16 (the P.V operand); the row sum adds the
      // rounded values two at a time
      float ps = 0.f;
      bf16x8_t pb[2][2];
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
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
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // the max moved for some query of the wave
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const bf16* vrow = Vt + (mb * 32 + lq) * VLD + 32 * kt + 16 * h + 4 * g;
            const u32x2_t lo = *(const u32x2_t*)vrow;
            const u32x2_t hi = *(const u32x2_t*)(vrow + 8);
            const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)&va, pb[kt][h], acc[mb], 0, 0, 0);
          }
    }
    if (T < T1) {
      stage(s0 + kKT, buf ^ 1);
      __syncthreads();
      fetch(min(T + 2, T1) * kKT);  // in flight while tile T+1 is multiplied
    }
  }

  // ---- normalise, gate, store: register r of block mb holds dim
  // 32 mb + 8 (r / 4) + 4 g + r % 4 of query lq
  if (!wave_live || iw0 + lq >= n) return;
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.0f / lt;
  const int row = b * n + iq;
  const float* gr = qkvg + (size_t)row * ld + gate_off;
  bf16* dst = ob + ((size_t)row * a.nq + hq) * HD;
  const float gh = gate == 2 ? sigmoidf_(gr[hq]) : 1.f;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * mb + 8 * rq + 4 * g;
      float gv[4] = {gh, gh, gh, gh};
      if (gate == 1) {
        const float4 g4 = *(const float4*)(gr + hq * HD + d0);
        gv[0] = sigmoidf_(g4.x);
        gv[1] = sigmoidf_(g4.y);
        gv[2] = sigmoidf_(g4.z);
        gv[3] = sigmoidf_(g4.w);
      }
      const bf16 o0 = from_f<bf16>(acc[mb][4 * rq + 0] * inv * gv[0]);
      const bf16 o1 = from_f<bf16>(acc[mb][4 * rq + 1] * inv * gv[1]);
      const bf16 o2 = from_f<bf16>(acc[mb][4 * rq + 2] * inv * gv[2]);
      const bf16 o3 = from_f<bf16>(acc[mb][4 * rq + 3] * inv * gv[3]);
      *(u32x2_t*)(dst + d0) = u32x2_t{(uint32_t)o0 | ((uint32_t)o1 << 16), (uint32_t)o2 | ((uint32_t)o3 << 16)};
    }
}

}  // namespace

// dtype 1 = bfloat16
bool attn_prefill_supported(int dtype, int hd, int nq, int nkv) {
  return dtype == 1 && (hd == 64 || hd == 128) && nkv > 0 && nq % nkv == 0;
}

hipError_t launch_attn_prefill(const AttnArgs& a, const float* qkvg, int64_t ld, int gate_off, int gate, void* ob,
                               hipStream_t st) {
  if (a.B * a.n <= 0) return hipSuccess;
  if (!attn_prefill_supported(1, a.hd, a.nq, a.nkv)) return hipErrorInvalidValue;
  if ((gate_off & 3) || (ld & 3)) return hipErrorInvalidValue;  // float4 gate reads
  const int G = a.nq / a.nkv;
  const int64_t items = (int64_t)((a.n + 31) / 32) * G;
  const int64_t blocks = (items + kNW - 1) / kNW * a.B * a.nkv;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.hd == 64) {
    dory_launch(k_attn_prefill<64>, dim3((unsigned)blocks), dim3(kNT), attn_pf_lds<64>(), st, a, qkvg, ld, gate_off,
                gate, (bf16*)ob);
  } else {
    // the double-buffered tiles of head dim 128 need more than the 64 KB of
    // LDS a launch gets by default (set once per process)
    static const hipError_t attr = hipFuncSetAttribute((const void*)k_attn_prefill<128>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)attn_pf_lds<128>());
    if (attr != hipSuccess) return attr;
    dory_launch(k_attn_prefill<128>, dim3((unsigned)blocks), dim3(kNT), attn_pf_lds<128>(), st, a, qkvg, ld,
                gate_off, gate, (bf16*)ob);
  }
  return hipGetLastError();
}

}  // namespace dory
