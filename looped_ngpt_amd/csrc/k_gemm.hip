// Matrix-core GEMMs y = x . W^T for the projections of the looped nGPT at
// more than 8 rows (prefill chunks, batched decode, the backward's gradient
// products). x is [M][K] (row stride ldx), W is [N][K] (row-major, the
// nn.Linear layout), y is [M][N] float32, or [M][N/2] in the model dtype with
// the SwiGLU epilogue (rows o and N/2 + o of W are the up and gate rows of
// output o; y = u * silu(v)).
//
//  * k_gemm_big: M >= 1024, bfloat16, K % 64 == 0. 256 x BN workgroup tiles
//    (BN 256 or 192), eight waves on v_mfma_f32_32x32x16_bf16, direct
//    global->LDS loads into a three / two slot ring, XCD-aware tile order.
//  * k_gemm_skinny: 9..64 rows (batched decode), weight-stream bound; the
//    narrow projections' contraction optionally in two halves side by side.
//  * k_gemm_mfma: the remaining bfloat16 shapes, 128 x 128 tiles.
//  * k_gemm_simple: float32 models and unaligned shapes.
#include "common.h"
#include "kernels.h"
#include "linear_common.h"

namespace dory {

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
// would leave the last round of workgroups half empty, e.g. N = 3072), eight
// waves, two per SIMD: a 2 x 4 grid of 128 x 64 wave tiles (BN = 256) or a
// 4 x 2 grid of 64 x 96 (BN = 192), accumulators of v_mfma_f32_32x32x16_bf16
// in registers (128 or 96 floats per lane).
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
// current one is multiplied: one LDS read before each of the first products,
// then the slice's direct global loads, one before each of the remaining
// products (sched_group_barrier), so the reads have most of the slice's
// products to land (reads after the loads, one after each product, measured
// 1-3.5% slower on three of the four prefill shapes).
//
// Workgroups are spread over the 8 XCDs in contiguous runs of tiles, grouped
// four M tiles at a time, so the tiles that run together on one XCD share A
// and B rows in its L2. The grid is one workgroup per CU at most and each
// walks its XCD's run (persistent): the next tile's first two stages go out
// before the current tile's stores, so a tile change waits for no launch and
// for little load latency (1-1.5% on the 8192-row shapes). SwiGLU (BN = 256 only): B tile rows come in 32-row
// chunks u, v, u, v of the same outputs, and a wave's two 32-column blocks
// are one (u, v) pair. Requires K % 64 == 0 and 16-byte aligned rows.
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

// Eight waves, two per SIMD (wave tiles of 128 x 64 for BN = 256, 64 x 96 for
// BN = 192; 128 or 96 accumulators per lane), so that one wave's products
// run while the other waits for its fragments (4-9% faster than four waves of
// 128 x 128 tiles, one per SIMD, at the same LDS traffic per stage).
template <int EPI, int BN>
__global__ __launch_bounds__(512) void k_gemm_big(const bf16* __restrict__ A, int64_t lda,
                                                   const bf16* __restrict__ B, void* __restrict__ C, int M, int N,
                                                   int K, float scale, int64_t ldb, void* __restrict__ C1) {
  static_assert(BN == 256 || (BN == 192 && EPI == EPI_F32), "tile widths");
  constexpr int WM = BN == 256 ? 2 : 4;  // waves along M
  constexpr int WN = 8 / WM;             // waves along N
  constexpr int TM = 256 / WM, TN = BN / WN;
  constexpr int MI = TM / 32, NJ = TN / 32;  // 32x32 blocks per wave
  constexpr int kHA = 256 * 128;       // A bytes per stage (32 KB)
  constexpr int kHB = BN * 128;        // B bytes per stage (32 or 24 KB)
  constexpr int kLA = kHA / 8192;      // 1 KB loads per wave per stage: A 4, B 4 or 3
  constexpr int kLB = kHB / 8192;
  extern __shared__ __align__(1024) unsigned char smem[];
  unsigned char* const sA = smem;             // 3 x kHA
  unsigned char* const sB = smem + 3 * kHA;   // 2 x kHB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int F = N / 2;
  const int nM = (M + 255) / 256;
  const int nN = EPI == EPI_SWIGLU ? (F + 127) / 128 : (N + BN - 1) / BN;
  const int nt = nM * nN;
  const int per = (nt + 7) / 8;
  // persistent: the workgroups of XCD x (blockIdx.x % 8) walk that XCD's run
  // of tiles x per .. x per + per - 1 in strides of the workgroups it holds
  const int xs = (int)(gridDim.x >> 3);
  const int tbase = (blockIdx.x & 7) * per, tend = min(tbase + per, nt);
  int t = tbase + (blockIdx.x >> 3);
  if (t >= tend) return;
  // split of the contraction (blockIdx.y): columns y K .. y K + K - 1 of A
  // and B, partial sums into C (y = 0) or C1 (y = 1)
  if (blockIdx.y) {
    A += (size_t)blockIdx.y * K;
    B += (size_t)blockIdx.y * K;
    C = C1;
  }
  const int lr = lane >> 3, ls = lane & 7;
  const bf16* srcA[kLA];
  const bf16* srcB[kLB];
  int m0, n0;
  // tile t: its corner and this thread's direct-load sources
  auto setup = [&](int tt) __attribute__((always_inline)) {
    const int grp = tt / (kBigGroupM * nN);
    const int gs = min(kBigGroupM, nM - grp * kBigGroupM);
    const int loc = tt - grp * kBigGroupM * nN;
    m0 = (grp * kBigGroupM + loc % gs) * 256;
    n0 = EPI == EPI_SWIGLU ? (loc / gs) * 128 : (loc / gs) * BN;
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
      srcB[i] = B + (size_t)wr * ldb + (ls ^ ((r >> 1) & 7)) * 8;
    }
  };
  setup(t);
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

  f32x16_t acc[MI][NJ];

  const int nK = K / kBigBK;
  const int l32 = lane & 31, lh = lane >> 5;
  auto frag = [&](int kt, int ks, bf16x8_t (&fa)[MI], bf16x8_t (&fb)[NJ]) {
    const unsigned char* a = sA + (kt % 3) * kHA;
    const unsigned char* b = sB + (kt & 1) * kHB;
    const int c = ks * 2 + lh;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = *(const bf16x8_t*)(a + big_off(wm * TM + i * 32 + l32, c));
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = *(const bf16x8_t*)(b + big_off(wn * TN + j * 32 + l32, c));
  };
  auto mma = [&](const bf16x8_t (&fa)[MI], const bf16x8_t (&fb)[NJ]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  bf16x8_t fa[2][MI], fb[2][NJ];
  auto issue01 = [&]() __attribute__((always_inline)) {
    issueA(0, 0, kLA);
    issueB(0);
    if (nK > 1) {
      issueA(1, 0, kLA);
      issueB(1);
    }
  };
  issue01();
  if (nK > 1) DORY_WAIT_VM(kLA + kLB); else DORY_WAIT_VM(0);
  for (;;) {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  frag(0, 0, fa[0], fb[0]);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  DORY_WAIT_LGKM0();
  constexpr int c0[3] = {0, kLA / 3, 2 * kLA / 3}, c1[3] = {kLA / 3, 2 * kLA / 3, kLA};
  for (int kt = 0; kt < nK; ++kt) {
    const bool moreA = kt + 2 < nK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) {
        if (moreA) issueA(kt + 2, c0[s], c1[s]);
        frag(kt, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
        mma(fa[s & 1], fb[s & 1]);
#pragma unroll
        for (int q = 0; q < MI + NJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_DS_RD, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < c1[s] - c0[s]; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_VMEM_RD, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
        }
      } else {
        if (moreA) DORY_WAIT_VM(kLA); else DORY_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 2 < nK) issueB(kt + 2);
        frag(kt + 1, 0, fa[0], fb[0]);  // unconditional (past the last stage: a stale slot, unused): exact waits
        mma(fa[1], fb[1]);
#pragma unroll
        for (int q = 0; q < MI + NJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_DS_RD, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < kLB; ++q) {
          __builtin_amdgcn_sched_group_barrier(DORY_SG_VMEM_RD, 1, 0);
          __builtin_amdgcn_sched_group_barrier(DORY_SG_MFMA, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      DORY_WAIT_LGKM0();
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the next tile's first two stages go out before this tile's stores (every
  // wave is past the last barrier, so no stage slot is still read)
  const int m0c = m0, n0c = n0;
  const int tn = t + xs;
  if (tn < tend) {
    setup(tn);
    issue01();
  }

  // C layout of a 32x32 block: register r of lane l -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0c + wm * TM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
        // this wave's blocks (0, 1) are the u and v rows of outputs n0 + wn * 32 + 0..31
        const int o = n0c + wn * 32 + l32;
        if (o < F)
          ((bf16*)C)[(size_t)row * F + o] = from_f<bf16>(acc[i][0][r] * scale * silu_(acc[i][1][r] * scale));
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = n0c + wn * TN + j * 32 + l32;
          if (col < N) ((float*)C)[(size_t)row * N + col] = acc[i][j][r] * scale;
        }
      }
    }
  }
  if (tn >= tend) break;
  t = tn;
  DORY_WAIT_VM(0);  // the next tile's stages (and this tile's stores)
  }
}

// LDS bytes of k_gemm_big (three A slots and two B slots of one stage)
static constexpr uint32_t big_lds(int bn) { return 3 * 256 * 128 + 2 * bn * 128; }

// k_gemm_big<EPI, BN> with its dynamic LDS above the 64 KB default allowed
// (set once per process)
template <int EPI, int BN>
static void big_launch(dim3 grid, const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K, float scale,
                       hipStream_t st, int64_t ldw, void* y1 = nullptr) {
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_gemm_big<EPI, BN>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)big_lds(BN));
  (void)attr;
  dory_launch((k_gemm_big<EPI, BN>), grid, dim3(512), big_lds(BN), st, x, ldx, W, y, M, N, K, scale, ldw, y1);
}

// tile width for a large-M GEMM with N outputs (run `splits` times over, one
// per part of the contraction): 192 when 256-wide tiles would leave the last
// round of workgroups (one per CU) at most half full and 192-wide ones do better
static int big_tile_n(int M, int N, int splits = 1) {
  auto eff = [&](int bn) {
    const long tiles = (long)splits * ((M + 255) / 256) * ((N + bn - 1) / bn);
    const long rounds = (tiles + kNumCUs - 1) / kNumCUs;
    return (double)tiles / (double)(rounds * kNumCUs) * (bn == 256 ? 1.0 : 0.93);  // 192: more LDS reads per FLOP
  };
  return eff(192) > eff(256) ? 192 : 256;
}

// ---------------------------------------------------------------------------
// Batched-decode GEMM (9..64 rows): weight-stream bound. A workgroup owns 16
// outputs (16 weight rows; SwiGLU: those 16 u rows and the 16 matching v
// rows) and all M rows (MB = 16, 32 or 64 staged, rows past M clamped). K
// goes in windows of 64: each window's X rows and weight rows are copied
// into LDS by direct global->LDS loads laid out like k_gemm_big's stages
// (one 1 KB load covers 8 rows x 128 B, whole cache lines, chunks
// XOR-swizzled by (row/2) % 8), in a ring of D windows so that D - 1
// windows are in flight while one is multiplied (one barrier per window).
// The loads of a window are spread over the four waves; each 16-row block of
// X is one wave's 16 x 16 output block (v_mfma_f32_16x16x32_bf16, two
// 32-deep steps per window), written straight from its accumulators.
// Every workgroup streams all of X (M x K) from L2 beside its 16 weight rows;
// operand loads taken straight from global memory in the MFMA layout (16
// rows per 16-lane group) ran the wide projections at about half this rate.
// A projection whose 16-output tiles leave CUs idle (N = 3072: 192 tiles) can
// run its contraction in two halves side by side (blockIdx.y; weight rows ldw
// apart, the second half's sums into C1), which its reader adds.
// Requires K % 64 == 0 and 16-byte aligned rows.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kStrBK = 64;

// s_waitcnt vmcnt(n) for a wave-uniform runtime n in [0, 63]
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
#define DORY_WV(i) \
  case i: DORY_WAIT_VM(i); break;
    DORY_WV(0) DORY_WV(1) DORY_WV(2) DORY_WV(3) DORY_WV(4) DORY_WV(5) DORY_WV(6) DORY_WV(7) DORY_WV(8)
    DORY_WV(9) DORY_WV(10) DORY_WV(11) DORY_WV(12) DORY_WV(13) DORY_WV(14) DORY_WV(15) DORY_WV(16)
    DORY_WV(17) DORY_WV(18) DORY_WV(19) DORY_WV(20) DORY_WV(21) DORY_WV(22) DORY_WV(23) DORY_WV(24)
    DORY_WV(25) DORY_WV(26) DORY_WV(27) DORY_WV(28) DORY_WV(29) DORY_WV(30) DORY_WV(31) DORY_WV(32)
    DORY_WV(33) DORY_WV(34) DORY_WV(35) DORY_WV(36) DORY_WV(37) DORY_WV(38) DORY_WV(39) DORY_WV(40)
    DORY_WV(41) DORY_WV(42) DORY_WV(43) DORY_WV(44) DORY_WV(45) DORY_WV(46) DORY_WV(47) DORY_WV(48)
#undef DORY_WV
    default: DORY_WAIT_VM(0); break;
  }
}

template <int MB, int EPI, int D>
__global__ __launch_bounds__(256) void k_gemm_skinny(const bf16* __restrict__ X, int64_t ldx,
                                                     const bf16* __restrict__ W, void* __restrict__ C, int M, int N,
                                                     int K, float scale, int64_t ldw, void* __restrict__ C1) {
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;  // weight blocks (u, v)
  constexpr int ROWS = MB + 16 * NR;             // window rows: X, then weights
  constexpr int NL = ROWS / 8;                   // 1 KB loads per window
  constexpr int LMAX = (NL + 3) / 4;             // loads per wave at most
  constexpr int WIN = ROWS * 128;                // window bytes
  static_assert(D >= 2 && (D - 2) * LMAX <= 48, "ring depth");
  extern __shared__ __align__(1024) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const int o0 = blockIdx.x * 16;
  const int nl = wave < NL ? (NL - wave + 3) / 4 : 0;  // this wave's loads per window (wave-uniform)
  // part blockIdx.y of a contraction split in two: columns y K .. y K + K - 1
  // of X and W (rows ldw apart), its sums into C (y = 0) or C1 (y = 1)
  if (blockIdx.y) {
    X += (size_t)K;
    W += (size_t)K;
    C = C1;
  }

  // load i of this wave fills window rows 8 (wave + 4 i) + 0..7
  const int lr = lane >> 3, ls = lane & 7;
  const bf16* src[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    const int r = min(8 * (wave + 4 * i) + lr, ROWS - 1);
    const bf16* base;
    if (r < MB) {
      base = X + (size_t)min(r, M - 1) * ldx;
    } else {
      const int wr = r - MB;
      const int o = min(o0 + (wr & 15), nout - 1);
      base = W + (size_t)((wr >= 16 ? nout : 0) + o) * ldw;
    }
    src[i] = base + (ls ^ ((r >> 1) & 7)) * 8;
  }
  const int nK = K / kStrBK;
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % D) * WIN;
#pragma unroll
    for (int i = 0; i < LMAX; ++i)
      if (i < nl) lds_load16(src[i] + kt * kStrBK, st + (wave + 4 * i) * 1024);
  };

  // wave w multiplies X rows 16w..16w+15 (waves past MB/16 only load)
  const bool active = wave < MB / 16;
  const int r16 = lane & 15, cq = lane >> 4;
  f32x4_t acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](int kt) {
    const unsigned char* st = smem + (kt % D) * WIN;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + cq;  // 16-byte chunk: K elements 32 s + 8 (lane / 16) ..
      const bf16x8_t a = *(const bf16x8_t*)(st + big_off(16 * wave + r16, c));
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const bf16x8_t w = *(const bf16x8_t*)(st + big_off(MB + 16 * j + r16, c));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc[j], 0, 0, 0);
      }
    }
  };

  const int pre = min(D - 1, nK);
  for (int kt = 0; kt < pre; ++kt) issue(kt);
  // steady state: window kt + D - 1 goes out while window kt is multiplied
  int kt = 0;
  for (; kt + D - 1 < nK; ++kt) {
    wait_vm_dyn(nl * (D - 2));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + D - 1);  // into the slot window kt - 1 used (every wave is past it)
    if (active) mul(kt);
    __builtin_amdgcn_sched_barrier(0);
  }
  // tail: no more loads
  for (; kt < nK; ++kt) {
    wait_vm_dyn(nl * (nK - 1 - kt));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (active) mul(kt);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!active) return;
  // D layout of a 16x16 block: register i of lane l -> row 4 (l / 16) + i, column l % 16
  const int o = o0 + r16;
  if (o >= nout) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 16 * wave + 4 * cq + i;
    if (m >= M) continue;
    if (EPI == EPI_SWIGLU)
      ((bf16*)C)[(size_t)m * nout + o] = from_f<bf16>(acc[0][i] * scale * silu_(acc[1][i] * scale));
    else
      ((float*)C)[(size_t)m * N + o] = acc[0][i] * scale;
  }
}

template <int MB, int EPI, int D>
static void skinny_launch_mb(dim3 grid, const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K,
                             float scale, hipStream_t st, int64_t ldw = -1, void* y1 = nullptr) {
  constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr uint32_t lds = D * (MB + 16 * NR) * 128;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_gemm_skinny<MB, EPI, D>,
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  dory_launch((k_gemm_skinny<MB, EPI, D>), grid, dim3(256), lds, st, x, ldx, W, y, M, N, K, scale,
              ldw < 0 ? (int64_t)K : ldw, y1);
}

// Ring depth in windows: 16 (one workgroup per CU) or 8 (two per CU) at 16 and
// 32 rows, 12 or 6 at 64 rows. Deeper rings measured slower (18-36 windows:
// -10 to -30%).
template <int MB, bool ONE>
constexpr int skinny_depth() {
  return MB == 64 ? (ONE ? 12 : 6) : (ONE ? 16 : 8);
}

template <int EPI>
static void skinny_launch(const bf16* x, int64_t ldx, const bf16* W, void* y, int M, int N, int K, float scale,
                          hipStream_t st) {
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const dim3 grid((nout + 15) / 16);
  // one workgroup per CU (a deep ring) below 512 workgroups, else two per CU
  const bool one = grid.x < 512;
#define DORY_SK(MB)                                                                                      \
  if (one) skinny_launch_mb<MB, EPI, skinny_depth<MB, true>()>(grid, x, ldx, W, y, M, N, K, scale, st); \
  else skinny_launch_mb<MB, EPI, skinny_depth<MB, false>()>(grid, x, ldx, W, y, M, N, K, scale, st);
  if (M <= 16) {
    DORY_SK(16)
  } else if (M <= 32) {
    DORY_SK(32)
  } else {
    DORY_SK(64)
  }
#undef DORY_SK
}

bool gemm_skinny_split2_pays(int dtype, int M, int N, int K) {
  // 16 outputs per workgroup: below one workgroup per CU the contraction
  // runs in two halves side by side (the N = 3072 projections: 192 -> 384
  // workgroups, 1.8-2x faster at 64 rows)
  return dtype == 1 && M > 8 && M <= 64 && N > 0 && (N + 15) / 16 < kNumCUs && K % (2 * kStrBK) == 0;
}

hipError_t launch_gemm_skinny_split2(const void* x, int64_t ldx, const void* W, float* y0, float* y1, int M, int N,
                                     int K, float scale, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool al16 = ldx % 8 == 0 && (((uintptr_t)x & 15) == 0) && (((uintptr_t)W & 15) == 0);
  if (!gemm_skinny_split2_pays(1, M, N, K) || !al16 || y0 == nullptr || y1 == nullptr) return hipErrorInvalidValue;
  const dim3 grid((N + 15) / 16, 2);
  const bf16* xb = (const bf16*)x;
  const bf16* wb = (const bf16*)W;
  // two workgroups per CU (the grid is below 512): the shallower ring
  if (M <= 16)
    skinny_launch_mb<16, EPI_F32, skinny_depth<16, false>()>(grid, xb, ldx, wb, y0, M, N, K / 2, scale, st, K, y1);
  else if (M <= 32)
    skinny_launch_mb<32, EPI_F32, skinny_depth<32, false>()>(grid, xb, ldx, wb, y0, M, N, K / 2, scale, st, K, y1);
  else
    skinny_launch_mb<64, EPI_F32, skinny_depth<64, false>()>(grid, xb, ldx, wb, y0, M, N, K / 2, scale, st, K, y1);
  return hipGetLastError();
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

template <typename T, int EPI>
static hipError_t gemm_dispatch(const T* x, int64_t ldx, const T* W, void* y, int M, int N, int K, float scale,
                                hipStream_t st) {
  const int nout = EPI == EPI_SWIGLU ? N / 2 : N;
  const bool al16 = ldx % 8 == 0 && (((uintptr_t)x & 15) == 0) && (((uintptr_t)W & 15) == 0);
  if (sizeof(T) == 2 && al16 && K % kBigBK == 0 && M >= 1024) {
    const int bn = EPI == EPI_SWIGLU ? 256 : big_tile_n(M, N);
    const int tiles = ((M + 255) / 256) * (EPI == EPI_SWIGLU ? (nout + 127) / 128 : (N + bn - 1) / bn);
    if (bn == 192)
      big_launch<EPI_F32, 192>(dim3(std::min((tiles + 7) / 8, kNumCUs / 8) * 8), (const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st, K);
    else
      big_launch<EPI, 256>(dim3(std::min((tiles + 7) / 8, kNumCUs / 8) * 8), (const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st, K);
  } else if (sizeof(T) == 2 && al16 && K % kStrBK == 0 && M <= 64) {
    skinny_launch<EPI>((const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st);
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

bool gemm_split2_pays(int dtype, int M, int N, int K) {
  if (dtype != 1 || M < 1024 || N <= 0 || K % (2 * kBigBK) != 0 || K / 2 < 16 * kBigBK) return false;
  const int bn = big_tile_n(M, N);
  const long tiles = (long)((M + 255) / 256) * ((N + bn - 1) / bn);
  return 2 * tiles <= kNumCUs;
}

hipError_t launch_gemm_split2(const void* x, int64_t ldx, const void* W, float* y0, float* y1, int M, int N, int K,
                              float scale, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool al16 = ldx % 8 == 0 && (((uintptr_t)x & 15) == 0) && (((uintptr_t)W & 15) == 0);
  if (!al16 || K % (2 * kBigBK) != 0 || y0 == nullptr || y1 == nullptr) return hipErrorInvalidValue;
  const int bn = big_tile_n(M, N, 2);
  const int tiles = ((M + 255) / 256) * ((N + bn - 1) / bn);
  const dim3 grid(std::min((tiles + 7) / 8, kNumCUs / 16) * 8, 2);
  if (bn == 192)
    big_launch<EPI_F32, 192>(grid, (const bf16*)x, ldx, (const bf16*)W, y0, M, N, K / 2, scale, st, K, y1);
  else
    big_launch<EPI_F32, 256>(grid, (const bf16*)x, ldx, (const bf16*)W, y0, M, N, K / 2, scale, st, K, y1);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, const void* x, int64_t ldx, const void* W, void* y, int M, int N, int K, int epi,
                       float scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (dtype == 0)
    return epi == EPI_SWIGLU ? gemm_dispatch<float, EPI_SWIGLU>((const float*)x, ldx, (const float*)W, y, M, N, K, scale, st)
                             : gemm_dispatch<float, EPI_F32>((const float*)x, ldx, (const float*)W, y, M, N, K, scale, st);
  return epi == EPI_SWIGLU ? gemm_dispatch<bf16, EPI_SWIGLU>((const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st)
                           : gemm_dispatch<bf16, EPI_F32>((const bf16*)x, ldx, (const bf16*)W, y, M, N, K, scale, st);
}

}  // namespace dory
