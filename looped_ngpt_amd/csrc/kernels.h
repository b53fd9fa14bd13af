// Launch wrappers of the gfx950 kernels. Plain pointers and sizes; every
// wrapper enqueues on `st` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dory {

// Timing tap: events that the next launch of a kernel wrapper on this host
// thread records as part of its dispatch (hipExtLaunchKernel), so that the
// pair brackets that kernel alone. Consumed by one launch.
struct LaunchEvents { hipEvent_t start, stop; };
void set_next_launch_events(hipEvent_t start, hipEvent_t stop);
LaunchEvents take_next_launch_events();  // and clears them

// Mixed loop counts: row r of a launch belongs to sequence r / n, which runs
// loops[r / n] passes of the recurrent block. At pass `loop` a row whose count
// has passed is left untouched (its residual and bf16 copy keep the value of
// its own last pass). loops == NULL: every row is active.
struct RowGate {
  const int* loops;
  int loop, n;
};

// h = norm(E[tok]) per row; xb = h in the model dtype; h2 (optional) = h.
hipError_t launch_embed(int dtype, const int32_t* tok, const void* E, float* h, float* h2, void* xb,
                        int rows, int d, int vocab, int* err, hipStream_t st);

// nGPT step per row: h = norm(h + alpha * (norm(y) - h)); xb = h (dtype); h2 (optional) = h.
// y1 (optional): y is the sum y + y1 of a split product's two halves.
hipError_t launch_update(int dtype, float* h, const float* y, const float* alpha, void* xb, float* h2,
                         int rows, int d, hipStream_t st, RowGate gate = RowGate{nullptr, 0, 1},
                         const float* y1 = nullptr);

// Loop re-injection per row: h = norm(wh * h + we * e); xb = h (dtype).
hipError_t launch_combine(int dtype, float* h, const float* e, float wh, float we, void* xb, int rows,
                          int d, hipStream_t st, RowGate gate = RowGate{nullptr, 0, 1});

// dst[i] = loops[i], i < n (n <= 64 per launch).
struct RowLoops {
  int n;
  int k[64];
};
hipError_t launch_set_rows(int* dst, const RowLoops& a, hipStream_t st);

// tab[pos][i] = (cos, sin)(pos * base^(-2i/hd)), angles in float64.
hipError_t launch_rope_table(float2* tab, int max_ctx, int hd, double base, hipStream_t st);

// Rows r = b*n + i at position p0 + i. Reads q|k|v of the fused projection
// (float32, row stride ld); writes RoPE'd, per-head unit q and k and plain v
// in the model dtype to q_out [rows][nq][hd], k_out [rows][nkv][hd] and,
// transposed, v_out [B][nkv][hd][vld] (position i at column i).
// If kc is not NULL also writes k, v to the cache slot of each position
// (only valid when no other position of the same launch maps to that slot).
// a multi-position call's q / k (RoPE + per-head norm) into q_out / k_out
// (rows of [heads][hd]) and its values into v_out ([B][nkv][hd][vld], V^T per
// kv head, zeros from n to vld); rows = B * n, hd <= 128
struct RopeArgs {
  const float* qkvg; int64_t ld;
  const float2* tab;
  int p0, B, n, rows, nq, nkv, hd, vld;
  void* q_out; void* k_out; void* v_out;
};
hipError_t launch_rope_qk(int dtype, const RopeArgs& a, hipStream_t st);

// Copies this call's keys and values (kw rows, vw transposed with row length
// vld) into the cache: every position of a full layer, the last
// min(n, slots) positions of a sliding-window ring. wloops (optional, per
// sequence): sequence b is written only when wloops[b] == loop (its last pass).
hipError_t launch_kv_write(int dtype, const void* kw, const void* vw, int vld, void* kc, void* vc, int B, int n,
                           int p0, int nkv, int hd, int slots, int window, int is_full, hipStream_t st,
                           const int* wloops = nullptr, int loop = 0);

// Split-K softmax attention. For query row r = b*n + i (position p0 + i) and
// query head hq (kv head hq / G) the allowed keys are s <= t (and t - s <
// window for sliding layers); keys s >= p0 come from kw / vw (vw transposed,
// row length vld), earlier ones from the cache. Writes (m, l, acc[hd]) per
// (r, hq, split) to part.
struct AttnArgs {
  const void* q; const void* kw; const void* vw; const void* kc; const void* vc;
  int B, n, p0, nq, nkv, hd, slots, window, is_full, n_split, vld;
  float scale;
  float* part;
};
hipError_t launch_attn_split(int dtype, const AttnArgs& a, hipStream_t st);

// Prefill attention on the matrix cores (bfloat16, hd 64 or 128): the same
// keys and softmax as launch_attn_split with one split, followed by what
// launch_attn_combine does (normalise, sigmoid gate read at gate_off of the
// projection rows, store ob [rows][nq*hd]) in one launch.
hipError_t launch_attn_prefill(const AttnArgs& a, const float* qkvg, int64_t ld, int gate_off, int gate, void* ob,
                               hipStream_t st);
bool attn_prefill_supported(int dtype, int hd, int nq, int nkv);

// Merges the splits, applies the sigmoid gate (gate 1: elementwise, 2: per
// head, 0: none) read from the fused projection, stores ob [rows][nq*hd] (dtype).
hipError_t launch_attn_combine(int dtype, const float* part, const float* qkvg, int64_t ld, int gate_off,
                               int gate, void* ob, int rows, int nq, int hd, int n_split, hipStream_t st);

// Decode attention for one new position t of B sequences (all at position t),
// fused with RoPE and the q/k normalisation: every workgroup (key split,
// sequence x kv head) builds its G query heads from the fused projection; the
// workgroup whose split holds t also builds the new key/value (and writes
// them to the cache slot of t when write_kv). Keys s < t come from the cache.
// Writes partials (m in log2 units, l, acc[hd]) per (b, q head, split).
// The position t of the new key is read from t_dev, so one recorded graph
// serves every step; n_split is fixed by capacity and the kernel spreads the
// actual key range over it (trailing splits may be empty).
// wloops (optional, per sequence): with write_kv, sequence b writes its new
// key/value only when wloops[b] == loop (mixed loop counts, its last pass).
struct AttnDecArgs {
  const float* qkvg; int64_t ld;
  const float2* tab;
  const int* t_dev;
  int t_now;  // position of the new key if >= 0 (eager calls), else read *t_dev
  int B, nq, nkv, hd, slots, window, is_full, write_kv, n_split;
  float scale;
  void* kc; void* vc;
  float* part;
  const int* wloops; int loop;
  // optional (matrix-core kernel): instead of per-split partials, add the
  // split's sums as fixed point with 64-bit integer atomics (order-
  // independent, hence deterministic) into acc. The sums are referenced to
  // the largest possible score (q and k are unit vectors, so a score never
  // exceeds `scale`); a workgroup whose sum p lies in [2^(-16(b+1)),
  // 2^(-16b)) takes bin b (b < acc_nb; b = 0 from 2^-16 up), where one unit
  // is 2^-(36 + 16b), so its largest term keeps at least 21 bits however far
  // below the bound every score lies. Layout per (row, q head):
  // acc_nb x hd words of sum p v times the sigmoid gate (read at gate_off of
  // the projection row; gate 1 elementwise, 2 per head, 0 none), bin-major,
  // then 8 words whose first acc_nb hold sum p per bin (the rest stay zero).
  // acc must start at zero.
  unsigned long long* acc;
  int acc_nb;
  int gate_off, gate;
};
constexpr int kAttnAccPad = 8;       // words per (row, head) beyond the bins' value words
constexpr int kAttnAccBinsMax = 4;   // sum-p words fit in the pad; covers scale log2(e) < 32
constexpr int kAttnAccBinBits = 16;  // binary orders of magnitude per bin
// words per (row, q head) of the accumulators
__host__ __device__ inline int attn_acc_stride(int hd, int nb) { return nb * hd + kAttnAccPad; }
// bins the accumulators need for the softmax scale `scale` (every sum p of a
// workgroup is >= its largest term >= 2^(-2 scale log2 e)); 0 when more than
// kAttnAccBinsMax would be needed (the float split + merge path then runs)
int attn_acc_bins(float scale);
hipError_t launch_attn_decode(int dtype, const AttnDecArgs& a, hipStream_t st);
// True when launch_attn_decode takes the matrix-core kernel, which splits the
// keys in tiles of 32 positions (bfloat16, slots and window multiples of 4).
bool attn_decode_uses_mfma(int dtype, int hd, int slots, int window, int is_full);

// Merges the decode partials (log2 units), applies the sigmoid gate (gate 1
// elementwise, 2 per head, 0 none; read at gate_off of the projection row),
// stores the gated heads in ob [B][nq*hd]. One workgroup per (q head, row).
// (Merging inside the attention kernel by its last workgroup measured slower
// on gfx950 than this separate launch, both with device-scope fences and with
// coherent stores and loads of the partials.)
hipError_t launch_attn_merge(int dtype, const float* part, const float* qkvg, int64_t ld, int gate_off, int gate,
                             void* ob, int B, int nq, int hd, int n_split, hipStream_t st);

// The output projection fed straight from the decode attention accumulators
// (AttnDecArgs::acc): input element (row m, head h, dim d) = (gated sum p v)
// / (sum p), rounded to bfloat16 — the merge folded into the GEMV's
// activation staging. (The concat norm before W_o is left out: the update
// only sees norm(y), and norm(c W x) = norm(W x).)
// waves per workgroup of the one-output-per-wave GEMVs for `nout` outputs
int rows_waves(int nout);

struct AttnX {
  const unsigned long long* acc;
  int hd; int nq; int nb;  // accumulators as AttnDecArgs::acc with acc_nb = nb
};
hipError_t launch_zero_u64(unsigned long long* p, int64_t n, hipStream_t st);
// a[M][F] = (scale u) silu(scale v) from a bfloat16 projection [M][2F] (u | v per row); F % 8 == 0
hipError_t launch_swiglu_rows(const void* p, int M, int F, float scale, void* a, hipStream_t st);
// bfloat16 weights W [N][K = nq*hd], M <= 8 rows, y float32 [M][N] * scale
hipError_t launch_linear_attn(const AttnX& ax, const void* W, float* y, int M, int N, int K, float scale,
                              hipStream_t st);
bool linear_attn_supported(int M, int K);
// the same for low-bit weights (fmt as launch_linear_lowbit)
hipError_t launch_linear_lowbit_attn(int fmt, const AttnX& ax, const void* Wq, const void* Ws, float* y, int M, int N,
                                     int K, float scale, hipStream_t st);

// y = x . W^T (see dory_op_linear): GEMVs up to 8 rows (algo 0), else launch_gemm.
hipError_t launch_linear(int dtype, const void* x, int64_t ldx, const void* W, void* y, int M, int N, int K,
                         int epi, float scale, int algo, hipStream_t st);
// the matrix-core GEMMs of launch_linear (any M; meant for M > 8)
hipError_t launch_gemm(int dtype, const void* x, int64_t ldx, const void* W, void* y, int M, int N, int K, int epi,
                       float scale, hipStream_t st);
// The contraction of a float32-output bfloat16 GEMM in two halves that one
// launch runs side by side: y0 = x[:, :K/2] . W[:, :K/2]^T and
// y1 = x[:, K/2:] . W[:, K/2:]^T (y0 + y1 is the product). For large-M shapes
// whose output tiles alone fill at most half of the CUs (gemm_split2_pays).
// Needs K % 128 == 0 and 16-byte aligned operands, else hipErrorInvalidValue.
bool gemm_split2_pays(int dtype, int M, int N, int K);
// 9..64 rows (batched decode), bfloat16, float32 out: the batched-decode GEMM
// with its contraction in two halves side by side, y0 = x[:, :K/2] . W[:, :K/2]^T
// and y1 = the rest (the reader adds y0 + y1), when its output tiles alone
// leave CUs idle (gemm_skinny_split2_pays). K % 128 == 0.
bool gemm_skinny_split2_pays(int dtype, int M, int N, int K);
hipError_t launch_gemm_skinny_split2(const void* x, int64_t ldx, const void* W, float* y0, float* y1, int M, int N,
                                     int K, float scale, hipStream_t st);
hipError_t launch_gemm_split2(const void* x, int64_t ldx, const void* W, float* y0, float* y1, int M, int N, int K,
                              float scale, hipStream_t st);

// Decode GEMV whose input row is produced in its own prologue: every
// workgroup first issues its weight loads, then computes for each of the M
// rows   u = norm(h_in + alpha * (norm(y) - h_in))            (nGPT update)
//        x = e ? norm(wh * u + we * e) : u                    (loop re-injection)
// in float32, stages bfloat16(x) in LDS and multiplies. Workgroup 0 writes x
// to h_out (the new residual) and, if e_out, u to e_out. bfloat16 only,
// M <= 8, K = d_model <= 8192. Returns hipErrorInvalidValue when unsupported.
struct GemvPro {
  const float* y; const float* h_in; const float* alpha; const float* e;
  float wh, we;
  float* h_out; float* e_out;
  unsigned long long* zero; int zero_n;  // optional: cleared by the workgroups (decode attention accumulators)
};
hipError_t launch_linear_pro(const GemvPro& p, const void* W, void* y, int M, int N, int K, int epi, float scale,
                             hipStream_t st);
bool linear_pro_supported(int M, int K);

// Low-bit weights of the layer projections; fmt is a dory_weight_format
// (1: MXFP8 — E4M3 codes [N][K], E8M0 scales [N][K/32]; 2: NVFP4-style —
// E2M1 codes [N][K/2], E4M3 scales [N][K/16], a float32 tensor scale applied
// through `scale`).
hipError_t launch_quant_mxfp8(const void* W_bf16, int N, int K, void* q, void* s, hipStream_t st);
// tscale: one device float, receives the tensor scale g
hipError_t launch_quant_nvfp4(const void* W_bf16, int N, int K, void* q, void* s, float* tscale, hipStream_t st);
// codes -> bfloat16 (MXFP8: the weights; NVFP4: e2m1 * e4m3, g left to the GEMM's scale)
hipError_t launch_dequant_lowbit(int fmt, const void* q, const void* s, int N, int K, void* W_bf16, hipStream_t st);
// decode GEMV (M <= 8): y = scale * x . W^T; SwiGLU: u = scale * x . W_u^T, v likewise
hipError_t launch_linear_lowbit(int fmt, const void* x, int64_t ldx, const void* Wq, const void* Ws, void* y, int M,
                                int N, int K, int epi, float scale, hipStream_t st);
bool linear_lowbit_supported(int fmt, int M, int K);
// launch_linear_pro for low-bit weights
hipError_t launch_linear_pro_lowbit(int fmt, const GemvPro& p, const void* Wq, const void* Ws, void* y, int M, int N,
                                    int K, int epi, float scale, hipStream_t st);
bool linear_pro_lowbit_supported(int fmt, int M, int K);

// partials (float2) held by the library for dory_op_argmax_noalloc: 64 KiB
// per GPU, batch x ceil(V / 1024) <= 8192 (batch 64 at a 131,072 vocabulary)
constexpr int kArgmaxNoAllocPartials = 8192;
// Greedy argmax; if pos_dev is not NULL the final pass also advances the
// device position counter by one (the end of a decode step).
hipError_t launch_argmax(const float* logits, int B, int V, int32_t* out, void* scratch, hipStream_t st,
                         int* pos_dev = nullptr);

// *pos_dev = value (one thread).
hipError_t launch_set_pos(int* pos_dev, int value, hipStream_t st);


// ---- depth-1 truncated backward (k_backward.hip); float32 unless a dtype
// `dt` (0 float32, 1 bfloat16) names the GEMM operand copies ----
struct BwAttn {
  const float* qn;   // [M][nq*hd] normalised, rotated queries
  const float* kn;   // [M][nkv*hd]
  const float* v;    // values: row r at v + r*ldv
  int ldv;
  int n, nq, nkv, hd;
  int window;        // 0: full causal
  float scale;
};
// Matrix-core attention of the backward (bfloat16 models, hd 64 / 128):
// head-major bfloat16 operand copies Q, K, V, dO [B][H][n][hd] and
// transposed ones QT, KT, VT, dOT [B][H][hd][nT] (nT = n rounded up to 8,
// zero past n); softmax statistics mst / lst and D [B*n][nq] (float32); o,
// dq [B*n][nq*hd] and dk, dv [B*n][nkv*hd] float32 rows.
struct BwFlash {
  const uint16_t *Q, *K, *V, *dO, *QT, *KT, *VT, *dOT;
  int B, n, nT, nq, nkv, hd, window;  // window 0: full causal
  float scale;
  float *mst, *lst;
  const float* D;
  float *o, *dq, *dk, *dv;
  float *dkh, *dvh;  // [B n][nq][hd] per-query-head partial dk, dv (scratch of the backward pass)
};
bool bw_flash_supported(int dtype, int hd, int nq, int nkv);
// dst [B][H][hd][nT] bfloat16 (zero past n) from float32 rows src[(b n + t) ld + off + h hd + d]
hipError_t launch_bw_heads_t(const float* src, int64_t ld, int off, int H, int hd, int n, int B, int nT, void* dst,
                             hipStream_t st);
// o, mst, lst from Q, K, VT
hipError_t launch_bw_flash_fwd(const BwFlash& a, hipStream_t st);
// dq from Q, dO, K, V, KT; dk, dv from K, V, Q, dO, QT, dOT (and mst, lst, D)
hipError_t launch_bw_flash_bwd(const BwFlash& a, hipStream_t st);
hipError_t launch_bw_cast(int dt_out, const float* in, void* out, int64_t n, hipStream_t st);
hipError_t launch_bw_transpose(int dt, const void* in, int64_t ld, void* out, int R, int C, hipStream_t st);
// out = a + b, or a + (b + b2) with b2 (the two partial sums of a split product)
hipError_t launch_bw_add(const float* a, const float* b, float* out, int64_t n, hipStream_t st,
                         const float* b2 = nullptr);
// out[j] = sum over the M rows of in[r][j]; part: scratch of ceil(M/64) * d floats
hipError_t launch_bw_colsum(const float* in, int M, int d, float* out, float* part, hipStream_t st);
// y2: optional second partial sum of y (y + y2 is the sublayer output)
hipError_t launch_bw_update_fwd(int dt, const float* h, const float* y, const float* alpha, int M, int d, float* yh,
                                float* ry, float* rz, float* hout, void* hout_t, hipStream_t st,
                                const float* y2 = nullptr);
hipError_t launch_bw_rope_norm_fwd(const float* P1, int ldp, const float2* tab, int n, int nq, int nkv, int hd, int M,
                                   float* qn, float* kn, float* rq, float* rk, hipStream_t st);
hipError_t launch_bw_attn_fwd(const BwAttn& a, int M, float* o, float* mst, float* lst, hipStream_t st);
hipError_t launch_bw_gate_fwd(int dt, const float* o, const float* P1, int ldp, int goff, int mode, int hd, int qd,
                              int M, float* oh, void* oh_t, float* rc, hipStream_t st);
hipError_t launch_bw_swiglu_fwd(int dt, const float* P2, int F, int M, float* a32, void* a_t, float* rs,
                                hipStream_t st);
hipError_t launch_bw_final(const float* h, const float* G, int M, int d, float* dh, hipStream_t st);
hipError_t launch_bw_update_bwd(int dt, const float* dho, const float* ho, const float* rz, const float* yh,
                                const float* ry, const float* h, const float* alpha, int M, int d, float* dres,
                                void* dy_t, float* contrib, hipStream_t st);
hipError_t launch_bw_swiglu_bwd(int dt, const float* da, const float* a32, const float* rs, const float* P2, int F,
                                int M, void* dP2, hipStream_t st);
// doh2: optional second partial sum of doh
hipError_t launch_bw_gate_bwd(const float* doh, const float* oh, const float* rc, const float* o, const float* P1,
                              int ldp, int goff, int mode, int hd, int qd, int M, float* dO, float* dP1,
                              hipStream_t st, const float* doh2 = nullptr);
hipError_t launch_bw_attn_bwd(const BwAttn& a, int M, const float* dO, const float* o, const float* mst,
                              const float* lst, float* D, float* dqn, float* dkn, float* dv, hipStream_t st);
// dst [B][H][n][hd] (dt: 0 float32, 1 bfloat16) from float32 rows src[(b n + t) ld + off + h hd + d]
hipError_t launch_bw_to_heads(int dt, const float* src, int64_t ld, int off, int H, int hd, int n, int B, void* dst,
                              hipStream_t st);
hipError_t launch_bw_attn_D(const float* dO, const float* o, int nq, int hd, int M, float* D, hipStream_t st);
hipError_t launch_bw_rope_norm_bwd(const float* dqn, const float* qn, const float* rq, const float* dkn,
                                   const float* kn, const float* rk, const float* dv, const float2* tab, int n, int nq,
                                   int nkv, int hd, int M, float* dP1, int ldp, hipStream_t st);

}  // namespace dory
