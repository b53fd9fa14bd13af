/*
 * dory.h - C ABI of the looped normalized-GPT forward pass on gfx950 (MI355X).
 *
 * The model. An input block of layers runs once, a shared recurrent block
 * runs n_loops = k times with the input block's output re-injected before
 * every pass, and an output block runs once ("Dory1.0-4B: A Looped
 * Normalized-GPT", ai.info summary, Key Contributions 1 and Methodology in
 * Plain English; goremy.ai blog "Dory 1.0 4B Benchmarks", What is
 * Dory1.0-4B?). Every layer is an attention sublayer and a SwiGLU sublayer,
 * each closed by the nGPT hypersphere update
 *     h <- norm(h + alpha * (norm(y) - h))
 * (summary, Methodology in Plain English). Attention layers are either
 * sliding-window or full, with grouped-query heads, RoPE (one base per layer
 * type), per-head L2-normalised q and k, and a sigmoid output gate (same
 * section). Keys and values are cached per loop or in last-loop mode, where
 * every loop overwrites one cache per recurrent layer (goremy.ai blog, How
 * does looping work at inference time?; broadside review "NVIDIA Nemotron
 * Labs Dory 1.0 4B", Key ideas).
 *
 * Conventions used by every call below.
 *   - All sizes are element counts unless a name ends in _bytes.
 *   - "device" pointers are HIP device memory (for example from PyTorch);
 *     "host" pointers are ordinary CPU memory.
 *   - The caller owns ALL device memory: weights, the KV buffer and the
 *     workspace. The library owns only its host-side context. No call after
 *     dory_create allocates device memory.
 *   - Compute calls enqueue work on the stream given to dory_create and
 *     return before it finishes; the caller synchronises that stream before
 *     it reads results on the host.
 *   - Validation happens on the host before anything is enqueued. A call
 *     that returns an error has enqueued nothing and changed no state.
 *   - The bfloat16 type is passed as its 16-bit pattern (uint16_t storage).
 */
#ifndef DORY_H
#define DORY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DORY_OK = 0,
  DORY_E_ARG = -1,       /* null pointer, bad size, inconsistent config      */
  DORY_E_CAPACITY = -2,  /* batch, chunk or context beyond the capacity       */
  DORY_E_LOOPS = -3,     /* n_loops < 1, > max_loops or > the per-loop caches,
                            or a loop-count change inside a per-loop sequence */
  DORY_E_KV_MODE = -4,   /* kv mode other than the one the buffer was laid out for */
  DORY_E_STATE = -5,     /* decode/logits before any prefill, batch change mid-sequence */
  DORY_E_HIP = -6        /* a HIP runtime call failed; see dory_last_error   */
} dory_status;

typedef enum { DORY_F32 = 0, DORY_BF16 = 1 } dory_dtype;

/* Per-loop: one cache per loop of each recurrent attention layer, so KV
 * memory grows with k. Last-loop: one cache per recurrent layer, overwritten
 * by every loop; the footprint equals the one-loop size at any k. */
typedef enum { DORY_KV_PER_LOOP = 0, DORY_KV_LAST_LOOP = 1 } dory_kv_mode;

/* Storage of the layer projections (q|k|v|gate, o, up/gate, down).
 * DORY_WEIGHTS_DTYPE: the config's dtype. The low-bit formats (bfloat16
 * models) are our readings of the MXFP8 and NVFP4 checkpoints the pages name
 * ("Dory1.0-4B: A Looped Normalized-GPT", AI summary, Key Contributions 4 and
 * Methodology in Plain English):
 * DORY_WEIGHTS_MXFP8: the OCP Microscaling (MX) v1.0 MXFP8 format, E4M3
 * element codes [N][K] (one byte each) and one E8M0 scale byte per block of
 * 32 consecutive elements along K, [N][K/32]; element code q of block scale
 * byte s stands for e4m3(q) * 2^(s - 127).
 * DORY_WEIGHTS_NVFP4: E2M1 element codes, two per byte with the even element
 * in the low nibble, [N][K/2]; one E4M3 scale byte (a positive finite E4M3
 * value, codes 1..126) per block of 16 consecutive elements along K,
 * [N][K/16]; one float32 scale g per tensor; code q of block scale s stands
 * for e2m1(q) * e4m3(s) * g.
 * The embedding / LM head stays in the dtype. */
typedef enum { DORY_WEIGHTS_DTYPE = 0, DORY_WEIGHTS_MXFP8 = 1, DORY_WEIGHTS_NVFP4 = 2 } dory_weight_format;

/* Model shape and capacity. Copied by dory_create (layer_is_full included). */
typedef struct {
  int32_t d_model;        /* residual-stream width d                                  */
  int32_t n_q_heads;      /* query heads                                               */
  int32_t n_kv_heads;     /* key/value heads; n_q_heads / n_kv_heads in {1,2,3,4,6,8}  */
  int32_t head_dim;       /* 64 or 128                                                 */
  int32_t d_ff;           /* SwiGLU hidden width                                       */
  int32_t vocab;          /* tied embedding / LM-head rows                             */
  int32_t n_in, n_rec, n_out;   /* input / recurrent / output layers                   */
  int32_t window;         /* sliding window in keys, the query included: t-W < s <= t  */
  const uint8_t* layer_is_full; /* host [n_in+n_rec+n_out]: 1 full attention, 0 window */
  double rope_base_swa;   /* RoPE base of sliding-window layers                        */
  double rope_base_full;  /* RoPE base of full-attention layers                        */
  int32_t dtype;          /* dory_dtype of weights, activations and KV cache           */
  int32_t attn_gate;      /* 0 none, 1 elementwise sigmoid gate, 2 one gate per q head */
  float attn_scale;       /* softmax scale on q.k of unit vectors; <= 0: sqrt(head_dim) */
  float logit_scale;      /* LM-head scale; <= 0: sqrt(d_model)                        */
  float combine_wh;       /* loop re-injection x_j = norm(wh*h_{j-1} + we*e), j >= 2   */
  float combine_we;
  int32_t max_batch;      /* sequences per call                                        */
  int32_t max_ctx;        /* positions per sequence (bfloat16 decode attention runs on
                             the matrix cores when max_ctx and window are multiples of 8) */
  int32_t max_chunk;      /* positions per prefill chunk (longer prompts are chunked)  */
  int32_t max_loops;      /* largest n_loops accepted                                  */
  int32_t weight_format;  /* dory_weight_format of the layer projections; MXFP8 and NVFP4
                             need bfloat16, d_model <= 8192 and d_model, n_q*hd and
                             d_ff multiples of 32                                     */
} dory_config;

/* Weights, all device pointers, row-major, of the config's dtype except alpha.
 * Arrays of per-layer pointers are host arrays of n_layers entries, copied by
 * dory_create; the device memory they point to must outlive the context.
 *   embed [vocab, d]                       input embedding and tied LM head
 *   qkvg  [q_dim + 2*kv_dim + gate_dim, d] rows: q | k | v | gate
 *         (q_dim = n_q*hd, kv_dim = n_kv*hd, gate_dim = q_dim, n_q or 0)
 *   o     [d, q_dim]                       attention output projection
 *   ug    [2*d_ff, d]                      rows 0..d_ff-1: u, rows d_ff..: v;
 *                                          the activation is u * silu(v)
 *   down  [d, d_ff]                        MLP down projection
 *   alpha_attn, alpha_mlp: float32 [d]     per-channel nGPT update weights
 * With a low-bit weight_format, qkvg / o / ug / down hold the element codes
 * (16-byte aligned) and qkvg_scale / o_scale / ug_scale / down_scale the
 * block scale bytes (NULL otherwise; 2-byte aligned for NVFP4); with
 * DORY_WEIGHTS_NVFP4, qkvg_tscale / o_tscale / ug_tscale / down_tscale are
 * HOST arrays of n_layers float32 tensor scales (copied by dory_create;
 * NULL otherwise). */
typedef struct {
  const void* embed;
  const void* const* qkvg;
  const void* const* o;
  const void* const* ug;
  const void* const* down;
  const float* const* alpha_attn;
  const float* const* alpha_mlp;
  const void* const* qkvg_scale;
  const void* const* o_scale;
  const void* const* ug_scale;
  const void* const* down_scale;
  const float* qkvg_tscale;
  const float* o_tscale;
  const float* ug_tscale;
  const float* down_tscale;
} dory_weights;

typedef struct dory_ctx dory_ctx;

/* ---- host-only queries (no HIP call; usable without a GPU) -------------- */

/* DORY_OK if the config is consistent and within the kernels' limits:
 * d_model <= 65536, d_ff <= 262144, n_q_heads <= 1024, vocab <= 2^26, at most
 * 4096 layers per block, max_batch <= 2^20, max_ctx <= 2^26, max_loops <= 64,
 * max_batch * n_kv_heads * head_dim * 2 * (max_ctx + 32) <= 2^40 (one cache),
 * finite attn_scale, logit_scale and combine weights. The layer_is_full array
 * is read only after the layer counts have passed these checks. */
dory_status dory_validate_config(const dory_config* cfg);

/* Bytes of the KV buffer for a kv mode. kv_loops is the number of per-loop
 * caches per recurrent layer (ignored in last-loop mode). Layout: caches
 * numbered layer by layer (a recurrent layer in per-loop mode owns kv_loops
 * consecutive ids, loop j -> base + j - 1); cache c holds K as
 * [max_batch][n_kv][slots_c][head_dim] and then V as
 * [max_batch][n_kv][vslots_c / 32][head_dim][32]: blocks of 32 slots, each
 * with the 32 values of one dimension contiguous (the operand order of the
 * P.V matrix-core product; one block is one contiguous run), with slots =
 * max_ctx for full layers and min(window, max_ctx) for sliding layers (a
 * ring, slot = pos mod window) and vslots_c = slots_c rounded up to 32.
 * Returns 0 for an invalid config. */
size_t dory_kv_bytes(const dory_config* cfg, int32_t kv_mode, int32_t kv_loops);

/* Bytes of the workspace dory_create needs (activations for max_batch *
 * max_chunk rows, attention partials and sums, RoPE tables, logits). 0 if
 * invalid. */
size_t dory_workspace_bytes(const dory_config* cfg);

/* Where the KV of (layer, loop, pos) lives: cache id, slot, and the element
 * offsets of dimension 0 of K and of V for batch row 0, kv head 0 in the KV
 * buffer (K's dimensions follow contiguously, V's every 32 elements).
 * loop is 1-based for recurrent layers and ignored for the others. */
dory_status dory_kv_slot(const dory_config* cfg, int32_t kv_mode, int32_t kv_loops,
                         int32_t layer, int32_t loop, int32_t pos,
                         int32_t* cache_id, int32_t* slot,
                         int64_t* k_offset, int64_t* v_offset);

const char* dory_status_string(dory_status s);

/* ---- context ------------------------------------------------------------ */

/* Binds caller memory; makes no HIP call and allocates nothing on the
 * device (every computation runs on this library's kernels, in memory the
 * caller owns). The first dory_prefill on
 * the context builds the RoPE tables (angles in float64, stored float32) in
 * the workspace on the stream. kv_dev must hold dory_kv_bytes(cfg, kv_mode,
 * kv_loops) bytes and ws_dev dory_workspace_bytes(cfg); both 256-byte
 * aligned. stream is a hipStream_t (NULL = the null stream). */
dory_status dory_create(const dory_config* cfg, const dory_weights* w,
                        void* kv_dev, size_t kv_bytes, int32_t kv_mode, int32_t kv_loops,
                        void* ws_dev, size_t ws_bytes, void* stream, dory_ctx** out);

void dory_destroy(dory_ctx* ctx);

/* Forget the sequence: position 0, no kv mode or loop count fixed yet.
 * Cache contents are not cleared; they are never read before rewritten. */
dory_status dory_reset(dory_ctx* ctx);

/* Continue sequences whose KV cache the caller has put in the KV buffer
 * (for example a saved session copied back, laid out as dory_kv_slot
 * describes): positions [0, pos) of `batch` sequences are taken as cached,
 * written with kv_mode and, in per-loop mode, n_loops loops (the count the
 * sequence must keep). The next call is a dory_prefill or a dory_decode_step
 * with explicit tokens (there are no logits to take greedy tokens from).
 * Enqueues the device-side position update on the stream.
 * Errors: DORY_E_CAPACITY (batch outside [1, max_batch], pos outside
 * [1, max_ctx - 1]), DORY_E_LOOPS, DORY_E_KV_MODE. */
dory_status dory_resume(dory_ctx* ctx, int32_t batch, int32_t pos, int32_t n_loops, int32_t kv_mode);

/* Process n prompt positions of `batch` sequences: tokens_dev is device
 * int32 [batch, n]. Prompts longer than max_chunk are cut into chunks of
 * max_chunk positions, processed in order. Afterwards the logits of the last
 * position and its greedy token are held in the context.
 * Errors: DORY_E_LOOPS, DORY_E_KV_MODE, DORY_E_CAPACITY (pos + n > max_ctx,
 * batch > max_batch), DORY_E_STATE (batch differs from the sequence's). */
dory_status dory_prefill(dory_ctx* ctx, const int32_t* tokens_dev, int32_t batch, int32_t n,
                         int32_t n_loops, int32_t kv_mode);

/* One decode position. tokens_dev: device int32 [batch], or NULL to feed the
 * greedy tokens of the previous call. next_tokens_dev: device int32 [batch]
 * that receives the greedy argmax (lowest index on ties), or NULL. In
 * last-loop mode n_loops may change from call to call; in per-loop mode it
 * must stay the sequence's. Errors as dory_prefill, plus DORY_E_STATE before
 * any prefill or dory_resume, and for tokens_dev NULL when no logits are held
 * (right after dory_resume). */
dory_status dory_decode_step(dory_ctx* ctx, const int32_t* tokens_dev, int32_t n_loops,
                             int32_t kv_mode, int32_t* next_tokens_dev);

/* Per-sequence loop counts in one batched call: the loop count is a
 * serve-time choice per request ("Dory1.0-4B: A Looped Normalized-GPT", AI
 * summary, Key Contributions 1; broadside review, Why it matters here).
 * Sequence b runs loops_host[b] passes of the recurrent block (host int32
 * [batch], each in [1, max_loops]); while the batch runs on, sequence b's
 * state stays as its own last pass left it, and its recurrent layers' K/V
 * are written on that pass. Each sequence's result is the one it would get
 * alone with its own count. Last-loop caching only (DORY_E_KV_MODE
 * otherwise); loops_host NULL or a count outside [1, max_loops] ->
 * DORY_E_ARG / DORY_E_LOOPS; the rest as dory_prefill / dory_decode_step. */
dory_status dory_prefill_mixed(dory_ctx* ctx, const int32_t* tokens_dev, int32_t batch, int32_t n,
                               const int32_t* loops_host, int32_t kv_mode);
dory_status dory_decode_step_mixed(dory_ctx* ctx, const int32_t* tokens_dev, const int32_t* loops_host,
                                   int32_t kv_mode, int32_t* next_tokens_dev);

/* Copy the float32 logits [batch, vocab] of the last processed position to
 * out_dev (device). DORY_E_STATE before any prefill. */
dory_status dory_logits(dory_ctx* ctx, float* out_dev);

/* Text of the last error on this context (empty if none). */
const char* dory_last_error(const dory_ctx* ctx);

/* Test tap: when trace_dev is not NULL, every layer application copies the
 * float32 residual stream h [rows, d_model] after its MLP update into
 * trace_dev + app * rows * d_model, app counting from 0 within each prefill
 * chunk or decode call; the buffer must hold max_apps entries (calls with more
 * layer applications return DORY_E_CAPACITY). NULL turns the tap off. */
dory_status dory_set_trace(dory_ctx* ctx, float* trace_dev, int32_t max_apps);

/* Recorded decode steps. With enable != 0, decode steps that continue from
 * the previous greedy tokens (tokens_dev NULL) on a bfloat16 model are
 * recorded once per (n_loops, batch) as a HIP graph and replayed afterwards on
 * a private stream that two events order after and before the context's
 * stream. enable = 0 (the default) launches every step kernel by kernel and
 * frees the recorded graphs. Results are bit-identical either way: every
 * kernel argument of a decode step is the same at every position (the
 * position is a device counter that prefill sets and each decode step's
 * argmax advances), which also lets a caller record dory_decode_step into a
 * graph of its own. Replays cost less host time per step and, on ROCm 7.2,
 * slightly more GPU time, so they pay off only when the host is the
 * bottleneck. */
dory_status dory_set_graphs(dory_ctx* ctx, int32_t enable);

/* Profiler ranges. With enable != 0, every dory_prefill, dory_decode_step
 * and dory_backward_last_loop call, and each layer application inside it
 * ("layer l loop j"; j = 0 outside the recurrent block), is bracketed by a
 * roctx range, host side (rocprofv3 --marker-trace shows them beside the
 * kernels they enqueue). The ROCm marker library (librocprofiler-sdk-roctx,
 * else libroctx64) is loaded on first use; DORY_E_ARG if neither loads. Off
 * by default; a switched-off context makes no marker call. */
dory_status dory_set_markers(dory_ctx* ctx, int32_t enable);

/* Kernel timing tap. When kind is not 0, every launch of one kernel class is
 * bracketed by HIP events recorded on the context's stream:
 *   1 SwiGLU up/gate projection   2 fused q|k|v|gate projection
 *   3 down projection             4 attention output projection
 *   5 split-K attention
 * At most max_launches launches are recorded (later ones are not). The events
 * are created here (host objects, no device memory); kind 0 releases them.
 * dory_kernel_time waits for the stream, returns the summed event time (ms)
 * and the count of recorded launches, and starts a new recording. */
dory_status dory_set_kernel_timing(dory_ctx* ctx, int32_t kind, int32_t max_launches);
dory_status dory_kernel_time(dory_ctx* ctx, double* total_ms, int32_t* launches);

/* ---- single-kernel entry points (used by the kernel tests) -------------- */

/* y = x . W^T on the stream. x [M, ldx-strided rows of K], W [N, K] (dtype),
 * epilogue 0: y float32 [M, N] scaled by `scale`;
 * epilogue 1: SwiGLU, N = 2*F: y (dtype) [M, F] = u * silu(v), u = scale times
 *             cols 0..F-1, v = scale times cols F..2F-1.
 * algo 0 picks by M, 1 forces the matrix-vector kernel (M <= 8), 2 the tiled
 * matrix kernel. */
dory_status dory_op_linear(int32_t dtype, const void* x, int64_t ldx, const void* W, void* y,
                           int32_t M, int32_t N, int32_t K, int32_t epilogue, float scale,
                           int32_t algo, void* stream);

/* out[b] = argmax_v logits[b, v] (lowest index on ties); logits device float32
 * [B, V], out device int32 [B]. scratch_dev: device, >= dory_argmax_scratch_bytes. */
size_t dory_argmax_scratch_bytes(int32_t B, int32_t V);

/* MXFP8 encoding of a bfloat16 matrix w_dev [N][K] (K % 32 == 0, 16-byte
 * aligned) into codes_dev [N][K] and scales_dev [N][K/32] (see
 * dory_weight_format): block scale X = floor(log2(max |w|)) - 8 (an all-zero
 * block takes X = -127), codes round w / 2^X to the nearest E4M3 value, ties
 * to the even code, saturating at 448. Enqueued on stream. */
dory_status dory_op_quant_mxfp8(const void* w_dev, int32_t N, int32_t K, void* codes_dev, void* scales_dev,
                                void* stream);

/* y = x . W^T with MXFP8 weights (codes, scales) for M <= 8 rows (the decode
 * kernel); arguments as dory_op_linear (bfloat16 x, epilogue 0: float32 y * scale,
 * 1: SwiGLU to bfloat16). K % 32 == 0; DORY_E_ARG otherwise. */
dory_status dory_op_linear_mx(const void* x, int64_t ldx, const void* codes, const void* scales, void* y,
                              int32_t M, int32_t N, int32_t K, int32_t epilogue, float scale, void* stream);

/* NVFP4 encoding (DORY_WEIGHTS_NVFP4) of a bfloat16 matrix w_dev [N][K]
 * (K % 32 == 0, 16-byte aligned) into codes_dev [N][K/2] (8-byte aligned),
 * scales_dev [N][K/16] and the tensor scale *tscale_dev (one device float32):
 * g = float32(max |w| / 2688) (1 for an all-zero matrix); for every block the
 * E4M3 scale 1..126 of least squared error (the pages' dynamic MSE scale
 * selection, "Dory1.0-4B: A Looped Normalized-GPT", AI summary, Methodology in
 * Plain English), computed in float64 in element order so that the choice is
 * reproducible, the smallest code on equal errors; elements rounded to the
 * nearest E2M1 magnitude of |w| / (e4m3 * g), ties to the even code,
 * saturating at 6, sign from w. Enqueued on stream (four kernels). */
dory_status dory_op_quant_nvfp4(const void* w_dev, int32_t N, int32_t K, void* codes_dev, void* scales_dev,
                                float* tscale_dev, void* stream);

/* y = x . W^T with NVFP4 weights (codes, block scales) for M <= 8 rows (the
 * decode kernel); the tensor scale g is not read here: pass scale = g (times
 * any other factor). Otherwise as dory_op_linear_mx; scales 2-byte aligned. */
dory_status dory_op_linear_fp4(const void* x, int64_t ldx, const void* codes, const void* scales, void* y,
                               int32_t M, int32_t N, int32_t K, int32_t epilogue, float scale, void* stream);
dory_status dory_op_argmax(const float* logits, int32_t B, int32_t V, int32_t* out,
                           void* scratch_dev, void* stream);

/* dory_op_argmax for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and result, with the partials in a 64 KiB device array
 * that the library holds, one copy per GPU, kept until the process ends. The
 * caller passes only the logits (device float32 [B, V]) and out (device
 * int32 [B]). Limit: B * ceil(V / 1024) <= 8192 (batch 64 at vocabulary
 * 131,072), else DORY_E_CAPACITY and nothing is enqueued; DORY_E_ARG for a
 * NULL pointer or B, V < 1; DORY_E_HIP if the array's address cannot be
 * found on the current device. Calls no allocator. Every call on one GPU
 * uses that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
dory_status dory_op_argmax_noalloc(const float* logits, int32_t B, int32_t V, int32_t* out, void* stream);

/* ---- depth-1 truncated backward of the last recurrent invocation -------- */

/* The pages train the looped stage with backpropagation truncated to depth
 * one: only the final invocation of the recurrent block receives gradients
 * ("Dory1.0-4B: A Looped Normalized-GPT", AI summary, Methodology in Plain
 * English). For a training chunk of `batch` sequences of n positions starting
 * at position 0: x_dev [batch, n, d] float32 is that invocation's input (the
 * re-injected input, a constant for the truncated backward), h_out =
 * norm(R(x)) with R the recurrent layers in order and attention over the
 * chunk's own positions (causal; t - s < window in sliding-window layers).
 * Given grad_out_dev = dL/dh_out [batch, n, d] float32, writes dL/dW of the
 * four projections and dL/dalpha of both updates of every recurrent layer
 * into `grads` (overwritten, not accumulated) and dL/dx into grad_x_dev (may
 * be NULL). Projections in the context's dtype (bfloat16 operands on the
 * matrix cores with float32 accumulation), everything else float32. Needs a
 * DORY_WEIGHTS_DTYPE context, n <= max_ctx, head_dim 64 or 128; independent
 * of the sequence state (no cache is read or written). ws_dev: device,
 * 256-byte aligned, caller-owned; with ws_bytes >= dory_backward_workspace_bytes
 * the forward values of every recurrent layer are kept from the forward sweep
 * (fastest), with ws_bytes >= dory_backward_workspace_min_bytes only each
 * layer's input is kept and its forward runs again during the backward (the
 * same results, bit for bit). Enqueued on the context's stream. DORY_E_ARG on
 * bad arguments or a smaller workspace (nothing enqueued), DORY_E_HIP on a
 * launch failure. */
typedef struct {            /* host arrays of n_rec device float32 pointers; entry i is
                               global layer n_in + i                                    */
  float* const* qkvg;       /* [qkvg_dim, d] */
  float* const* o;          /* [d, q_dim]    */
  float* const* ug;         /* [2*d_ff, d]   */
  float* const* down;       /* [d, d_ff]     */
  float* const* alpha_attn; /* [d]           */
  float* const* alpha_mlp;  /* [d]           */
} dory_grads;

/* workspace of the backward keeping every layer's forward values / of the one
 * recomputing them; 0 on a bad configuration or size */
size_t dory_backward_workspace_bytes(const dory_config* cfg, int32_t batch, int32_t n);
size_t dory_backward_workspace_min_bytes(const dory_config* cfg, int32_t batch, int32_t n);
dory_status dory_backward_last_loop(dory_ctx* ctx, const float* x_dev, const float* grad_out_dev, int32_t batch,
                                    int32_t n, const dory_grads* grads, float* grad_x_dev, void* ws_dev,
                                    size_t ws_bytes);

#ifdef __cplusplus
}
#endif
#endif /* DORY_H */
