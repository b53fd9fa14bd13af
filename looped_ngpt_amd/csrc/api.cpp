// C ABI and host runtime of the looped nGPT forward pass: argument
// validation (before anything is enqueued), KV-buffer binding, and the loop
// controller that runs the input block once, the shared recurrent block
// n_loops times with the input block's output re-injected before every pass,
// and the output block once.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dory.h"
#include "kernels.h"
#include "plan.h"

using namespace dory;

struct dory_ctx {
  Plan plan;
  KvLayout kv;
  const void* embed = nullptr;
  std::vector<const void*> qkvg, o, ug, down;
  std::vector<const void*> qkvg_s, o_s, ug_s, down_s;  // low-bit block scales (nullptr otherwise)
  std::vector<float> qkvg_g, o_g, ug_g, down_g;         // NVFP4 tensor scales (1 otherwise)
  std::vector<const float*> alpha_attn, alpha_mlp;
  char* kvb = nullptr;
  char* ws = nullptr;
  hipStream_t st = nullptr;
  // sequence state
  int pos = 0, batch = 0, seq_loops = 0, kv_mode_seq = -1;
  bool mixed = false;  // inside a call with per-sequence loop counts (workspace rowk)
  bool has_logits = false;
  bool device_ready = false;  // RoPE tables built, flags cleared
  // test tap
  float* trace = nullptr;
  int trace_max = 0;
  // recorded decode steps, keyed by (n_loops, batch)
  // Recorded and replayed on a private stream (the caller's may be the null
  // stream, which cannot be recorded), ordered after and before the caller's
  // stream by two events.
  bool graphs_on = false;
  bool markers = false;  // profiler ranges around calls, loop passes and layer applications
  // position of the decode step's new key, passed by value to the decode
  // attention on eager, uncaptured calls; -1: kernels read the device counter
  int t_now = -1;
  struct Graph { int k, B; hipGraph_t g; hipGraphExec_t x; };
  std::vector<Graph> graphs;
  hipStream_t gst = nullptr;
  hipEvent_t gev[2] = {nullptr, nullptr};
  // timing tap
  int time_kind = 0;
  std::vector<hipEvent_t> ev;
  size_t ev_used = 0;
  std::string err;
  void drop_graphs() {
    for (auto& g : graphs) {
      (void)hipGraphExecDestroy(g.x);
      (void)hipGraphDestroy(g.g);
    }
    graphs.clear();
  }
  ~dory_ctx() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    drop_graphs();
    for (hipEvent_t e : gev)
      if (e) (void)hipEventDestroy(e);
    if (gst) (void)hipStreamDestroy(gst);
  }
};

namespace {

template <typename P>
P* wsp(dory_ctx* c, size_t off) { return (P*)(c->ws + off); }

enum { TIME_NONE = 0, TIME_UG = 1, TIME_QKVG = 2, TIME_DOWN = 3, TIME_O = 4, TIME_ATTN = 5 };

// Hands a start/stop event pair to the first kernel launched inside the
// scope (recorded as part of its dispatch, so the pair times that kernel
// alone); counted only if a launch took it.
struct TimeScope {
  dory_ctx* c;
  bool on;
  TimeScope(dory_ctx* ctx, int kind) : c(ctx), on(ctx->time_kind == kind && ctx->ev_used + 2 <= ctx->ev.size()) {
    if (on) set_next_launch_events(c->ev[c->ev_used], c->ev[c->ev_used + 1]);
  }
  ~TimeScope() {
    if (on && !take_next_launch_events().start) c->ev_used += 2;
  }
};

dory_status set_err(dory_ctx* c, dory_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

#define HIP_TRY(ctx, call)                                                                         \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess)                                                                          \
      return set_err(ctx, DORY_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_));          \
  } while (0)

#define DORY_TRY(call)            \
  do {                            \
    dory_status s_ = (call);      \
    if (s_ != DORY_OK) return s_; \
  } while (0)

// y = x . W^T for one layer projection: the GEMV kernels up to 8 rows, the
// tiled matrix-core GEMMs above (SwiGLU in their epilogue). Low-bit weights:
// the decode GEMV for M <= 8 rows, otherwise the projection is first expanded
// to bfloat16 in the workspace and multiplied by the bfloat16 GEMM.
dory_status proj(dory_ctx* c, const void* W, const void* S, float g, const void* x, int64_t ldx, void* y, int M,
                 int N, int K, int epi, float scale) {
  const Plan& P = c->plan;
  const int dt = P.cfg.dtype;
  const int fmt = P.cfg.weight_format;
  if (fmt == DORY_WEIGHTS_DTYPE) {
    HIP_TRY(c, launch_linear(dt, x, ldx, W, y, M, N, K, epi, scale, 0, c->st));
  } else if (linear_lowbit_supported(fmt, M, K)) {
    HIP_TRY(c, launch_linear_lowbit(fmt, x, ldx, W, S, y, M, N, K, epi, scale * g, c->st));
  } else {
    void* wdq = c->ws + P.ws.wdq;
    HIP_TRY(c, launch_dequant_lowbit(fmt, W, S, N, K, wdq, c->st));
    HIP_TRY(c, launch_linear(dt, x, ldx, wdq, y, M, N, K, epi, scale * g, 0, c->st));
  }
  return DORY_OK;
}

// A projection into the residual branch y (output and down projections):
// at 9..64 rows (batched decode) with too few output tiles to fill the CUs,
// the contraction runs in two halves side by side, the second into the
// workspace's y1, and *y1 tells the update that reads y to add it.
dory_status proj_y(dory_ctx* c, const void* W, const void* S, float g, const void* x, int64_t ldx, float* y, int M,
                   int N, int K, const float** y1) {
  const Plan& P = c->plan;
  *y1 = nullptr;
  if (P.cfg.weight_format == DORY_WEIGHTS_DTYPE && gemm_skinny_split2_pays(P.cfg.dtype, M, N, K)) {
    float* y1w = wsp<float>(c, P.ws.y1);
    HIP_TRY(c, launch_gemm_skinny_split2(x, ldx, W, y, y1w, M, N, K, 1.f, c->st));
    *y1 = y1w;
    return DORY_OK;
  }
  return proj(c, W, S, g, x, ldx, y, M, N, K, 0, 1.f);
}

// The decode GEMV with the nGPT update in its prologue, for any weight format.
dory_status proj_pro(dory_ctx* c, const GemvPro& p, const void* W, const void* S, float g, void* y, int M, int N,
                     int K, int epi) {
  const int fmt = c->plan.cfg.weight_format;
  if (fmt != DORY_WEIGHTS_DTYPE)
    HIP_TRY(c, launch_linear_pro_lowbit(fmt, p, W, S, y, M, N, K, epi, g, c->st));
  else
    HIP_TRY(c, launch_linear_pro(p, W, y, M, N, K, epi, 1.f, c->st));
  return DORY_OK;
}

// Key splits of decode attention: about 128 keys per workgroup, at most
// kMaxSplits, and no more than ~4 workgroups per CU over all (row, kv head).
// Profiler ranges (roctx), resolved from the ROCm marker library on first
// use; a no-op unless the context has them switched on.
struct RoctxApi {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
const RoctxApi& roctx_api() {
  static RoctxApi api;
  static std::once_flag once;
  std::call_once(once, [] {
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      auto push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
      auto pop = (int (*)())dlsym(h, "roctxRangePop");
      if (push && pop) {
        api.push = push;
        api.pop = pop;
        return;
      }
    }
  });
  return api;
}

struct Range {
  bool on;
  Range(const dory_ctx* c, const char* fmt, int x = 0, int y = 0) : on(c->markers && roctx_api().push) {
    if (!on) return;
    char buf[96];
    std::snprintf(buf, sizeof buf, fmt, x, y);
    roctx_api().push(buf);
  }
  ~Range() {
    if (on) roctx_api().pop();
  }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

int choose_splits_decode(int keys, int B, int nkv) {
  int s = (keys + 127) / 128;
  const int cap = (1024 + B * nkv - 1) / (B * nkv);
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

dory_status decode_attention(dory_ctx* c, int l, int loop, int B, bool write_kv, bool to_acc = false);

// One layer application (attention sublayer + MLP sublayer) on `rows` rows.
// write_kv: store this application's K/V in the cache. In last-loop mode the
// recurrent layers store only on the final loop: earlier loops read this
// call's positions from the workspace and earlier positions from the cache,
// which must still hold the previous calls' entries (a ring slot overwritten
// by loop 1 would lose keys that loop 2 still needs).
dory_status run_layer(dory_ctx* c, int l, int loop, int B, int n, float* h2, int app, bool write_kv) {
  Range range(c, "layer %d loop %d", l, loop);
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const WsLayout& W = P.ws;
  const int rows = B * n;
  const int dt = C.dtype;
  const int full = P.is_full[l];
  const int cid = c->kv.first_id[l] + ((P.recurrent(l) && c->kv.kv_mode == DORY_KV_PER_LOOP) ? loop - 1 : 0);
  const int slots = P.slots(l);
  char* kc = c->kvb + (size_t)c->kv.offset[cid] * P.elem;
  char* vc = kc + (size_t)C.max_batch * C.n_kv_heads * slots * C.head_dim * P.elem;
  float* h = wsp<float>(c, W.h);
  void* xb = c->ws + W.xb;
  float* qkvg = wsp<float>(c, W.qkvg);
  float* y = wsp<float>(c, W.y);
  hipStream_t st = c->st;
  // mixed loop counts: rows past their count keep their state; K/V are
  // written on each sequence's own last pass
  const int* mix = (c->mixed && P.recurrent(l)) ? wsp<int>(c, W.rowk) : nullptr;
  const RowGate gate{mix, loop, n};

  {
    TimeScope ts(c, TIME_QKVG);
    DORY_TRY(proj(c, c->qkvg[l], c->qkvg_s[l], c->qkvg_g[l], xb, C.d_model, qkvg, rows, P.qkvg_dim, C.d_model, 0, 1.f));
  }

  if (n == 1) {
    dory_status s = decode_attention(c, l, loop, B, write_kv);
    if (s != DORY_OK) return s;
  } else {
    RopeArgs ra{};
    ra.qkvg = qkvg; ra.ld = P.qkvg_dim;
    ra.tab = wsp<float2>(c, full ? W.rope_full : W.rope_swa);
    ra.p0 = c->pos; ra.B = B; ra.n = n; ra.rows = rows; ra.nq = C.n_q_heads; ra.nkv = C.n_kv_heads;
    ra.hd = C.head_dim;
    ra.vld = chunk_vld(n);
    ra.q_out = c->ws + W.q; ra.k_out = c->ws + W.kw; ra.v_out = c->ws + W.vw;
    HIP_TRY(c, launch_rope_qk(dt, ra, st));

    AttnArgs aa{};
    aa.q = c->ws + W.q; aa.kw = c->ws + W.kw; aa.vw = c->ws + W.vw; aa.kc = kc; aa.vc = vc;
    aa.B = B; aa.n = n; aa.p0 = c->pos; aa.nq = C.n_q_heads; aa.nkv = C.n_kv_heads; aa.hd = C.head_dim;
    aa.slots = slots; aa.window = C.window; aa.is_full = full;
    aa.n_split = 1;
    aa.vld = ra.vld;
    aa.scale = P.attn_scale;
    aa.part = wsp<float>(c, W.part);
    const int gate_off = P.q_dim + 2 * P.kv_dim;
    if (attn_prefill_supported(dt, C.head_dim, C.n_q_heads, C.n_kv_heads)) {
      TimeScope ts(c, TIME_ATTN);
      HIP_TRY(c, launch_attn_prefill(aa, qkvg, P.qkvg_dim, gate_off, C.attn_gate, c->ws + W.ob, st));
    } else {
      {
        TimeScope ts(c, TIME_ATTN);
        HIP_TRY(c, launch_attn_split(dt, aa, st));
      }
      HIP_TRY(c, launch_attn_combine(dt, aa.part, qkvg, P.qkvg_dim, gate_off, C.attn_gate, c->ws + W.ob, rows,
                                     C.n_q_heads, C.head_dim, aa.n_split, st));
    }
    // after attention: the ring slots of this call's positions held keys it needed
    if (write_kv)
      HIP_TRY(c, launch_kv_write(dt, c->ws + W.kw, c->ws + W.vw, ra.vld, kc, vc, B, n, c->pos, C.n_kv_heads,
                                 C.head_dim, slots, C.window, full, st, mix, loop));
  }

  const float* y1 = nullptr;
  {
    TimeScope ts(c, TIME_O);
    DORY_TRY(proj_y(c, c->o[l], c->o_s[l], c->o_g[l], c->ws + W.ob, P.q_dim, y, rows, C.d_model, P.q_dim, &y1));
  }
  HIP_TRY(c, launch_update(dt, h, y, c->alpha_attn[l], xb, nullptr, rows, C.d_model, st, gate, y1));
  {
    TimeScope ts(c, TIME_UG);
    DORY_TRY(proj(c, c->ug[l], c->ug_s[l], c->ug_g[l], xb, C.d_model, c->ws + W.a, rows, 2 * C.d_ff, C.d_model, 1, 1.f));
  }
  {
    TimeScope ts(c, TIME_DOWN);
    DORY_TRY(proj_y(c, c->down[l], c->down_s[l], c->down_g[l], c->ws + W.a, C.d_ff, y, rows, C.d_model, C.d_ff, &y1));
  }
  HIP_TRY(c, launch_update(dt, h, y, c->alpha_mlp[l], xb, h2, rows, C.d_model, st, gate, y1));
  if (c->trace)
    HIP_TRY(c, hipMemcpyAsync(c->trace + (size_t)app * rows * C.d_model, h, (size_t)rows * C.d_model * 4,
                              hipMemcpyDeviceToDevice, st));
  return DORY_OK;
}

// Decode attention of layer l (loop j) on the fused projection rows: RoPE,
// q/k norm, split-K attention, new key/value into the cache, merge and gate.
dory_status decode_attention(dory_ctx* c, int l, int loop, int B, bool write_kv, bool to_acc) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const WsLayout& W = P.ws;
  const int full = P.is_full[l];
  const int cid = c->kv.first_id[l] + ((P.recurrent(l) && c->kv.kv_mode == DORY_KV_PER_LOOP) ? loop - 1 : 0);
  const int slots = P.slots(l);
  char* kc = c->kvb + (size_t)c->kv.offset[cid] * P.elem;
  char* vc = kc + (size_t)C.max_batch * C.n_kv_heads * slots * C.head_dim * P.elem;
  float* qkvg = wsp<float>(c, W.qkvg);
  AttnDecArgs da{};
  da.qkvg = qkvg; da.ld = P.qkvg_dim;
  da.tab = wsp<float2>(c, full ? W.rope_full : W.rope_swa);
  da.t_dev = wsp<int>(c, W.pos); da.t_now = c->t_now; da.B = B; da.nq = C.n_q_heads; da.nkv = C.n_kv_heads; da.hd = C.head_dim;
  da.slots = slots; da.window = C.window; da.is_full = full; da.write_kv = write_kv ? 1 : 0;
  // split count from the capacity (not the position), so a recorded graph
  // replays at every step; the kernel spreads the actual keys over the splits
  const int key_cap = full ? C.max_ctx : std::min(C.window, C.max_ctx);
  if (attn_decode_uses_mfma(C.dtype, C.head_dim, slots, C.window, full))
    // 32-slot tiles: a ring's tiles are fixed, positions 0..t of a full layer
    // may straddle one tile more
    da.n_split = choose_splits_decode(full ? ((key_cap + 31) / 32 + 1) * 32 : (slots + 31) / 32 * 32, B, C.n_kv_heads);
  else
    da.n_split = choose_splits_decode(key_cap, B, C.n_kv_heads);
  da.scale = P.attn_scale;
  da.kc = kc; da.vc = vc;
  da.part = wsp<float>(c, W.part);
  da.wloops = (c->mixed && P.recurrent(l)) ? wsp<int>(c, W.rowk) : nullptr;
  da.loop = loop;
  da.acc = to_acc ? wsp<unsigned long long>(c, W.attn_acc) : nullptr;
  da.acc_nb = attn_acc_bins(P.attn_scale);
  da.gate_off = P.q_dim + 2 * P.kv_dim;
  da.gate = C.attn_gate;
  {
    TimeScope ts(c, TIME_ATTN);
    HIP_TRY(c, launch_attn_decode(C.dtype, da, c->st));
  }
  if (!to_acc)
    HIP_TRY(c, launch_attn_merge(C.dtype, da.part, qkvg, P.qkvg_dim, P.q_dim + 2 * P.kv_dim, C.attn_gate,
                                   c->ws + W.ob, B, C.n_q_heads, C.head_dim, da.n_split, c->st));
  return DORY_OK;
}

// Decode attention summed into the workspace accumulators and the output
// projection built from them (no merge launch): bfloat16 activations, at
// most 8 rows, the matrix-core attention kernel for this layer, and an
// output GEMV that can stage its input from the accumulators.
bool attn_to_acc_ok(const dory_ctx* c, int l, int B) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  if (C.dtype != DORY_BF16 || B > 8 || C.head_dim % 8) return false;
  if (attn_acc_bins(P.attn_scale) == 0) return false;  // scale too large for the fixed-point bins
  if (!attn_decode_uses_mfma(C.dtype, C.head_dim, P.slots(l), C.window, P.is_full[l])) return false;
  return C.weight_format == DORY_WEIGHTS_DTYPE ? linear_attn_supported(B, P.q_dim)
                                               : linear_lowbit_supported(C.weight_format, B, P.q_dim);
}

// y = W_o . gate(attention) with the attention read from the accumulators
dory_status proj_attn_o(dory_ctx* c, int l, int B, float* y) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  AttnX ax{wsp<unsigned long long>(c, P.ws.attn_acc), C.head_dim, C.n_q_heads, attn_acc_bins(P.attn_scale)};
  if (C.weight_format == DORY_WEIGHTS_DTYPE)
    HIP_TRY(c, launch_linear_attn(ax, c->o[l], y, B, C.d_model, P.q_dim, 1.f, c->st));
  else
    HIP_TRY(c, launch_linear_lowbit_attn(C.weight_format, ax, c->o[l], c->o_s[l], y, B, C.d_model, P.q_dim,
                                         c->o_g[l], c->st));
  return DORY_OK;
}

// Decode with the nGPT updates folded into the consuming projections: per
// layer application the q|k|v|gate GEMV (its prologue applies the previous
// MLP update, and at the start of loops >= 2 the re-injection of e), the
// fused attention + merge, the output GEMV, the up/gate GEMV (prologue: the
// attention update) and the down GEMV. Residuals alternate between two
// buffers so the workgroup writing the new one never races readers of the old.
bool fused_decode_ok(const dory_ctx* c, int B) {
  const dory_config& C = c->plan.cfg;
  const bool pro_ok = C.weight_format != DORY_WEIGHTS_DTYPE ? linear_pro_lowbit_supported(C.weight_format, B, C.d_model)
                                                           : linear_pro_supported(B, C.d_model);
  return C.dtype == DORY_BF16 && !c->trace && !c->mixed && C.n_rec >= 1 && pro_ok;
}

dory_status run_decode_fused(dory_ctx* c, const int32_t* tok, int B, int k) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const WsLayout& W = P.ws;
  const int dt = C.dtype;
  const int d = C.d_model;
  hipStream_t st = c->st;
  float* cur = wsp<float>(c, W.h);
  float* alt = wsp<float>(c, W.hb);
  float* e = wsp<float>(c, W.e);
  float* y = wsp<float>(c, W.y);
  float* qkvg = wsp<float>(c, W.qkvg);
  void* xb = c->ws + W.xb;
  HIP_TRY(c, launch_embed(dt, tok, c->embed, cur, C.n_in == 0 ? e : nullptr, xb, B, d, C.vocab,
                          wsp<int>(c, W.flags), st));
  // attention accumulators: cleared here for the first layer application,
  // then by each q|k|v|gate GEMV (after the previous output GEMV read them)
  bool any_acc = false;
  for (int l = 0; l < P.n_layers; ++l) any_acc = any_acc || attn_to_acc_ok(c, l, B);
  unsigned long long* acc = wsp<unsigned long long>(c, W.attn_acc);
  const int acc_n = B * C.n_q_heads * attn_acc_stride(C.head_dim, attn_acc_bins(P.attn_scale));
  if (any_acc) HIP_TRY(c, launch_zero_u64(acc, acc_n, st));
  const float* pending_alpha = nullptr;  // MLP update not yet applied to the residual
  auto app = [&](int l, int j, bool write_kv) -> dory_status {
    Range range(c, "layer %d loop %d", l, j);
    if (pending_alpha) {
      const bool first_rec = l == C.n_in;
      GemvPro pr{};
      pr.y = y; pr.h_in = cur; pr.alpha = pending_alpha;
      pr.e = (first_rec && j >= 2) ? e : nullptr;
      pr.wh = C.combine_wh; pr.we = C.combine_we;
      pr.h_out = alt;
      pr.e_out = (first_rec && j == 1) ? e : nullptr;
      pr.zero = any_acc ? acc : nullptr;
      pr.zero_n = acc_n;
      TimeScope ts(c, TIME_QKVG);
      DORY_TRY(proj_pro(c, pr, c->qkvg[l], c->qkvg_s[l], c->qkvg_g[l], qkvg, B, P.qkvg_dim, d, 0));
      std::swap(cur, alt);
    } else {
      TimeScope ts(c, TIME_QKVG);
      DORY_TRY(proj(c, c->qkvg[l], c->qkvg_s[l], c->qkvg_g[l], xb, d, qkvg, B, P.qkvg_dim, d, 0, 1.f));
    }
    const bool to_acc = attn_to_acc_ok(c, l, B);
    dory_status s = decode_attention(c, l, j, B, write_kv, to_acc);
    if (s != DORY_OK) return s;
    {
      TimeScope ts(c, TIME_O);
      if (to_acc)
        DORY_TRY(proj_attn_o(c, l, B, y));
      else
        DORY_TRY(proj(c, c->o[l], c->o_s[l], c->o_g[l], c->ws + W.ob, P.q_dim, y, B, d, P.q_dim, 0, 1.f));
    }
    {
      GemvPro pr{};
      pr.y = y; pr.h_in = cur; pr.alpha = c->alpha_attn[l];
      pr.h_out = alt;
      TimeScope ts(c, TIME_UG);
      DORY_TRY(proj_pro(c, pr, c->ug[l], c->ug_s[l], c->ug_g[l], c->ws + W.a, B, 2 * C.d_ff, d, 1));
      std::swap(cur, alt);
    }
    {
      TimeScope ts(c, TIME_DOWN);
      DORY_TRY(proj(c, c->down[l], c->down_s[l], c->down_g[l], c->ws + W.a, C.d_ff, y, B, d, C.d_ff, 0, 1.f));
    }
    pending_alpha = c->alpha_mlp[l];
    return DORY_OK;
  };
  for (int l = 0; l < C.n_in; ++l) {
    dory_status s = app(l, 0, true);
    if (s != DORY_OK) return s;
  }
  for (int j = 1; j <= k; ++j) {
    const bool write_kv = c->kv.kv_mode == DORY_KV_PER_LOOP || j == k;
    for (int l = C.n_in; l < C.n_in + C.n_rec; ++l) {
      dory_status s = app(l, j, write_kv);
      if (s != DORY_OK) return s;
    }
  }
  for (int l = C.n_in + C.n_rec; l < P.n_layers; ++l) {
    dory_status s = app(l, 0, true);
    if (s != DORY_OK) return s;
  }
  // the last MLP update, then the tied LM head on the updated residual
  HIP_TRY(c, launch_update(dt, cur, y, pending_alpha, xb, nullptr, B, d, st));
  HIP_TRY(c, launch_linear(dt, xb, d, c->embed, wsp<float>(c, W.logits), B, C.vocab, d, 0, P.logit_scale, 0, st));
  HIP_TRY(c, launch_argmax(wsp<float>(c, W.logits), B, C.vocab, wsp<int32_t>(c, W.next), c->ws + W.amax, st,
                           wsp<int>(c, W.pos)));
  c->has_logits = true;
  return DORY_OK;
}

// First compute call on a context: RoPE tables and the device error flags.
dory_status device_init(dory_ctx* c) {
  if (c->device_ready) return DORY_OK;
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  HIP_TRY(c, launch_rope_table(wsp<float2>(c, P.ws.rope_swa), C.max_ctx, C.head_dim, C.rope_base_swa, c->st));
  HIP_TRY(c, launch_rope_table(wsp<float2>(c, P.ws.rope_full), C.max_ctx, C.head_dim, C.rope_base_full, c->st));
  HIP_TRY(c, hipMemsetAsync(c->ws + P.ws.flags, 0, 256, c->st));
  c->device_ready = true;
  return DORY_OK;
}

// n new positions of B sequences (one prefill chunk or one decode step).
// decode: the device position already equals c->pos (set by the last prefill,
// advanced by every decode step's argmax).
dory_status run_forward(dory_ctx* c, const int32_t* tok, int64_t tok_ld, int B, int n, int k, bool logits,
                        bool decode = false) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const WsLayout& W = P.ws;
  const int rows = B * n;
  const int dt = C.dtype;
  float* h = wsp<float>(c, W.h);
  float* e = wsp<float>(c, W.e);
  void* xb = c->ws + W.xb;
  hipStream_t st = c->st;

  // gather the chunk's token ids into rows r = b*n + i
  const int32_t* trows = tok;
  if (B > 1 && tok_ld != n) {
    int32_t* dst = wsp<int32_t>(c, W.part);  // free until the first attention of this call
    HIP_TRY(c, hipMemcpy2DAsync(dst, (size_t)n * 4, tok, (size_t)tok_ld * 4, (size_t)n * 4, B,
                                hipMemcpyDeviceToDevice, st));
    trows = dst;
  }
  if (n == 1 && !decode) HIP_TRY(c, launch_set_pos(wsp<int>(c, W.pos), c->pos, st));  // decode kernels read it
  HIP_TRY(c, launch_embed(dt, trows, c->embed, h, C.n_in == 0 ? e : nullptr, xb, rows, C.d_model, C.vocab,
                          wsp<int>(c, W.flags), st));
  int app = 0;
  for (int l = 0; l < C.n_in; ++l) {
    dory_status s = run_layer(c, l, 0, B, n, l == C.n_in - 1 ? e : nullptr, app++, true);
    if (s != DORY_OK) return s;
  }
  for (int j = 1; j <= k; ++j) {
    if (j >= 2)
      HIP_TRY(c, launch_combine(dt, h, e, C.combine_wh, C.combine_we, xb, rows, C.d_model, st,
                                RowGate{c->mixed ? wsp<int>(c, W.rowk) : nullptr, j, n}));
    // mixed counts: every pass may be some sequence's last (per-row predicate in the writers)
    const bool write_kv = c->mixed || c->kv.kv_mode == DORY_KV_PER_LOOP || j == k;
    for (int l = C.n_in; l < C.n_in + C.n_rec; ++l) {
      dory_status s = run_layer(c, l, j, B, n, nullptr, app++, write_kv);
      if (s != DORY_OK) return s;
    }
  }
  for (int l = C.n_in + C.n_rec; l < P.n_layers; ++l) {
    dory_status s = run_layer(c, l, 0, B, n, nullptr, app++, true);
    if (s != DORY_OK) return s;
  }
  if (logits) {
    const char* last = (const char*)xb + (size_t)(n - 1) * C.d_model * P.elem;
    HIP_TRY(c, launch_linear(dt, last, (int64_t)n * C.d_model, c->embed, wsp<float>(c, W.logits), B, C.vocab,
                             C.d_model, 0, P.logit_scale, 0, st));
    HIP_TRY(c, launch_argmax(wsp<float>(c, W.logits), B, C.vocab, wsp<int32_t>(c, W.next), c->ws + W.amax, st,
                             decode ? wsp<int>(c, W.pos) : nullptr));
    c->has_logits = true;
  }
  return DORY_OK;
}

// One decode step as a recorded HIP graph (recorded on first use for this
// (n_loops, batch); every argument is step-invariant: the position comes from
// the device counter and the tokens from the previous step's argmax).
dory_status decode_graph(dory_ctx* c, int k) {
  const int B = c->batch;
  if (!c->gst) {
    HIP_TRY(c, hipStreamCreateWithFlags(&c->gst, hipStreamNonBlocking));
    for (hipEvent_t& e : c->gev) HIP_TRY(c, hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  hipGraphExec_t x = nullptr;
  for (auto& g : c->graphs)
    if (g.k == k && g.B == B) x = g.x;
  if (!x) {
    dory_ctx::Graph g{k, B, nullptr, nullptr};
    hipStream_t user = c->st;
    c->st = c->gst;
    hipError_t e = hipStreamBeginCapture(c->gst, hipStreamCaptureModeThreadLocal);
    dory_status s = e == hipSuccess ? run_decode_fused(c, wsp<int32_t>(c, c->plan.ws.next), B, k) : DORY_OK;
    if (e == hipSuccess) e = hipStreamEndCapture(c->gst, &g.g);
    c->st = user;
    if (s != DORY_OK || e != hipSuccess) {
      if (g.g) (void)hipGraphDestroy(g.g);
      if (s != DORY_OK) return s;
      return set_err(c, DORY_E_HIP, std::string("recording the decode step: ") + hipGetErrorString(e));
    }
    e = hipGraphInstantiate(&g.x, g.g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(g.g);
      return set_err(c, DORY_E_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    }
    c->graphs.push_back(g);
    x = g.x;
  }
  if (c->st) {
    // straight onto the caller's stream (a graph recorded on one stream runs on any)
    HIP_TRY(c, hipGraphLaunch(x, c->st));
  } else {
    // the legacy null stream: on the private stream, ordered after and before it by events
    HIP_TRY(c, hipEventRecord(c->gev[0], c->st));
    HIP_TRY(c, hipStreamWaitEvent(c->gst, c->gev[0], 0));
    HIP_TRY(c, hipGraphLaunch(x, c->gst));
    HIP_TRY(c, hipEventRecord(c->gev[1], c->gst));
    HIP_TRY(c, hipStreamWaitEvent(c->st, c->gev[1], 0));
  }
  c->has_logits = true;
  return DORY_OK;
}

// The new key's position for the decode attention: c->pos on an eager call;
// -1 (read the device counter) while the caller's stream is being captured,
// so that a graph recorded around dory_decode_step stays step-invariant.
int eager_position(dory_ctx* c) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(c->st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return -1;
  return c->pos;
}

dory_status check_call(dory_ctx* c, int B, int n, int n_loops, int kv_mode) {
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  if (kv_mode != c->kv.kv_mode)
    return set_err(c, DORY_E_KV_MODE, "kv mode differs from the one the KV buffer was laid out for");
  if (c->kv_mode_seq >= 0 && kv_mode != c->kv_mode_seq)
    return set_err(c, DORY_E_KV_MODE, "kv mode changed inside a sequence");
  if (n_loops < 1 || n_loops > C.max_loops) return set_err(c, DORY_E_LOOPS, "n_loops outside [1, max_loops]");
  if (kv_mode == DORY_KV_PER_LOOP) {
    if (n_loops > c->kv.kv_loops) return set_err(c, DORY_E_LOOPS, "n_loops exceeds the allocated per-loop caches");
    if (c->seq_loops && n_loops != c->seq_loops)
      return set_err(c, DORY_E_LOOPS, "per-loop caching needs one loop count for the whole sequence");
  }
  if (B < 1 || B > C.max_batch) return set_err(c, DORY_E_CAPACITY, "batch outside [1, max_batch]");
  if (c->pos > 0 && B != c->batch) return set_err(c, DORY_E_STATE, "batch changed inside a sequence");
  if ((int64_t)c->pos + n > C.max_ctx) return set_err(c, DORY_E_CAPACITY, "context overflow (pos + n > max_ctx)");
  if (c->trace) {
    const int apps = C.n_in + C.n_out + n_loops * C.n_rec;
    if (apps > c->trace_max) return set_err(c, DORY_E_CAPACITY, "trace buffer too small for this call");
  }
  return DORY_OK;
}

void commit_call(dory_ctx* c, int B, int n, int n_loops, int kv_mode) {
  c->batch = B;
  c->kv_mode_seq = kv_mode;
  if (kv_mode == DORY_KV_PER_LOOP) c->seq_loops = n_loops;
  c->pos += n;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// depth-1 truncated backward
// ---------------------------------------------------------------------------
struct Bw {
  dory_ctx* c;
  BwLayout L;
  char* ws;
  int B, n, M;
  template <typename P>
  P* f(size_t off) const { return (P*)(ws + off); }
  float* h_at(int i) const { return f<float>(L.hin) + (size_t)i * M * c->plan.cfg.d_model; }
};

// y[M][N] = x[M][K] . W[N][K]^T, float32 out, operands in the model dtype
// y [M][N] = x . W^T in float32. With `part` (room for M x N floats), a
// product whose output tiles would leave half of the CUs idle runs the two
// halves of its contraction side by side: the first half's sums land in y,
// the second's in part, and *y2 = part tells the caller to read y + part;
// otherwise *y2 = nullptr and y holds the product
dory_status bw_gemm(dory_ctx* c, const void* x, int64_t ldx, const void* W, float* y, int M, int N, int K,
                    float* part = nullptr, const float** y2 = nullptr) {
  const int dt = c->plan.cfg.dtype;
  if (y2) *y2 = nullptr;
  if (part && y2 && gemm_split2_pays(dt, M, N, K)) {
    HIP_TRY(c, launch_gemm_split2(x, ldx, W, y, part, M, N, K, 1.f, c->st));
    *y2 = part;
    return DORY_OK;
  }
  HIP_TRY(c, launch_linear(dt, x, ldx, W, y, M, N, K, 0, 1.f, 0, c->st));
  return DORY_OK;
}

// arguments of the matrix-core backward attention on this layer's buffers
BwFlash bw_flash_args(const Bw& b, bool full) {
  const Plan& P = b.c->plan;
  const dory_config& C = P.cfg;
  const BwLayout& L = b.L;
  BwFlash fa{};
  fa.Q = b.f<uint16_t>(L.fQ); fa.K = b.f<uint16_t>(L.fK); fa.V = b.f<uint16_t>(L.fV); fa.dO = b.f<uint16_t>(L.fdO);
  fa.QT = b.f<uint16_t>(L.fQT); fa.KT = b.f<uint16_t>(L.fKT); fa.VT = b.f<uint16_t>(L.fVT);
  fa.dOT = b.f<uint16_t>(L.fdOT);
  fa.B = b.B; fa.n = b.n; fa.nT = L.nT; fa.nq = C.n_q_heads; fa.nkv = C.n_kv_heads; fa.hd = C.head_dim;
  fa.window = full ? 0 : C.window;
  fa.scale = P.attn_scale;
  fa.mst = b.f<float>(L.mst); fa.lst = b.f<float>(L.lst); fa.D = b.f<float>(L.D);
  fa.o = b.f<float>(L.o); fa.dq = b.f<float>(L.dqn); fa.dk = b.f<float>(L.dkn); fa.dv = b.f<float>(L.dv);
  fa.dkh = b.f<float>(L.fdkh); fa.dvh = b.f<float>(L.fdvh);
  return fa;
}

// forward of recurrent layer l on h_in -> h_out, keeping what its backward reads
dory_status bw_layer_fwd(const Bw& b, int l, const float* h_in, float* h_out) {
  dory_ctx* c = b.c;
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const int dt = C.dtype, M = b.M, d = C.d_model, F = C.d_ff, Q = P.qkvg_dim, qd = P.q_dim;
  const BwLayout& L = b.L;
  hipStream_t st = c->st;
  const bool full = P.is_full[l];
  const float2* tab = wsp<float2>(c, full ? P.ws.rope_full : P.ws.rope_swa);
  HIP_TRY(c, launch_bw_cast(dt, h_in, b.ws + L.xb, (int64_t)M * d, st));
  DORY_TRY(bw_gemm(c, b.ws + L.xb, d, c->qkvg[l], b.f<float>(L.P1), M, Q, d));
  HIP_TRY(c, launch_bw_rope_norm_fwd(b.f<float>(L.P1), Q, tab, b.n, C.n_q_heads, C.n_kv_heads, C.head_dim, M,
                                     b.f<float>(L.qn), b.f<float>(L.kn), b.f<float>(L.rq), b.f<float>(L.rk), st));
  if (bw_flash_supported(dt, C.head_dim, C.n_q_heads, C.n_kv_heads)) {
    BwFlash fa = bw_flash_args(b, full);
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.qn), qd, 0, C.n_q_heads, C.head_dim, b.n, b.B, b.ws + L.fQ, st));
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.kn), P.kv_dim, 0, C.n_kv_heads, C.head_dim, b.n, b.B, b.ws + L.fK,
                                  st));
    HIP_TRY(c, launch_bw_heads_t(b.f<float>(L.P1), Q, qd + P.kv_dim, C.n_kv_heads, C.head_dim, b.n, b.B, L.nT,
                                 b.ws + L.fVT, st));
    HIP_TRY(c, launch_bw_flash_fwd(fa, st));
  } else {
    BwAttn a{b.f<float>(L.qn), b.f<float>(L.kn), b.f<float>(L.P1) + qd + P.kv_dim, Q, b.n, C.n_q_heads,
             C.n_kv_heads, C.head_dim, full ? 0 : C.window, P.attn_scale};
    HIP_TRY(c, launch_bw_attn_fwd(a, M, b.f<float>(L.o), b.f<float>(L.mst), b.f<float>(L.lst), st));
  }
  HIP_TRY(c, launch_bw_gate_fwd(dt, b.f<float>(L.o), b.f<float>(L.P1), Q, qd + 2 * P.kv_dim, C.attn_gate,
                                C.head_dim, qd, M, b.f<float>(L.oh), b.ws + L.ohb, b.f<float>(L.rc), st));
  const float* y2 = nullptr;
  DORY_TRY(bw_gemm(c, b.ws + L.ohb, qd, c->o[l], b.f<float>(L.y), M, d, qd, b.f<float>(L.part), &y2));
  HIP_TRY(c, launch_bw_update_fwd(dt, h_in, b.f<float>(L.y), c->alpha_attn[l], M, d, b.f<float>(L.yh),
                                  b.f<float>(L.ry), b.f<float>(L.rz), b.f<float>(L.h1), b.ws + L.h1b, st, y2));
  DORY_TRY(bw_gemm(c, b.ws + L.h1b, d, c->ug[l], b.f<float>(L.P2), M, 2 * F, d));
  HIP_TRY(c, launch_bw_swiglu_fwd(dt, b.f<float>(L.P2), F, M, b.f<float>(L.a32), b.ws + L.ab, b.f<float>(L.rs),
                                  st));
  DORY_TRY(bw_gemm(c, b.ws + L.ab, F, c->down[l], b.f<float>(L.y), M, d, F, b.f<float>(L.part), &y2));
  HIP_TRY(c, launch_bw_update_fwd(dt, b.f<float>(L.h1), b.f<float>(L.y), c->alpha_mlp[l], M, d, b.f<float>(L.y2h),
                                  b.f<float>(L.ry2), b.f<float>(L.rz2), h_out, nullptr, st, y2));
  return DORY_OK;
}

// dW [N][K] = dY^T X from dY [M][N] and X [M][K] (model dtype): both are
// transposed into TA / TB, then one GEMM over the M rows
dory_status bw_wgrad(const Bw& b, const void* dY, int N, const void* X, int K, float* dW) {
  dory_ctx* c = b.c;
  const int dt = c->plan.cfg.dtype;
  HIP_TRY(c, launch_bw_transpose(dt, dY, N, b.ws + b.L.TA, b.M, N, c->st));
  HIP_TRY(c, launch_bw_transpose(dt, X, K, b.ws + b.L.TB, b.M, K, c->st));
  return bw_gemm(c, b.ws + b.L.TA, b.M, b.ws + b.L.TB, dW, N, K, b.M);
}

// dX [M][K] = dY [M][N] . W [N][K]: W is transposed into WT, then one GEMM
// (split as bw_gemm says when dX2 is given and M x K floats fit its buffer:
// then dX + *dX2 is the gradient)
dory_status bw_xgrad(const Bw& b, const void* dY, const void* W, int N, int K, float* dX,
                     const float** dX2 = nullptr) {
  dory_ctx* c = b.c;
  HIP_TRY(c, launch_bw_transpose(c->plan.cfg.dtype, W, K, b.ws + b.L.WT, N, K, c->st));
  const Plan& P = c->plan;
  float* part = K <= std::max(P.cfg.d_model, P.q_dim) ? b.f<float>(b.L.part) : nullptr;
  return bw_gemm(c, dY, N, b.ws + b.L.WT, dX, b.M, K, N, part, dX2);
}

// backward of recurrent layer l (its forward values in the workspace):
// dho = dL/d(output) -> dhi = dL/d(input); gradients into g (index i)
dory_status bw_layer_bwd(const Bw& b, int l, int i, const float* h_in, const float* h_out, const float* dho,
                         float* dhi, const dory_grads* g) {
  dory_ctx* c = b.c;
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  const int dt = C.dtype, M = b.M, d = C.d_model, F = C.d_ff, Q = P.qkvg_dim, qd = P.q_dim;
  const BwLayout& L = b.L;
  hipStream_t st = c->st;
  const bool full = P.is_full[l];
  const float2* tab = wsp<float2>(c, full ? P.ws.rope_full : P.ws.rope_swa);
  float* tmp = b.f<float>(L.tmp);

  // MLP sublayer
  HIP_TRY(c, launch_bw_update_bwd(dt, dho, h_out, b.f<float>(L.rz2), b.f<float>(L.y2h), b.f<float>(L.ry2),
                                  b.f<float>(L.h1), c->alpha_mlp[l], M, d, b.f<float>(L.dres), b.ws + L.dyb,
                                  b.f<float>(L.contrib), st));
  HIP_TRY(c, launch_bw_colsum(b.f<float>(L.contrib), M, d, g->alpha_mlp[i], tmp, st));
  DORY_TRY(bw_wgrad(b, b.ws + L.dyb, d, b.ws + L.ab, F, g->down[i]));
  DORY_TRY(bw_xgrad(b, b.ws + L.dyb, c->down[l], d, F, tmp));                     // da [M][F]
  HIP_TRY(c, launch_bw_swiglu_bwd(dt, tmp, b.f<float>(L.a32), b.f<float>(L.rs), b.f<float>(L.P2), F, M,
                                  b.ws + L.dP2b, st));
  DORY_TRY(bw_wgrad(b, b.ws + L.dP2b, 2 * F, b.ws + L.h1b, d, g->ug[i]));
  const float* tmp2 = nullptr;
  DORY_TRY(bw_xgrad(b, b.ws + L.dP2b, c->ug[l], 2 * F, d, tmp, &tmp2));           // [M][d]
  float* dh1 = b.f<float>(L.dh2);
  HIP_TRY(c, launch_bw_add(b.f<float>(L.dres), tmp, dh1, (int64_t)M * d, st, tmp2));

  // attention sublayer
  HIP_TRY(c, launch_bw_update_bwd(dt, dh1, b.f<float>(L.h1), b.f<float>(L.rz), b.f<float>(L.yh), b.f<float>(L.ry),
                                  h_in, c->alpha_attn[l], M, d, b.f<float>(L.dres), b.ws + L.dyb,
                                  b.f<float>(L.contrib), st));
  HIP_TRY(c, launch_bw_colsum(b.f<float>(L.contrib), M, d, g->alpha_attn[i], tmp, st));
  DORY_TRY(bw_wgrad(b, b.ws + L.dyb, d, b.ws + L.ohb, qd, g->o[i]));
  DORY_TRY(bw_xgrad(b, b.ws + L.dyb, c->o[l], d, qd, tmp, &tmp2));                // doh [M][qd]
  HIP_TRY(c, launch_bw_gate_bwd(tmp, b.f<float>(L.oh), b.f<float>(L.rc), b.f<float>(L.o), b.f<float>(L.P1), Q,
                                qd + 2 * P.kv_dim, C.attn_gate, C.head_dim, qd, M, b.f<float>(L.dO),
                                b.f<float>(L.dP1), st, tmp2));
  if (bw_flash_supported(dt, C.head_dim, C.n_q_heads, C.n_kv_heads)) {
    // operand copies of this layer (the forward's may belong to another layer)
    const int nq = C.n_q_heads, nkv = C.n_kv_heads, hd = C.head_dim, kvd = P.kv_dim;
    HIP_TRY(c, launch_bw_attn_D(b.f<float>(L.dO), b.f<float>(L.o), nq, hd, M, b.f<float>(L.D), st));
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.qn), qd, 0, nq, hd, b.n, b.B, b.ws + L.fQ, st));
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.dO), qd, 0, nq, hd, b.n, b.B, b.ws + L.fdO, st));
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.kn), kvd, 0, nkv, hd, b.n, b.B, b.ws + L.fK, st));
    HIP_TRY(c, launch_bw_to_heads(1, b.f<float>(L.P1), Q, qd + kvd, nkv, hd, b.n, b.B, b.ws + L.fV, st));
    HIP_TRY(c, launch_bw_heads_t(b.f<float>(L.qn), qd, 0, nq, hd, b.n, b.B, L.nT, b.ws + L.fQT, st));
    HIP_TRY(c, launch_bw_heads_t(b.f<float>(L.dO), qd, 0, nq, hd, b.n, b.B, L.nT, b.ws + L.fdOT, st));
    HIP_TRY(c, launch_bw_heads_t(b.f<float>(L.kn), kvd, 0, nkv, hd, b.n, b.B, L.nT, b.ws + L.fKT, st));
    HIP_TRY(c, launch_bw_flash_bwd(bw_flash_args(b, full), st));
  } else {
    BwAttn a{b.f<float>(L.qn), b.f<float>(L.kn), b.f<float>(L.P1) + qd + P.kv_dim, Q, b.n, C.n_q_heads,
             C.n_kv_heads, C.head_dim, full ? 0 : C.window, P.attn_scale};
    HIP_TRY(c, launch_bw_attn_bwd(a, M, b.f<float>(L.dO), b.f<float>(L.o), b.f<float>(L.mst), b.f<float>(L.lst),
                                  b.f<float>(L.D), b.f<float>(L.dqn), b.f<float>(L.dkn), b.f<float>(L.dv), st));
  }
  HIP_TRY(c, launch_bw_rope_norm_bwd(b.f<float>(L.dqn), b.f<float>(L.qn), b.f<float>(L.rq), b.f<float>(L.dkn),
                                     b.f<float>(L.kn), b.f<float>(L.rk), b.f<float>(L.dv), tab, b.n, C.n_q_heads,
                                     C.n_kv_heads, C.head_dim, M, b.f<float>(L.dP1), Q, st));
  HIP_TRY(c, launch_bw_cast(dt, b.f<float>(L.dP1), b.ws + L.dP1b, (int64_t)M * Q, st));
  DORY_TRY(bw_wgrad(b, b.ws + L.dP1b, Q, b.ws + L.xb, d, g->qkvg[i]));
  DORY_TRY(bw_xgrad(b, b.ws + L.dP1b, c->qkvg[l], Q, d, tmp, &tmp2));             // [M][d]
  HIP_TRY(c, launch_bw_add(b.f<float>(L.dres), tmp, dhi, (int64_t)M * d, st, tmp2));
  return DORY_OK;
}

}  // namespace

extern "C" {

const char* dory_status_string(dory_status s) {
  switch (s) {
    case DORY_OK: return "ok";
    case DORY_E_ARG: return "invalid argument";
    case DORY_E_CAPACITY: return "capacity exceeded";
    case DORY_E_LOOPS: return "invalid loop count";
    case DORY_E_KV_MODE: return "invalid kv mode";
    case DORY_E_STATE: return "invalid state";
    case DORY_E_HIP: return "HIP error";
  }
  return "unknown status";
}

dory_status dory_validate_config(const dory_config* cfg) {
  Plan p;
  std::string why;
  return make_plan(cfg, &p, &why);
}

size_t dory_kv_bytes(const dory_config* cfg, int32_t kv_mode, int32_t kv_loops) {
  Plan p;
  if (make_plan(cfg, &p, nullptr) != DORY_OK) return 0;
  KvLayout kv;
  if (make_kv_layout(p, kv_mode, kv_loops, &kv, nullptr) != DORY_OK) return 0;
  return kv.bytes;
}

size_t dory_workspace_bytes(const dory_config* cfg) {
  Plan p;
  if (make_plan(cfg, &p, nullptr) != DORY_OK) return 0;
  return p.ws.total;
}

dory_status dory_kv_slot(const dory_config* cfg, int32_t kv_mode, int32_t kv_loops, int32_t layer, int32_t loop,
                         int32_t pos, int32_t* cache_id, int32_t* slot, int64_t* k_offset, int64_t* v_offset) {
  Plan p;
  dory_status s = make_plan(cfg, &p, nullptr);
  if (s != DORY_OK) return s;
  KvLayout kv;
  s = make_kv_layout(p, kv_mode, kv_loops, &kv, nullptr);
  if (s != DORY_OK) return s;
  if (layer < 0 || layer >= p.n_layers || pos < 0 || pos >= p.cfg.max_ctx) return DORY_E_ARG;
  int j = 0;
  if (p.recurrent(layer) && kv.kv_mode == DORY_KV_PER_LOOP) {
    if (loop < 1 || loop > kv.kv_loops) return DORY_E_LOOPS;
    j = loop - 1;
  }
  const int id = kv.first_id[layer] + j;
  const int sl = p.is_full[layer] ? pos : pos % p.cfg.window;
  const int64_t half = (int64_t)p.cfg.max_batch * p.cfg.n_kv_heads * p.slots(layer) * p.cfg.head_dim;
  if (cache_id) *cache_id = id;
  if (slot) *slot = sl;
  if (k_offset) *k_offset = kv.offset[id] + (int64_t)sl * p.cfg.head_dim;
  // values in 32-position blocks [hd][32]: dimension d at + 32 * d
  if (v_offset) *v_offset = kv.offset[id] + half + (int64_t)(sl / 32 * 32) * p.cfg.head_dim + sl % 32;
  return DORY_OK;
}

dory_status dory_create(const dory_config* cfg, const dory_weights* w, void* kv_dev, size_t kv_bytes,
                        int32_t kv_mode, int32_t kv_loops, void* ws_dev, size_t ws_bytes, void* stream,
                        dory_ctx** out) {
  if (!out) return DORY_E_ARG;
  *out = nullptr;
  dory_ctx* c = new dory_ctx();
  std::string why;
  dory_status s = make_plan(cfg, &c->plan, &why);
  if (s == DORY_OK) s = make_kv_layout(c->plan, kv_mode, kv_loops, &c->kv, &why);
  if (s != DORY_OK) {
    delete c;
    return s;
  }
  const Plan& P = c->plan;
  if (!w || !w->embed || !w->qkvg || !w->o || !w->ug || !w->down || !w->alpha_attn || !w->alpha_mlp || !kv_dev ||
      !ws_dev) {
    delete c;
    return DORY_E_ARG;
  }
  if (kv_bytes < c->kv.bytes || ws_bytes < P.ws.total || ((uintptr_t)kv_dev & 255) || ((uintptr_t)ws_dev & 255)) {
    delete c;
    return DORY_E_ARG;
  }
  c->embed = w->embed;
  for (int l = 0; l < P.n_layers; ++l) {
    if (!w->qkvg[l] || !w->o[l] || !w->ug[l] || !w->down[l] || !w->alpha_attn[l] || !w->alpha_mlp[l]) {
      delete c;
      return DORY_E_ARG;
    }
    c->qkvg.push_back(w->qkvg[l]);
    c->o.push_back(w->o[l]);
    c->ug.push_back(w->ug[l]);
    c->down.push_back(w->down[l]);
    const int fmt = P.cfg.weight_format;
    if (fmt != DORY_WEIGHTS_DTYPE) {
      const bool have = w->qkvg_scale && w->o_scale && w->ug_scale && w->down_scale;
      bool ok = have && w->qkvg_scale[l] && w->o_scale[l] && w->ug_scale[l] && w->down_scale[l] &&
                !((uintptr_t)w->qkvg[l] & 15) && !((uintptr_t)w->o[l] & 15) &&
                !((uintptr_t)w->ug[l] & 15) && !((uintptr_t)w->down[l] & 15);
      if (ok && fmt == DORY_WEIGHTS_NVFP4) {
        ok = w->qkvg_tscale && w->o_tscale && w->ug_tscale && w->down_tscale &&
             !((uintptr_t)w->qkvg_scale[l] & 1) && !((uintptr_t)w->o_scale[l] & 1) &&
             !((uintptr_t)w->ug_scale[l] & 1) && !((uintptr_t)w->down_scale[l] & 1);
        if (ok)
          for (float g : {w->qkvg_tscale[l], w->o_tscale[l], w->ug_tscale[l], w->down_tscale[l]})
            ok = ok && std::isfinite(g) && g > 0.f;
      }
      if (!ok) {
        delete c;
        return DORY_E_ARG;
      }
      c->qkvg_s.push_back(w->qkvg_scale[l]);
      c->o_s.push_back(w->o_scale[l]);
      c->ug_s.push_back(w->ug_scale[l]);
      c->down_s.push_back(w->down_scale[l]);
    } else {
      c->qkvg_s.push_back(nullptr);
      c->o_s.push_back(nullptr);
      c->ug_s.push_back(nullptr);
      c->down_s.push_back(nullptr);
    }
    const bool fp4 = fmt == DORY_WEIGHTS_NVFP4;
    c->qkvg_g.push_back(fp4 ? w->qkvg_tscale[l] : 1.f);
    c->o_g.push_back(fp4 ? w->o_tscale[l] : 1.f);
    c->ug_g.push_back(fp4 ? w->ug_tscale[l] : 1.f);
    c->down_g.push_back(fp4 ? w->down_tscale[l] : 1.f);
    c->alpha_attn.push_back(w->alpha_attn[l]);
    c->alpha_mlp.push_back(w->alpha_mlp[l]);
  }
  c->kvb = (char*)kv_dev;
  c->ws = (char*)ws_dev;
  c->st = (hipStream_t)stream;
  *out = c;
  return DORY_OK;
}

void dory_destroy(dory_ctx* ctx) { delete ctx; }

dory_status dory_reset(dory_ctx* c) {
  if (!c) return DORY_E_ARG;
  c->pos = 0;
  c->batch = 0;
  c->seq_loops = 0;
  c->kv_mode_seq = -1;
  c->has_logits = false;
  c->err.clear();
  return DORY_OK;
}

dory_status dory_resume(dory_ctx* c, int32_t batch, int32_t pos, int32_t n_loops, int32_t kv_mode) {
  if (!c) return DORY_E_ARG;
  const dory_config& C = c->plan.cfg;
  if (batch < 1 || batch > C.max_batch) return set_err(c, DORY_E_CAPACITY, "batch outside [1, max_batch]");
  if (pos < 1 || pos >= C.max_ctx) return set_err(c, DORY_E_CAPACITY, "pos outside [1, max_ctx - 1]");
  if (kv_mode != c->kv.kv_mode)
    return set_err(c, DORY_E_KV_MODE, "kv mode differs from the one the KV buffer was laid out for");
  if (n_loops < 1 || n_loops > C.max_loops) return set_err(c, DORY_E_LOOPS, "n_loops outside [1, max_loops]");
  if (kv_mode == DORY_KV_PER_LOOP && n_loops > c->kv.kv_loops)
    return set_err(c, DORY_E_LOOPS, "n_loops exceeds the allocated per-loop caches");
  c->err.clear();
  dory_status s = device_init(c);
  if (s != DORY_OK) return s;
  HIP_TRY(c, launch_set_pos(wsp<int>(c, c->plan.ws.pos), pos, c->st));
  c->pos = pos;
  c->batch = batch;
  c->kv_mode_seq = kv_mode;
  c->seq_loops = kv_mode == DORY_KV_PER_LOOP ? n_loops : 0;
  c->has_logits = false;
  return DORY_OK;
}

dory_status dory_prefill(dory_ctx* c, const int32_t* tokens_dev, int32_t batch, int32_t n, int32_t n_loops,
                         int32_t kv_mode) {
  if (!c) return DORY_E_ARG;
  if (!tokens_dev) return set_err(c, DORY_E_ARG, "tokens_dev is NULL");
  if (n < 0) return set_err(c, DORY_E_ARG, "n < 0");
  if (n == 0) return DORY_OK;
  dory_status s = check_call(c, batch, n, n_loops, kv_mode);
  if (s != DORY_OK) return s;
  c->err.clear();
  s = device_init(c);
  if (s != DORY_OK) return s;
  Range range(c, "dory_prefill n=%d k=%d", n, n_loops);
  const int chunk = c->plan.cfg.max_chunk;
  for (int s0 = 0; s0 < n; s0 += chunk) {
    const int m = std::min(chunk, n - s0);
    const bool last = s0 + m >= n;
    s = run_forward(c, tokens_dev + s0, n, batch, m, n_loops, last);
    if (s != DORY_OK) return s;
    commit_call(c, batch, m, n_loops, kv_mode);
  }
  HIP_TRY(c, launch_set_pos(wsp<int>(c, c->plan.ws.pos), c->pos, c->st));  // next decode position
  return DORY_OK;
}

dory_status dory_decode_step(dory_ctx* c, const int32_t* tokens_dev, int32_t n_loops, int32_t kv_mode,
                             int32_t* next_tokens_dev) {
  if (!c) return DORY_E_ARG;
  if (c->pos == 0) return set_err(c, DORY_E_STATE, "decode before prefill");
  if (!tokens_dev && !c->has_logits) return set_err(c, DORY_E_STATE, "no greedy tokens to continue from");
  dory_status s = check_call(c, c->batch, 1, n_loops, kv_mode);
  if (s != DORY_OK) return s;
  c->err.clear();
  const Plan& P = c->plan;
  const int32_t* tok = tokens_dev ? tokens_dev : wsp<int32_t>(c, P.ws.next);
  const bool fused = fused_decode_ok(c, c->batch);
  Range range(c, "dory_decode_step k=%d batch=%d", n_loops, c->batch);
  if (fused && c->graphs_on && !tokens_dev && c->time_kind == 0) {
    s = decode_graph(c, n_loops);
  } else {
    c->t_now = eager_position(c);
    s = fused ? run_decode_fused(c, tok, c->batch, n_loops)
              : run_forward(c, tok, 1, c->batch, 1, n_loops, true, true);
    c->t_now = -1;
  }
  if (s != DORY_OK) return s;
  commit_call(c, c->batch, 1, n_loops, kv_mode);
  if (next_tokens_dev)
    HIP_TRY(c, hipMemcpyAsync(next_tokens_dev, c->ws + P.ws.next, (size_t)c->batch * 4, hipMemcpyDeviceToDevice,
                              c->st));
  return DORY_OK;
}

namespace {

// Validates per-sequence loop counts (last-loop caches only) and stores them
// in the workspace; returns the largest count.
dory_status mixed_setup(dory_ctx* c, int B, const int32_t* loops_host, int kv_mode, int* kmax) {
  const dory_config& C = c->plan.cfg;
  if (!loops_host) return set_err(c, DORY_E_ARG, "loops is NULL");
  if (kv_mode != DORY_KV_LAST_LOOP || c->kv.kv_mode != DORY_KV_LAST_LOOP)
    return set_err(c, DORY_E_KV_MODE, "per-sequence loop counts need last-loop caching");
  if (B < 1 || B > C.max_batch) return set_err(c, DORY_E_CAPACITY, "batch outside [1, max_batch]");
  int km = 0;
  for (int b = 0; b < B; ++b) {
    if (loops_host[b] < 1 || loops_host[b] > C.max_loops)
      return set_err(c, DORY_E_LOOPS, "a loop count is outside [1, max_loops]");
    km = std::max(km, (int)loops_host[b]);
  }
  *kmax = km;
  return DORY_OK;
}

dory_status mixed_upload(dory_ctx* c, int B, const int32_t* loops_host) {
  int* dst = wsp<int>(c, c->plan.ws.rowk);
  for (int b0 = 0; b0 < B; b0 += 64) {
    RowLoops a{};
    a.n = std::min(64, B - b0);
    for (int i = 0; i < a.n; ++i) a.k[i] = loops_host[b0 + i];
    HIP_TRY(c, launch_set_rows(dst + b0, a, c->st));
  }
  return DORY_OK;
}

struct MixedScope {
  dory_ctx* c;
  explicit MixedScope(dory_ctx* ctx) : c(ctx) { c->mixed = true; }
  ~MixedScope() { c->mixed = false; }
};

}  // namespace

dory_status dory_prefill_mixed(dory_ctx* c, const int32_t* tokens_dev, int32_t batch, int32_t n,
                               const int32_t* loops_host, int32_t kv_mode) {
  if (!c) return DORY_E_ARG;
  if (!tokens_dev) return set_err(c, DORY_E_ARG, "tokens_dev is NULL");
  if (n < 0) return set_err(c, DORY_E_ARG, "n < 0");
  int kmax = 0;
  dory_status s = mixed_setup(c, batch, loops_host, kv_mode, &kmax);
  if (s != DORY_OK) return s;
  if (n == 0) return DORY_OK;
  s = check_call(c, batch, n, kmax, kv_mode);
  if (s != DORY_OK) return s;
  c->err.clear();
  s = device_init(c);
  if (s != DORY_OK) return s;
  s = mixed_upload(c, batch, loops_host);
  if (s != DORY_OK) return s;
  MixedScope ms(c);
  const int chunk = c->plan.cfg.max_chunk;
  for (int s0 = 0; s0 < n; s0 += chunk) {
    const int m = std::min(chunk, n - s0);
    s = run_forward(c, tokens_dev + s0, n, batch, m, kmax, s0 + m >= n);
    if (s != DORY_OK) return s;
    commit_call(c, batch, m, kmax, kv_mode);
  }
  HIP_TRY(c, launch_set_pos(wsp<int>(c, c->plan.ws.pos), c->pos, c->st));
  return DORY_OK;
}

dory_status dory_decode_step_mixed(dory_ctx* c, const int32_t* tokens_dev, const int32_t* loops_host,
                                   int32_t kv_mode, int32_t* next_tokens_dev) {
  if (!c) return DORY_E_ARG;
  if (c->pos == 0) return set_err(c, DORY_E_STATE, "decode before prefill");
  if (!tokens_dev && !c->has_logits) return set_err(c, DORY_E_STATE, "no greedy tokens to continue from");
  int kmax = 0;
  dory_status s = mixed_setup(c, c->batch, loops_host, kv_mode, &kmax);
  if (s != DORY_OK) return s;
  s = check_call(c, c->batch, 1, kmax, kv_mode);
  if (s != DORY_OK) return s;
  c->err.clear();
  s = mixed_upload(c, c->batch, loops_host);
  if (s != DORY_OK) return s;
  {
    MixedScope ms(c);
    const int32_t* tok = tokens_dev ? tokens_dev : wsp<int32_t>(c, c->plan.ws.next);
    s = run_forward(c, tok, 1, c->batch, 1, kmax, true, true);
  }
  if (s != DORY_OK) return s;
  commit_call(c, c->batch, 1, kmax, kv_mode);
  if (next_tokens_dev)
    HIP_TRY(c, hipMemcpyAsync(next_tokens_dev, c->ws + c->plan.ws.next, (size_t)c->batch * 4,
                              hipMemcpyDeviceToDevice, c->st));
  return DORY_OK;
}

dory_status dory_logits(dory_ctx* c, float* out_dev) {
  if (!c || !out_dev) return DORY_E_ARG;
  if (!c->has_logits) return set_err(c, DORY_E_STATE, "no logits before prefill");
  HIP_TRY(c, hipMemcpyAsync(out_dev, c->ws + c->plan.ws.logits, (size_t)c->batch * c->plan.cfg.vocab * 4,
                            hipMemcpyDeviceToDevice, c->st));
  return DORY_OK;
}

const char* dory_last_error(const dory_ctx* c) { return c ? c->err.c_str() : "null context"; }

dory_status dory_set_trace(dory_ctx* c, float* trace_dev, int32_t max_apps) {
  if (!c) return DORY_E_ARG;
  if (trace_dev && max_apps < 1) return DORY_E_ARG;
  c->trace = trace_dev;
  c->trace_max = trace_dev ? max_apps : 0;
  return DORY_OK;
}

dory_status dory_set_markers(dory_ctx* c, int32_t enable) {
  if (!c) return DORY_E_ARG;
  if (enable && !roctx_api().push) return set_err(c, DORY_E_ARG, "no ROCm marker (roctx) library could be loaded");
  c->markers = enable != 0;
  return DORY_OK;
}

dory_status dory_set_graphs(dory_ctx* c, int32_t enable) {
  if (!c) return DORY_E_ARG;
  c->graphs_on = enable != 0;
  if (!c->graphs_on) c->drop_graphs();
  return DORY_OK;
}

dory_status dory_set_kernel_timing(dory_ctx* c, int32_t kind, int32_t max_launches) {
  if (!c) return DORY_E_ARG;
  if (kind < TIME_NONE || kind > TIME_ATTN || (kind != TIME_NONE && max_launches < 1)) return DORY_E_ARG;
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  c->ev.clear();
  c->ev_used = 0;
  c->time_kind = TIME_NONE;
  if (kind == TIME_NONE) return DORY_OK;
  c->ev.resize((size_t)2 * max_launches);
  for (auto& e : c->ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      c->ev.clear();
      return set_err(c, DORY_E_HIP, std::string("hipEventCreate: ") + hipGetErrorString(r));
    }
  }
  c->time_kind = kind;
  return DORY_OK;
}

dory_status dory_kernel_time(dory_ctx* c, double* total_ms, int32_t* launches) {
  if (!c || !total_ms || !launches) return DORY_E_ARG;
  HIP_TRY(c, hipStreamSynchronize(c->st));
  double t = 0.0;
  for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
    float ms = 0.f;
    HIP_TRY(c, hipEventElapsedTime(&ms, c->ev[i], c->ev[i + 1]));
    t += ms;
  }
  *total_ms = t;
  *launches = (int32_t)(c->ev_used / 2);
  c->ev_used = 0;
  return DORY_OK;
}

dory_status dory_op_linear(int32_t dtype, const void* x, int64_t ldx, const void* W, void* y, int32_t M, int32_t N,
                           int32_t K, int32_t epilogue, float scale, int32_t algo, void* stream) {
  if (!x || !W || !y) return DORY_E_ARG;
  if ((dtype != DORY_F32 && dtype != DORY_BF16) || M < 0 || N < 1 || K < 1 || ldx < K) return DORY_E_ARG;
  if (epilogue != 0 && epilogue != 1) return DORY_E_ARG;
  if (epilogue == 1 && N % 2) return DORY_E_ARG;
  if (algo < 0 || algo > 2) return DORY_E_ARG;
  hipError_t e = launch_linear(dtype, x, ldx, W, y, M, N, K, epilogue, scale, algo, (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

size_t dory_argmax_scratch_bytes(int32_t B, int32_t V) { return B > 0 && V > 0 ? argmax_partials(B, V) * 8 : 0; }

dory_status dory_op_argmax(const float* logits, int32_t B, int32_t V, int32_t* out, void* scratch, void* stream) {
  if (!logits || !out || !scratch || B < 1 || V < 1) return DORY_E_ARG;
  hipError_t e = launch_argmax(logits, B, V, out, scratch, (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

dory_status dory_op_quant_mxfp8(const void* w_dev, int32_t N, int32_t K, void* codes_dev, void* scales_dev,
                                void* stream) {
  if (!w_dev || !codes_dev || !scales_dev || N < 0 || K < 32 || K % 32) return DORY_E_ARG;
  hipError_t e = launch_quant_mxfp8(w_dev, N, K, codes_dev, scales_dev, (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : (e == hipErrorInvalidValue ? DORY_E_ARG : DORY_E_HIP);
}

dory_status dory_op_linear_mx(const void* x, int64_t ldx, const void* codes, const void* scales, void* y,
                              int32_t M, int32_t N, int32_t K, int32_t epilogue, float scale, void* stream) {
  if (!x || !codes || !scales || !y || M < 1 || M > 8 || N < 1 || K < 32 || K % 32 || ldx < K) return DORY_E_ARG;
  if (epilogue != 0 && epilogue != 1) return DORY_E_ARG;
  if (epilogue == 1 && N % 2) return DORY_E_ARG;
  if (!linear_lowbit_supported(DORY_WEIGHTS_MXFP8, M, K)) return DORY_E_ARG;
  hipError_t e = launch_linear_lowbit(DORY_WEIGHTS_MXFP8, x, ldx, codes, scales, y, M, N, K, epilogue, scale,
                                      (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : (e == hipErrorInvalidValue ? DORY_E_ARG : DORY_E_HIP);
}

size_t dory_backward_workspace_bytes(const dory_config* cfg, int32_t batch, int32_t n) {
  Plan p;
  if (!cfg || batch < 1 || n < 1 || (int64_t)batch * n > kMaxBwRows || make_plan(cfg, &p, nullptr) != DORY_OK)
    return 0;
  return make_bw_layout(p, batch, n, true).total;
}

size_t dory_backward_workspace_min_bytes(const dory_config* cfg, int32_t batch, int32_t n) {
  Plan p;
  if (!cfg || batch < 1 || n < 1 || (int64_t)batch * n > kMaxBwRows || make_plan(cfg, &p, nullptr) != DORY_OK)
    return 0;
  return make_bw_layout(p, batch, n, false).total;
}

dory_status dory_backward_last_loop(dory_ctx* c, const float* x, const float* grad_out, int32_t batch, int32_t n,
                                    const dory_grads* g, float* grad_x, void* ws_dev, size_t ws_bytes) {
  if (!c) return DORY_E_ARG;
  const Plan& P = c->plan;
  const dory_config& C = P.cfg;
  if (!x || !grad_out || !g || !ws_dev || batch < 1 || n < 1 || n > C.max_ctx)
    return set_err(c, DORY_E_ARG, "backward: bad arguments");
  if (C.weight_format != DORY_WEIGHTS_DTYPE || (C.head_dim != 64 && C.head_dim != 128) || C.n_rec < 1)
    return set_err(c, DORY_E_ARG, "backward: needs dtype weights, head_dim 64 or 128 and a recurrent block");
  if ((int64_t)batch * n > kMaxBwRows) return set_err(c, DORY_E_ARG, "backward: batch * n too large");
  if (!g->qkvg || !g->o || !g->ug || !g->down || !g->alpha_attn || !g->alpha_mlp)
    return set_err(c, DORY_E_ARG, "backward: null gradient array");
  for (int i = 0; i < C.n_rec; ++i)
    if (!g->qkvg[i] || !g->o[i] || !g->ug[i] || !g->down[i] || !g->alpha_attn[i] || !g->alpha_mlp[i])
      return set_err(c, DORY_E_ARG, "backward: null gradient pointer");
  // every layer's forward values kept when the workspace holds them, else
  // each layer's forward runs again just before its backward
  const bool stored = ws_bytes >= make_bw_layout(P, batch, n, true).total;
  Bw b{c, make_bw_layout(P, batch, n, stored), (char*)ws_dev, batch, n, batch * n};
  if (ws_bytes < b.L.total || ((uintptr_t)ws_dev & (kAlign - 1)))
    return set_err(c, DORY_E_ARG, "backward: workspace too small or misaligned");
  DORY_TRY(device_init(c));
  auto at = [&](int i) { return Bw{b.c, bw_layer_view(b.L, i), b.ws, b.B, b.n, b.M}; };
  const size_t rows = (size_t)b.M * C.d_model;
  Range range(c, "dory_backward_last_loop rows=%d", b.M);
  HIP_TRY(c, hipMemcpyAsync(b.h_at(0), x, rows * 4, hipMemcpyDeviceToDevice, c->st));
  for (int i = 0; i < C.n_rec; ++i) {
    Range r(c, "forward layer %d", C.n_in + i);
    DORY_TRY(bw_layer_fwd(at(i), C.n_in + i, b.h_at(i), b.h_at(i + 1)));
  }
  float* dh = b.f<float>(b.L.dh);
  HIP_TRY(c, launch_bw_final(b.h_at(C.n_rec), grad_out, b.M, C.d_model, dh, c->st));
  for (int i = C.n_rec - 1; i >= 0; --i) {
    Range r(c, "backward layer %d", C.n_in + i);
    if (!stored && i < C.n_rec - 1) DORY_TRY(bw_layer_fwd(b, C.n_in + i, b.h_at(i), b.h_at(i + 1)));  // recompute
    DORY_TRY(bw_layer_bwd(at(i), C.n_in + i, i, b.h_at(i), b.h_at(i + 1), dh, dh, g));
  }
  if (grad_x) HIP_TRY(c, hipMemcpyAsync(grad_x, dh, rows * 4, hipMemcpyDeviceToDevice, c->st));
  return DORY_OK;
}

dory_status dory_op_quant_nvfp4(const void* w_dev, int32_t N, int32_t K, void* codes_dev, void* scales_dev,
                                float* tscale_dev, void* stream) {
  if (!w_dev || !codes_dev || !scales_dev || !tscale_dev || N < 0 || K < 32 || K % 32) return DORY_E_ARG;
  hipError_t e = launch_quant_nvfp4(w_dev, N, K, codes_dev, scales_dev, tscale_dev, (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : (e == hipErrorInvalidValue ? DORY_E_ARG : DORY_E_HIP);
}

dory_status dory_op_linear_fp4(const void* x, int64_t ldx, const void* codes, const void* scales, void* y,
                               int32_t M, int32_t N, int32_t K, int32_t epilogue, float scale, void* stream) {
  if (!x || !codes || !scales || !y || M < 1 || M > 8 || N < 1 || K < 32 || K % 32 || ldx < K) return DORY_E_ARG;
  if (epilogue != 0 && epilogue != 1) return DORY_E_ARG;
  if (epilogue == 1 && N % 2) return DORY_E_ARG;
  if (!linear_lowbit_supported(DORY_WEIGHTS_NVFP4, M, K)) return DORY_E_ARG;
  hipError_t e = launch_linear_lowbit(DORY_WEIGHTS_NVFP4, x, ldx, codes, scales, y, M, N, K, epilogue, scale,
                                      (hipStream_t)stream);
  return e == hipSuccess ? DORY_OK : (e == hipErrorInvalidValue ? DORY_E_ARG : DORY_E_HIP);
}

}  // extern "C"
