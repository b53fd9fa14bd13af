// Host-only plan: validation, KV layout, workspace layout (no HIP calls).
#include "plan.h"

#include "kernels.h"

#include <algorithm>

#include <cmath>
#include <cstring>

namespace dory {

int Plan::slots(int l) const {
  if (is_full[l]) return cfg.max_ctx;
  return cfg.window < cfg.max_ctx ? cfg.window : cfg.max_ctx;
}

static dory_status fail(std::string* why, const char* msg) {
  if (why) *why = msg;
  return DORY_E_ARG;
}

dory_status make_plan(const dory_config* c, Plan* p, std::string* why) {
  if (!c) return fail(why, "config is NULL");
  if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->d_ff <= 0 || c->vocab <= 0)
    return fail(why, "model sizes must be positive");
  if (c->d_model > kMaxDModel || c->d_ff > kMaxDFF || c->n_q_heads > kMaxHeads || c->vocab > kMaxVocab)
    return fail(why, "model sizes beyond the library's limits (d_model, d_ff, heads, vocab)");
  if (c->n_in < 0 || c->n_rec < 0 || c->n_out < 0 || (int64_t)c->n_in + c->n_rec + c->n_out < 1)
    return fail(why, "layer split must be non-negative with at least one layer");
  if (c->n_in > kMaxLayers || c->n_rec > kMaxLayers || c->n_out > kMaxLayers)
    return fail(why, "more layers per block than the library's limit");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(why, "head_dim must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads != 0) return fail(why, "n_q_heads must be a multiple of n_kv_heads");
  {
    const int g = c->n_q_heads / c->n_kv_heads;
    if (g != 1 && g != 2 && g != 3 && g != 4 && g != 6 && g != 8)
      return fail(why, "query heads per kv head must be 1, 2, 3, 4, 6 or 8");
  }
  if (c->window < 1) return fail(why, "window must be >= 1");
  if (!c->layer_is_full) return fail(why, "layer_is_full is NULL");
  if (c->dtype != DORY_F32 && c->dtype != DORY_BF16) return fail(why, "dtype must be DORY_F32 or DORY_BF16");
  if (c->attn_gate < 0 || c->attn_gate > 2) return fail(why, "attn_gate must be 0, 1 or 2");
  if (!(c->rope_base_swa > 1.0) || !(c->rope_base_full > 1.0) || !std::isfinite(c->rope_base_swa) ||
      !std::isfinite(c->rope_base_full))
    return fail(why, "RoPE bases must be finite and > 1");
  if (c->max_batch < 1 || c->max_ctx < 1 || c->max_chunk < 1 || c->max_loops < 1)
    return fail(why, "capacities must be >= 1");
  if (c->max_batch > kMaxBatch || c->max_ctx > kMaxCtx || c->max_loops > kMaxLoops)
    return fail(why, "capacities beyond the library's limits (max_batch, max_ctx, max_loops)");
  // elements of one cache (keys and value blocks) within 2^40, so that every
  // KV offset and byte count stays far inside 64 bits
  if ((int64_t)c->max_batch * c->n_kv_heads * c->head_dim * 2 * ((int64_t)c->max_ctx + 32) > ((int64_t)1 << 40))
    return fail(why, "KV cache too large");
  if (c->max_chunk > c->max_ctx) return fail(why, "max_chunk must not exceed max_ctx");
  if (c->dtype == DORY_BF16 && (c->d_model % 8 || c->d_ff % 8 || c->head_dim % 8))
    return fail(why, "bfloat16 models need d_model, d_ff and head_dim multiples of 8");
  if ((int64_t)c->max_batch * c->max_chunk > (1 << 24)) return fail(why, "max_batch * max_chunk too large");
  if (!std::isfinite(c->combine_wh) || !std::isfinite(c->combine_we)) return fail(why, "combine weights must be finite");
  if (!std::isfinite(c->attn_scale) || !std::isfinite(c->logit_scale))
    return fail(why, "attn_scale and logit_scale must be finite (<= 0 selects the default)");
  if (c->weight_format != DORY_WEIGHTS_DTYPE && c->weight_format != DORY_WEIGHTS_MXFP8 &&
      c->weight_format != DORY_WEIGHTS_NVFP4)
    return fail(why, "weight_format must be DORY_WEIGHTS_DTYPE, DORY_WEIGHTS_MXFP8 or DORY_WEIGHTS_NVFP4");
  if (c->weight_format != DORY_WEIGHTS_DTYPE &&
      (c->dtype != DORY_BF16 || c->d_model % 32 || (c->n_q_heads * c->head_dim) % 32 || c->d_ff % 32 ||
       c->d_model > 8192))
    return fail(why, "low-bit weights need bfloat16, d_model <= 8192 and d_model, n_q*hd, d_ff multiples of 32");

  p->cfg = *c;
  p->n_layers = c->n_in + c->n_rec + c->n_out;
  p->is_full.assign(c->layer_is_full, c->layer_is_full + p->n_layers);
  for (auto& f : p->is_full) f = f ? 1 : 0;
  p->cfg.layer_is_full = nullptr;  // the plan keeps its own copy
  p->q_dim = c->n_q_heads * c->head_dim;
  p->kv_dim = c->n_kv_heads * c->head_dim;
  p->gate_dim = c->attn_gate == 1 ? p->q_dim : (c->attn_gate == 2 ? c->n_q_heads : 0);
  p->qkvg_dim = p->q_dim + 2 * p->kv_dim + p->gate_dim;
  p->elem = c->dtype == DORY_F32 ? 4 : 2;
  p->max_rows = c->max_batch * c->max_chunk;
  p->attn_scale = c->attn_scale > 0.f ? c->attn_scale : std::sqrt((float)c->head_dim);
  p->logit_scale = c->logit_scale > 0.f ? c->logit_scale : std::sqrt((float)c->d_model);
  p->ws = make_ws_layout(*p);
  return DORY_OK;
}

dory_status make_kv_layout(const Plan& p, int kv_mode, int kv_loops, KvLayout* kv, std::string* why) {
  if (kv_mode != DORY_KV_PER_LOOP && kv_mode != DORY_KV_LAST_LOOP) {
    if (why) *why = "unknown kv mode";
    return DORY_E_KV_MODE;
  }
  if (kv_mode == DORY_KV_LAST_LOOP) kv_loops = 1;
  if (kv_loops < 1 || kv_loops > p.cfg.max_loops) {
    if (why) *why = "kv_loops must be in [1, max_loops]";
    return DORY_E_LOOPS;
  }
  kv->kv_mode = kv_mode;
  kv->kv_loops = kv_loops;
  kv->first_id.assign(p.n_layers, 0);
  kv->n_ids.assign(p.n_layers, 1);
  kv->offset.clear();
  kv->id_layer.clear();
  int64_t off = 0;
  const int64_t per_slot = (int64_t)p.cfg.max_batch * p.cfg.n_kv_heads * p.cfg.head_dim;
  for (int l = 0; l < p.n_layers; ++l) {
    kv->first_id[l] = (int)kv->offset.size();
    kv->n_ids[l] = (p.recurrent(l) && kv_mode == DORY_KV_PER_LOOP) ? kv_loops : 1;
    for (int j = 0; j < kv->n_ids[l]; ++j) {
      kv->offset.push_back(off);
      kv->id_layer.push_back(l);
      off += per_slot * ((int64_t)p.slots(l) + p.vslots(l));  // K rows, then value blocks
    }
  }
  kv->bytes = (size_t)off * p.elem;
  return DORY_OK;
}

size_t argmax_partials(int32_t B, int32_t V) {
  return (size_t)B * (size_t)(((int64_t)V + kArgmaxBlock - 1) / kArgmaxBlock);
}

WsLayout make_ws_layout(const Plan& p) {
  WsLayout w;
  const auto& c = p.cfg;
  const size_t R = (size_t)p.max_rows;
  const size_t el = p.elem;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    size_t o = at;
    at = align_up(at + (bytes ? bytes : 1));
    return o;
  };
  const size_t rope = (size_t)c.max_ctx * (c.head_dim / 2) * 8;
  w.rope_swa = take(rope);
  w.rope_full = take(rope);
  w.h = take(R * c.d_model * 4);
  w.e = take(R * c.d_model * 4);
  w.xb = take(R * c.d_model * el);
  w.hb = take((size_t)c.max_batch * c.d_model * 4);
  w.qkvg = take(R * p.qkvg_dim * 4);
  w.q = take(R * p.q_dim * el);
  w.kw = take(R * p.kv_dim * el);
  w.vw = take((size_t)c.max_batch * chunk_vld(c.max_chunk) * p.kv_dim * el);  // V^T rows of chunk_vld(n)
  const size_t dec = (size_t)c.max_batch * c.n_q_heads * kMaxSplits;
  const size_t pre = R * c.n_q_heads;
  w.part = take((dec > pre ? dec : pre) * (c.head_dim + 2) * 4);
  w.ob = take(R * p.q_dim * el);
  w.y = take(R * c.d_model * 4);
  w.y1 = take(std::min<size_t>(R, 64) * c.d_model * 4);
  w.a = take(R * c.d_ff * el);
  w.logits = take((size_t)c.max_batch * c.vocab * 4);
  w.next = take((size_t)c.max_batch * 4);
  w.amax = take(argmax_partials(c.max_batch, c.vocab) * 8);
  w.flags = take(256);
  w.pos = take(4);
  w.rowk = take((size_t)c.max_batch * 4);
  w.attn_acc = take((size_t)std::min(c.max_batch, 8) * c.n_q_heads * attn_acc_stride(c.head_dim, kAttnAccBinsMax) * 8);
  if (c.weight_format != DORY_WEIGHTS_DTYPE) {  // one projection expanded to bfloat16 for prefill GEMMs
    const size_t d = c.d_model;
    size_t big = (size_t)p.qkvg_dim * d;
    big = std::max(big, d * (size_t)p.q_dim);
    big = std::max(big, 2 * (size_t)c.d_ff * d);
    w.wdq = take(big * 2);
  }
  w.total = at;
  return w;
}

BwLayout make_bw_layout(const Plan& p, int B, int n, bool stored) {
  BwLayout w;
  const auto& c = p.cfg;
  const size_t M = (size_t)B * n, d = c.d_model, F = c.d_ff, Q = p.qkvg_dim, qd = p.q_dim, kvd = p.kv_dim;
  const size_t nq = c.n_q_heads, el = p.elem;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    size_t o = at;
    at = align_up(at + (bytes ? bytes : 1));
    return o;
  };
  // scratch shared by the layers
  w.hin = take((size_t)(c.n_rec + 1) * M * d * 4);
  w.y = take(M * d * 4);
  w.dres = take(M * d * 4);
  w.contrib = take(M * d * 4);
  w.tmp = take(M * std::max(d, std::max(F, qd)) * 4);
  w.part = take(M * std::max(d, qd) * 4);
  w.dh = take(M * d * 4);
  w.dh2 = take(M * d * 4);
  w.dO = take(M * qd * 4);
  w.D = take(M * nq * 4);
  w.dqn = take(M * qd * 4);
  w.dkn = take(M * kvd * 4);
  w.dv = take(M * kvd * 4);
  w.dP1 = take(M * Q * 4);
  w.dyb = take(M * d * el);
  w.dP2b = take(M * 2 * F * el);
  w.dP1b = take(M * Q * el);
  w.TA = take(M * std::max(Q, std::max(2 * F, d)) * el);
  w.TB = take(M * std::max(d, std::max(F, qd)) * el);
  w.WT = take(std::max(std::max(Q * d, 2 * F * d), std::max(d * qd, d * F)) * el);
  if (c.dtype == DORY_BF16) {
    w.nT = (n + 7) / 8 * 8;
    const size_t rowsT = (size_t)B * w.nT;
    w.fQ = take(M * qd * 2);
    w.fdO = take(M * qd * 2);
    w.fK = take(M * kvd * 2);
    w.fV = take(M * kvd * 2);
    w.fQT = take(rowsT * qd * 2);
    w.fdOT = take(rowsT * qd * 2);
    w.fKT = take(rowsT * kvd * 2);
    w.fVT = take(rowsT * kvd * 2);
    w.fdkh = take(M * qd * 4);
    w.fdvh = take(M * qd * 4);
  }
  // one layer's forward values
  const size_t g0 = at;
  w.P1 = take(M * Q * 4);
  w.qn = take(M * qd * 4);
  w.kn = take(M * kvd * 4);
  w.rq = take(M * nq * 4);
  w.rk = take(M * c.n_kv_heads * 4);
  w.o = take(M * qd * 4);
  w.mst = take(M * nq * 4);
  w.lst = take(M * nq * 4);
  w.oh = take(M * qd * 4);
  w.rc = take(M * 4);
  w.yh = take(M * d * 4);
  w.ry = take(M * 4);
  w.rz = take(M * 4);
  w.h1 = take(M * d * 4);
  w.P2 = take(M * 2 * F * 4);
  w.a32 = take(M * F * 4);
  w.rs = take(M * 4);
  w.y2h = take(M * d * 4);
  w.ry2 = take(M * 4);
  w.rz2 = take(M * 4);
  w.xb = take(M * d * el);
  w.ohb = take(M * qd * el);
  w.h1b = take(M * d * el);
  w.ab = take(M * F * el);
  w.layer_bytes = at - g0;
  w.stored = stored;
  w.total = at + (stored ? (size_t)(c.n_rec - 1) * w.layer_bytes : 0);
  return w;
}

BwLayout bw_layer_view(const BwLayout& L, int i) {
  BwLayout v = L;
  if (!L.stored || i == 0) return v;
  const size_t s = (size_t)i * L.layer_bytes;
  for (size_t* f : {&v.P1, &v.qn, &v.kn, &v.rq, &v.rk, &v.o, &v.mst, &v.lst, &v.oh, &v.rc, &v.yh, &v.ry, &v.rz,
                    &v.h1, &v.P2, &v.a32, &v.rs, &v.y2h, &v.ry2, &v.rz2, &v.xb, &v.ohb, &v.h1b, &v.ab})
    *f += s;
  return v;
}

}  // namespace dory
