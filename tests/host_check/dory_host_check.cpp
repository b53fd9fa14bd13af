// Host-side check of the library's validation, layout and offset arithmetic,
// built with AddressSanitizer and UndefinedBehaviorSanitizer and run by
// tests/test_host_sanitizers.py. It calls only entry points that make no HIP
// call on the paths taken here (queries, argument errors, contexts over
// host memory that no call dereferences):
//   * seeded random configurations: every KV element that dory_kv_slot's
//     offsets address (all caches, batch rows, kv heads, slots, dimensions)
//     lies inside dory_kv_bytes and belongs to exactly one cache position;
//     ring slots are pos mod window, full slots pos;
//   * the same queries on configurations with one field pushed to an extreme
//     (zero, negative, INT32_MAX, huge products): no undefined behaviour, and
//     whatever is accepted has consistent, non-overflowing sizes;
//   * every documented argument error of the context calls.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "dory.h"

namespace {

int g_fail = 0;
long g_checks = 0;

#define CHECK(cond, ...)                                         \
  do {                                                           \
    ++g_checks;                                                  \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "FAIL line %d: ", __LINE__);          \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fputc('\n', stderr);                                  \
      if (++g_fail > 50) std::exit(1);                           \
    }                                                            \
  } while (0)

struct Rng {  // 64-bit LCG (Knuth's MMIX constants), upper bits
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 2862933555777941757ULL + 3037000493ULL) {}
  uint32_t next() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(s >> 33);
  }
  int range(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }
};

struct Cfg {
  dory_config c{};
  std::vector<uint8_t> full;
  void bind() { c.layer_is_full = full.data(); }
};

Cfg tiny_cfg() {
  Cfg k;
  dory_config& c = k.c;
  c.d_model = 128; c.n_q_heads = 4; c.n_kv_heads = 2; c.head_dim = 64; c.d_ff = 96; c.vocab = 256;
  c.n_in = 1; c.n_rec = 2; c.n_out = 1; c.window = 5;
  c.rope_base_swa = 1e4; c.rope_base_full = 1e6; c.dtype = DORY_BF16; c.attn_gate = 1;
  c.attn_scale = 0.f; c.logit_scale = 0.f; c.combine_wh = 1.f; c.combine_we = 1.f;
  c.max_batch = 2; c.max_ctx = 64; c.max_chunk = 16; c.max_loops = 4; c.weight_format = DORY_WEIGHTS_DTYPE;
  k.full = {0, 0, 1, 0};
  k.bind();
  return k;
}

Cfg random_cfg(Rng& r) {
  Cfg k = tiny_cfg();
  dory_config& c = k.c;
  static const int groups[] = {1, 2, 3, 4, 6, 8};
  c.head_dim = r.range(0, 1) ? 64 : 128;
  c.n_kv_heads = r.range(1, 3);
  c.n_q_heads = c.n_kv_heads * groups[r.range(0, 5)];
  c.d_model = 8 * r.range(1, 40);
  c.d_ff = 8 * r.range(1, 40);
  c.vocab = r.range(1, 300);
  c.n_in = r.range(0, 2); c.n_rec = r.range(0, 3); c.n_out = r.range(0, 2);
  if (c.n_in + c.n_rec + c.n_out == 0) c.n_rec = 1;
  c.window = r.range(1, 80);
  c.dtype = r.range(0, 1) ? DORY_BF16 : DORY_F32;
  c.attn_gate = r.range(0, 2);
  c.max_batch = r.range(1, 3);
  c.max_ctx = r.range(1, 150);
  c.max_chunk = r.range(1, c.max_ctx);
  c.max_loops = r.range(1, 4);
  const int L = c.n_in + c.n_rec + c.n_out;
  k.full.resize(L);
  for (int l = 0; l < L; ++l) k.full[l] = (uint8_t)r.range(0, 1);
  k.bind();
  return k;
}

int64_t slots_of(const dory_config& c, int layer) {
  return c.layer_is_full[layer] ? c.max_ctx : std::min(c.window, c.max_ctx);
}

// Every element of every cache, through dory_kv_slot's offsets.
void check_kv_layout(const dory_config& c, int mode, int loops) {
  const size_t bytes = dory_kv_bytes(&c, mode, loops);
  CHECK(bytes > 0, "kv_bytes 0 for a valid config");
  if (bytes == 0) return;
  const size_t elem = c.dtype == DORY_F32 ? 4 : 2;
  CHECK(bytes % elem == 0, "kv_bytes %zu not a multiple of the element size", bytes);
  const int64_t n_el = (int64_t)(bytes / elem);
  if (n_el > (int64_t)64 << 20) return;  // keep the bitmap small
  std::vector<uint8_t> owner(n_el, 0);
  const int L = c.n_in + c.n_rec + c.n_out;
  const int hd = c.head_dim;
  const int kl = mode == DORY_KV_PER_LOOP ? loops : 1;
  std::vector<int> seen_ids;
  for (int l = 0; l < L; ++l) {
    const bool rec = l >= c.n_in && l < c.n_in + c.n_rec;
    const int nloops = rec ? kl : 1;
    for (int j = 1; j <= nloops; ++j) {
      const int64_t S = slots_of(c, l), VS = (S + 31) / 32 * 32;
      int64_t kbase = -1, vbase = -1;
      int id0 = -1;
      for (int pos = 0; pos < c.max_ctx; ++pos) {
        int32_t id = -1, slot = -1;
        int64_t ko = -1, vo = -1;
        const dory_status s = dory_kv_slot(&c, mode, loops, l, j, pos, &id, &slot, &ko, &vo);
        CHECK(s == DORY_OK, "kv_slot layer %d loop %d pos %d: status %d", l, j, pos, (int)s);
        if (s != DORY_OK) return;
        const int want = c.layer_is_full[l] ? pos : pos % c.window;
        CHECK(slot == want, "layer %d pos %d: slot %d, expected %d", l, pos, slot, want);
        CHECK(slot >= 0 && slot < S, "slot %d outside [0, %lld)", slot, (long long)S);
        const int64_t kb = ko - (int64_t)slot * hd;
        const int64_t vb = vo - ((int64_t)(slot / 32) * 32 * hd + slot % 32);
        if (pos == 0) {
          kbase = kb; vbase = vb; id0 = id;
        } else {
          CHECK(id == id0 && kb == kbase && vb == vbase, "layer %d pos %d: cache bases move", l, pos);
        }
      }
      CHECK(vbase == kbase + (int64_t)c.max_batch * c.n_kv_heads * S * hd, "values do not follow keys");
      seen_ids.push_back(id0);
      // keys [B][n_kv][S][hd], values [B][n_kv][VS/32][hd][32]
      const int64_t klen = (int64_t)c.max_batch * c.n_kv_heads * S * hd;
      const int64_t vlen = (int64_t)c.max_batch * c.n_kv_heads * VS * hd;
      CHECK(kbase >= 0 && vbase + vlen <= n_el, "cache %d [%lld, %lld) outside %lld elements", id0,
            (long long)kbase, (long long)(vbase + vlen), (long long)n_el);
      if (kbase < 0 || vbase + vlen > n_el) return;
      for (int64_t e = kbase; e < kbase + klen + vlen; ++e) {
        CHECK(owner[e] == 0, "element %lld of cache %d already owned", (long long)e, id0);
        owner[e] = 1;
      }
    }
  }
  for (size_t i = 0; i < seen_ids.size(); ++i)
    CHECK(seen_ids[i] == (int)i, "cache ids not numbered layer by layer: %d at %zu", seen_ids[i], i);
  // out-of-range queries
  int32_t id, slot;
  int64_t ko, vo;
  CHECK(dory_kv_slot(&c, mode, loops, -1, 1, 0, &id, &slot, &ko, &vo) != DORY_OK, "layer -1 accepted");
  CHECK(dory_kv_slot(&c, mode, loops, L, 1, 0, &id, &slot, &ko, &vo) != DORY_OK, "layer L accepted");
  CHECK(dory_kv_slot(&c, mode, loops, 0, 1, -1, &id, &slot, &ko, &vo) != DORY_OK, "pos -1 accepted");
  CHECK(dory_kv_slot(&c, mode, loops, 0, 1, c.max_ctx, &id, &slot, &ko, &vo) != DORY_OK, "pos max_ctx accepted");
  if (c.n_rec > 0 && mode == DORY_KV_PER_LOOP) {
    CHECK(dory_kv_slot(&c, mode, loops, c.n_in, 0, 0, &id, &slot, &ko, &vo) != DORY_OK, "loop 0 accepted");
    CHECK(dory_kv_slot(&c, mode, loops, c.n_in, loops + 1, 0, &id, &slot, &ko, &vo) != DORY_OK,
          "loop past kv_loops accepted");
  }
}

void check_sizes(const dory_config& c) {
  const size_t ws = dory_workspace_bytes(&c);
  CHECK(ws > 0, "workspace 0 for a valid config");
  for (int b = 1; b <= c.max_batch; ++b)
    for (int n : {1, 7, c.max_ctx}) {
      const size_t full = dory_backward_workspace_bytes(&c, b, n);
      const size_t mn = dory_backward_workspace_min_bytes(&c, b, n);
      if (c.n_rec >= 1) CHECK(full >= mn && mn > 0, "backward workspace %zu / %zu", full, mn);
    }
}

// One field at a time pushed to an extreme value.
void check_extremes() {
  const int32_t vals[] = {0, -1, -7, 1, 3, 65, 4097, 1 << 20, 1 << 28, std::numeric_limits<int32_t>::max(),
                          std::numeric_limits<int32_t>::min()};
  int32_t dory_config::*fields[] = {&dory_config::d_model, &dory_config::n_q_heads, &dory_config::n_kv_heads,
                                    &dory_config::head_dim, &dory_config::d_ff, &dory_config::vocab,
                                    &dory_config::n_in, &dory_config::n_rec, &dory_config::n_out,
                                    &dory_config::window, &dory_config::dtype, &dory_config::attn_gate,
                                    &dory_config::max_batch, &dory_config::max_ctx, &dory_config::max_chunk,
                                    &dory_config::max_loops, &dory_config::weight_format};
  long accepted = 0;
  for (auto f : fields)
    for (int32_t v : vals) {
      Cfg k = tiny_cfg();
      k.full.assign(3 * 4096, 1);  // entries for any layer count the limits accept
      k.bind();
      k.c.*f = v;
      const dory_config& c = k.c;
      const bool ok = dory_validate_config(&c) == DORY_OK;
      for (int mode : {DORY_KV_PER_LOOP, DORY_KV_LAST_LOOP}) {
        const size_t kb = dory_kv_bytes(&c, mode, 2);
        CHECK(ok == (kb > 0) || (mode == DORY_KV_PER_LOOP && c.max_loops < 2),
              "kv_bytes %zu disagrees with validation %d", kb, (int)ok);
        int32_t id, slot;
        int64_t ko, vo;
        (void)dory_kv_slot(&c, mode, 1, 0, 1, 0, &id, &slot, &ko, &vo);
      }
      const size_t ws = dory_workspace_bytes(&c);
      CHECK(ok == (ws > 0), "workspace %zu disagrees with validation %d", ws, (int)ok);
      (void)dory_backward_workspace_bytes(&c, 1, 1);
      (void)dory_backward_workspace_min_bytes(&c, 1, 1);
      accepted += ok;
    }
  // non-finite scales and bases
  const double dbad[] = {0.0, 1.0, -1.0, NAN, INFINITY};
  for (double v : dbad) {
    Cfg k = tiny_cfg();
    k.c.rope_base_swa = v;
    CHECK(dory_validate_config(&k.c) != DORY_OK, "RoPE base %g accepted", v);
  }
  const float fbad[] = {NAN, INFINITY, -INFINITY};
  for (float v : fbad) {
    Cfg k = tiny_cfg();
    k.c.combine_wh = v;
    CHECK(dory_validate_config(&k.c) != DORY_OK, "combine weight %g accepted", (double)v);
    Cfg k2 = tiny_cfg();
    k2.c.attn_scale = v;
    CHECK(dory_validate_config(&k2.c) != DORY_OK, "attn_scale %g accepted", (double)v);
    Cfg k3 = tiny_cfg();
    k3.c.logit_scale = v;
    CHECK(dory_validate_config(&k3.c) != DORY_OK, "logit_scale %g accepted", (double)v);
  }
  CHECK(dory_validate_config(nullptr) != DORY_OK, "NULL config accepted");
  CHECK(dory_kv_bytes(nullptr, DORY_KV_LAST_LOOP, 1) == 0, "kv_bytes of NULL");
  CHECK(dory_workspace_bytes(nullptr) == 0, "workspace of NULL");
  std::printf("extremes: %ld accepted\n", accepted);
}

// Context calls over host buffers: only their argument errors run (none of
// them reaches a HIP call), so the buffers are never dereferenced.
void check_context_errors() {
  Cfg k = tiny_cfg();
  const dory_config& c = k.c;
  const int L = c.n_in + c.n_rec + c.n_out;
  const size_t kvb = dory_kv_bytes(&c, DORY_KV_LAST_LOOP, 1), wsb = dory_workspace_bytes(&c);
  void* kv = std::aligned_alloc(256, (kvb + 255) / 256 * 256);
  void* ws = std::aligned_alloc(256, (wsb + 255) / 256 * 256);
  alignas(256) static unsigned char dummy[256];
  std::vector<const void*> P(L, dummy);
  std::vector<const float*> A(L, (const float*)dummy);
  dory_weights w{};
  w.embed = dummy; w.qkvg = P.data(); w.o = P.data(); w.ug = P.data(); w.down = P.data();
  w.alpha_attn = A.data(); w.alpha_mlp = A.data();
  dory_ctx* ctx = nullptr;
  CHECK(dory_create(&c, &w, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, nullptr) == DORY_E_ARG, "NULL out");
  CHECK(dory_create(nullptr, &w, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) != DORY_OK && !ctx,
        "NULL cfg");
  CHECK(dory_create(&c, nullptr, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_E_ARG && !ctx,
        "NULL weights");
  CHECK(dory_create(&c, &w, kv, kvb - 1, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_E_ARG, "small KV");
  CHECK(dory_create(&c, &w, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb - 1, nullptr, &ctx) == DORY_E_ARG, "small ws");
  CHECK(dory_create(&c, &w, (char*)kv + 16, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_E_ARG,
        "misaligned KV");
  CHECK(dory_create(&c, &w, kv, kvb, 7, 1, ws, wsb, nullptr, &ctx) == DORY_E_KV_MODE, "bad kv mode");
  {
    std::vector<const void*> Q = P;
    Q[L - 1] = nullptr;
    dory_weights w2 = w;
    w2.down = Q.data();
    CHECK(dory_create(&c, &w2, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_E_ARG,
          "NULL layer weight");
  }
  {
    dory_weights w3 = w;
    w3.qkvg_scale = P.data();  // scales with dtype weights are ignored, not an error
    CHECK(dory_create(&c, &w3, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_OK,
          "create with unused scales");
    dory_destroy(ctx);
    ctx = nullptr;
  }
  CHECK(dory_create(&c, &w, kv, kvb, DORY_KV_LAST_LOOP, 1, ws, wsb, nullptr, &ctx) == DORY_OK && ctx, "create");
  if (!ctx) return;
  const int32_t* tok = (const int32_t*)dummy;
  int32_t* out = (int32_t*)dummy;
  CHECK(dory_prefill(ctx, nullptr, 1, 4, 2, DORY_KV_LAST_LOOP) == DORY_E_ARG, "NULL tokens");
  CHECK(dory_prefill(ctx, tok, 1, -1, 2, DORY_KV_LAST_LOOP) == DORY_E_ARG, "n < 0");
  CHECK(dory_prefill(ctx, tok, 1, 0, 2, DORY_KV_LAST_LOOP) == DORY_OK, "n == 0 is a no-op");
  CHECK(dory_prefill(ctx, tok, 0, 4, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "batch 0");
  CHECK(dory_prefill(ctx, tok, c.max_batch + 1, 4, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "batch > max");
  CHECK(dory_prefill(ctx, tok, 1, 4, 0, DORY_KV_LAST_LOOP) == DORY_E_LOOPS, "0 loops");
  CHECK(dory_prefill(ctx, tok, 1, 4, c.max_loops + 1, DORY_KV_LAST_LOOP) == DORY_E_LOOPS, "loops > max");
  CHECK(dory_prefill(ctx, tok, 1, 4, 2, DORY_KV_PER_LOOP) == DORY_E_KV_MODE, "kv mode of another layout");
  CHECK(dory_prefill(ctx, tok, 1, c.max_ctx + 1, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "context overflow");
  CHECK(dory_prefill(ctx, tok, 1, std::numeric_limits<int32_t>::max(), 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY,
        "n = INT32_MAX");
  CHECK(std::strlen(dory_last_error(ctx)) > 0, "no error text");
  CHECK(dory_decode_step(ctx, tok, 2, DORY_KV_LAST_LOOP, out) == DORY_E_STATE, "decode before prefill");
  CHECK(dory_decode_step(nullptr, tok, 2, DORY_KV_LAST_LOOP, out) == DORY_E_ARG, "NULL context");
  CHECK(dory_logits(ctx, (float*)dummy) == DORY_E_STATE, "logits before prefill");
  CHECK(dory_logits(ctx, nullptr) == DORY_E_ARG, "NULL logits buffer");
  CHECK(dory_resume(ctx, 0, 5, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "resume batch 0");
  CHECK(dory_resume(ctx, 1, 0, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "resume pos 0");
  CHECK(dory_resume(ctx, 1, c.max_ctx, 2, DORY_KV_LAST_LOOP) == DORY_E_CAPACITY, "resume pos max_ctx");
  CHECK(dory_resume(ctx, 1, 5, 2, DORY_KV_PER_LOOP) == DORY_E_KV_MODE, "resume kv mode");
  CHECK(dory_resume(ctx, 1, 5, 0, DORY_KV_LAST_LOOP) == DORY_E_LOOPS, "resume 0 loops");
  const int32_t loops_bad[2] = {1, c.max_loops + 1}, loops_ok[2] = {1, 2};
  CHECK(dory_prefill_mixed(ctx, tok, 2, 4, nullptr, DORY_KV_LAST_LOOP) == DORY_E_ARG, "mixed NULL loops");
  CHECK(dory_prefill_mixed(ctx, tok, 2, 4, loops_bad, DORY_KV_LAST_LOOP) == DORY_E_LOOPS, "mixed loop count");
  CHECK(dory_prefill_mixed(ctx, tok, 2, 4, loops_ok, DORY_KV_PER_LOOP) == DORY_E_KV_MODE, "mixed per-loop");
  CHECK(dory_decode_step_mixed(ctx, tok, loops_ok, DORY_KV_LAST_LOOP, out) == DORY_E_STATE,
        "mixed decode before prefill");
  {
    const dory_status m = dory_set_markers(ctx, 1);  // the marker library may be absent: then an argument error
    CHECK(m == DORY_OK || m == DORY_E_ARG, "set_markers status %d", (int)m);
    CHECK(dory_set_markers(ctx, 0) == DORY_OK, "markers off");
    CHECK(dory_set_markers(nullptr, 1) == DORY_E_ARG, "markers on a NULL context");
  }
  CHECK(dory_set_trace(ctx, (float*)dummy, 0) == DORY_E_ARG, "trace of 0 entries");
  CHECK(dory_set_trace(ctx, nullptr, 0) == DORY_OK, "trace off");
  CHECK(dory_reset(ctx) == DORY_OK && std::strlen(dory_last_error(ctx)) == 0, "reset clears the error");
  CHECK(dory_reset(nullptr) == DORY_E_ARG, "reset NULL");
  {
    std::vector<float*> G(c.n_rec, (float*)dummy);
    dory_grads g{};
    g.qkvg = G.data(); g.o = G.data(); g.ug = G.data(); g.down = G.data();
    g.alpha_attn = G.data(); g.alpha_mlp = G.data();
    const float* x = (const float*)dummy;
    const size_t bwb = dory_backward_workspace_bytes(&c, 1, 8);
    CHECK(dory_backward_last_loop(ctx, nullptr, x, 1, 8, &g, (float*)dummy, ws, bwb) == DORY_E_ARG, "bw NULL x");
    CHECK(dory_backward_last_loop(ctx, x, x, 1, c.max_ctx + 1, &g, (float*)dummy, ws, bwb) == DORY_E_ARG,
          "bw n > max_ctx");
    CHECK(dory_backward_last_loop(ctx, x, x, 0, 8, &g, (float*)dummy, ws, bwb) == DORY_E_ARG, "bw batch 0");
    CHECK(dory_backward_last_loop(ctx, x, x, 1, 8, &g, (float*)dummy, ws, 0) == DORY_E_ARG, "bw no workspace");
    CHECK(dory_backward_last_loop(ctx, x, x, 1, 8, &g, (float*)dummy, (char*)ws + 8, bwb) == DORY_E_ARG,
          "bw misaligned workspace");
    G[0] = nullptr;
    CHECK(dory_backward_last_loop(ctx, x, x, 1, 8, &g, (float*)dummy, ws, bwb) == DORY_E_ARG, "bw NULL grad");
  }
  dory_destroy(ctx);
  dory_destroy(nullptr);
  for (int s = -12; s < 4; ++s) CHECK(dory_status_string((dory_status)s) != nullptr, "status string %d", s);
  CHECK(std::strlen(dory_last_error(nullptr)) > 0, "last error of NULL");
  std::free(kv);
  std::free(ws);
}

}  // namespace

int main(int argc, char** argv) {
  const int n_random = argc > 1 ? std::atoi(argv[1]) : 300;
  Rng r(20261203);
  int valid = 0;
  for (int i = 0; i < n_random; ++i) {
    Cfg k = random_cfg(r);
    const dory_config& c = k.c;
    if (dory_validate_config(&c) != DORY_OK) continue;
    ++valid;
    check_sizes(c);
    check_kv_layout(c, DORY_KV_LAST_LOOP, 1);
    check_kv_layout(c, DORY_KV_PER_LOOP, c.max_loops);
    if (c.max_loops > 1) check_kv_layout(c, DORY_KV_PER_LOOP, 1);
  }
  check_extremes();
  check_context_errors();
  std::printf("random configs: %d valid of %d; %ld checks, %d failed\n", valid, n_random, g_checks, g_fail);
  return g_fail ? 1 : 0;
}
