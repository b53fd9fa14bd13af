// Host-only model plan: config validation, KV-buffer layout and workspace
// layout. No HIP calls here, so this part is testable on a machine without a
// GPU through the host-only entry points of dory.h.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "dory.h"

namespace dory {

constexpr int kMaxHeadDim = 128;
constexpr int kMaxSplits = 64;        // split-K pieces per (row, kv head) in decode attention
constexpr int kArgmaxBlock = 1024;    // logits per argmax partial
constexpr size_t kAlign = 256;
// Shape and capacity limits of a config: every size the plan derives stays
// far inside 64-bit arithmetic (and every per-row count inside int32).
constexpr int kMaxDModel = 1 << 16;
constexpr int kMaxDFF = 1 << 18;
constexpr int kMaxHeads = 1024;
constexpr int kMaxVocab = 1 << 26;
constexpr int kMaxLayers = 4096;       // per block (input, recurrent, output)
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxCtx = 1 << 26;
constexpr int kMaxLoops = 64;
constexpr int64_t kMaxBwRows = 1 << 21;  // batch * positions of one backward call

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
// Row length of a call's transposed values [B][n_kv][hd][vld]: n rounded up
// to 8 positions, so that every row starts 16-byte aligned.
inline int chunk_vld(int n) { return (n + 7) / 8 * 8; }

struct WsLayout {
  size_t rope_swa = 0, rope_full = 0;  // float2 [max_ctx][hd/2]
  size_t h = 0, e = 0, xb = 0;         // [rows, d]   f32, f32, dtype
  size_t hb = 0;                       // [max_batch, d] f32: second residual buffer (decode ping-pong)
  size_t qkvg = 0;                     // [rows, qkvg_dim] f32
  size_t q = 0, kw = 0;                // [rows, n_q|n_kv, hd] dtype
  size_t vw = 0;                       // [B, n_kv, hd, chunk_vld(n)] dtype (values transposed)
  size_t part = 0;                     // attention partials f32
  size_t ob = 0;                       // [rows, q_dim] dtype
  size_t y = 0;                        // [rows, d] f32
  size_t y1 = 0;                       // [min(rows, 64), d] f32: second half of a split batched-decode product
  size_t a = 0;                        // [rows, d_ff] dtype
  size_t logits = 0;                   // [max_batch, vocab] f32
  size_t next = 0;                     // [max_batch] int32
  size_t amax = 0;                     // argmax partials
  size_t flags = 0;                    // device error flags
  size_t pos = 0;                      // int: position counter read by decode kernels
  size_t rowk = 0;                     // int [max_batch]: per-sequence loop counts of a mixed call
  size_t wdq = 0;                      // bf16: one low-bit projection expanded for a prefill GEMM
  size_t attn_acc = 0;                 // uint64 [min(max_batch, 8)][n_q][hd + 8]: decode attention sums
  size_t total = 0;
};

struct Plan {
  dory_config cfg{};
  std::vector<uint8_t> is_full;
  int n_layers = 0, q_dim = 0, kv_dim = 0, gate_dim = 0, qkvg_dim = 0, elem = 0;
  int max_rows = 0;
  float attn_scale = 0.f, logit_scale = 0.f;
  WsLayout ws;
  bool recurrent(int l) const { return l >= cfg.n_in && l < cfg.n_in + cfg.n_rec; }
  int slots(int l) const;
  int vslots(int l) const { return (slots(l) + 31) / 32 * 32; }  // value cache: 32-position blocks
};

// Fills `plan` from `cfg`; returns DORY_OK or DORY_E_ARG with `why` set.
dory_status make_plan(const dory_config* cfg, Plan* plan, std::string* why);

struct KvLayout {
  int kv_mode = DORY_KV_LAST_LOOP, kv_loops = 1;
  std::vector<int> first_id;           // per layer: first cache id
  std::vector<int> n_ids;              // per layer: caches owned
  std::vector<int64_t> offset;         // per cache id: element offset of K (V follows)
  std::vector<int> id_layer;           // per cache id: its layer
  size_t bytes = 0;
};

dory_status make_kv_layout(const Plan& p, int kv_mode, int kv_loops, KvLayout* kv, std::string* why);

WsLayout make_ws_layout(const Plan& p);

// Workspace of the depth-1 backward for B sequences of n positions (M = B*n
// rows): byte offsets. float32 unless marked; "T" arrays are GEMM operand
// copies in the model dtype.
struct BwLayout {
  size_t hin = 0;                                   // [n_rec + 1][M][d]: layer inputs, then the block output
  size_t P1 = 0, qn = 0, kn = 0, rq = 0, rk = 0;    // fused projection; rotated normalised q / k and their norms
  size_t o = 0, mst = 0, lst = 0;                   // attention output; softmax max / sum per (row, head)
  size_t oh = 0, rc = 0;                            // gated normalised attention output, |c|
  size_t y = 0, yh = 0, ry = 0, rz = 0, h1 = 0;     // output projection / update of the attention sublayer
  size_t P2 = 0, a32 = 0, rs = 0;                   // up/gate projection, activation, |s|
  size_t y2h = 0, ry2 = 0, rz2 = 0;                 // update of the MLP sublayer
  size_t dres = 0, contrib = 0, tmp = 0, dh = 0, dh2 = 0;
  size_t part = 0;  // second partial sum of a GEMM whose contraction is split in two ([M][max(d, qd)])
  size_t dO = 0, D = 0, dqn = 0, dkn = 0, dv = 0, dP1 = 0;
  size_t xb = 0, ohb = 0, h1b = 0, ab = 0, dyb = 0, dP2b = 0, dP1b = 0;  // T
  size_t TA = 0, TB = 0, WT = 0;                    // T: transposed operands of the gradient GEMMs
  // matrix-core attention (bfloat16 models): head-major operand copies
  // [B][H][n][hd] and transposed [B][H][hd][nT] (bfloat16), remade per layer
  size_t fQ = 0, fK = 0, fV = 0, fdO = 0, fQT = 0, fKT = 0, fVT = 0, fdOT = 0;
  size_t fdkh = 0, fdvh = 0;  // per-query-head dk, dv (float32 [M][qd])
  int nT = 0;
  // The values a layer's backward reads from its forward (P1 .. rz2 above
  // but y, and the T copies xb .. ab) sit in one group at the end
  // of the layout, layer_bytes long; with every layer's group kept
  // (stored = true: n_rec groups) the backward reads them instead of running
  // each layer's forward again.
  size_t layer_bytes = 0;
  bool stored = false;
  size_t total = 0;
};

// stored: one group of forward values per recurrent layer (else one, refilled
// by recomputing each layer's forward during the backward)
BwLayout make_bw_layout(const Plan& p, int B, int n, bool stored);
// the layout with the forward-value group of recurrent layer i (stored layouts)
BwLayout bw_layer_view(const BwLayout& L, int i);

size_t argmax_partials(int32_t B, int32_t V);

}  // namespace dory
