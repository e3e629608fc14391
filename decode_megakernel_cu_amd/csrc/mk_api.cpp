// mk_api.cpp -- host side of the C ABI in include/mk.h: validation, arena and workspace layouts,
// weight loading (with the one repack the kernel wants), the single launch per decode step, and
// device status polling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "mk_internal.h"

namespace mk {
size_t kernel_lds_bytes();
bool device_trace_built();
hipError_t launch_decode(const Params& p, int nblocks, bool matrix_cores, hipStream_t stream);
hipError_t launch_transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl, hipStream_t stream);
hipError_t launch_fold_router(const uint16_t* router, const uint16_t* gain, const uint16_t* wo, float* out, int E, int H,
                              int K, hipStream_t stream);
hipError_t occupancy(int* blocks_per_cu);
int max_grid();
hipError_t static_scratch(int device, void** out);
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream);
}  // namespace mk

using namespace mk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr uint64_t kAlign = 256;
constexpr int kMfmaMinRows = MK_MFMA_MIN_ROWS;  // steps of 3..16 token rows on the matrix cores
constexpr int kThreadsHost = kThreads;
uint64_t align_up(uint64_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Slot {
  uint64_t off = 0, bytes = 0;
  int repack = 0;  // 1: W_uk transposed per head
};

using Key = std::tuple<int, int, int>;  // kind, layer (or slot), expert

int layer_kind(const mk_config& c, int l) {
  if (c.attn_kind == MK_ATTN_GQA) return kGqa;
  if (c.attn_kind == MK_ATTN_MLA) return kMla;
  return (l % c.hybrid_period == c.hybrid_period - 1) ? kMla : kKda;
}

struct Layout {
  std::map<Key, Slot> tensors;
  std::vector<LayerDev> layers;  // offsets (as pointers relative to 0) until rebased
  uint64_t arena = 0;
  uint64_t derived = 0;  // bytes of the arena holding tensors derived at load time (rwx)
  WsLayout ws{};
  uint64_t kv = 0, state = 0;
  int n_mla = 0, n_kda = 0, n_gqa = 0;
  int nsplit_max = 0;
};

// Split-KV chunks per (sequence, kv head) that a step can have: a chunk holds at least kChunk
// positions and at least the step's cache rows divided by the grid, so there is at most one
// chunk per workgroup of the grid whatever the sequence length. The merge's LDS batches and the
// workspace's partial results are sized for this many.
int max_splits(int kv_capacity) { return std::min((kv_capacity + kChunk - 1) / kChunk, max_grid()); }

int check_config(const mk_config* c) {
  if (!c) return fail(MK_E_INVAL, "config is NULL");
  if (c->preset < 0 || c->preset > 6) return fail(MK_E_INVAL, "preset %d is not 0 (custom) or a preset id 1..6", c->preset);
  if (c->n_layers < 1 || c->hidden < 8 || c->vocab < 1) return fail(MK_E_INVAL, "n_layers, hidden and vocab must be positive");
  if (c->hidden % 8) return fail(MK_E_UNSUPPORTED, "hidden must be a multiple of 8");
  if (c->attn_kind < 0 || c->attn_kind > 2) return fail(MK_E_INVAL, "attn_kind %d unknown", c->attn_kind);
  if (c->max_batch < 1 || c->max_batch > MK_MAX_BATCH) return fail(MK_E_INVAL, "max_batch must be in 1..%d", MK_MAX_BATCH);
  if (c->max_new_tokens < 1 || c->max_new_tokens > MK_MAX_NEW_TOKENS)
    return fail(MK_E_INVAL, "max_new_tokens must be in 1..%d", MK_MAX_NEW_TOKENS);
  if (c->kv_capacity < c->max_new_tokens) return fail(MK_E_INVAL, "kv_capacity below max_new_tokens");
  if (c->n_experts == 0) {  // dense: the feed-forward block is the shared SwiGLU block alone
    if (c->top_k != 0 || c->shared_ffn < 8 || c->shared_ffn % 8)
      return fail(MK_E_INVAL, "a dense model (n_experts 0) needs top_k 0 and shared_ffn a positive multiple of 8");
  } else {
    if (c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 8)
      return fail(MK_E_INVAL, "need 1 <= top_k <= min(n_experts, 8)");
    if (c->n_experts > kMaxExperts) return fail(MK_E_UNSUPPORTED, "at most %d experts", kMaxExperts);
    if (c->ffn < 8 || c->ffn % 8 || c->shared_ffn < 0 || c->shared_ffn % 8)
      return fail(MK_E_UNSUPPORTED, "ffn and shared_ffn must be multiples of 8");
  }
  if (c->expert_pool_layers < 0) return fail(MK_E_INVAL, "expert_pool_layers must be >= 0");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(MK_E_INVAL, "rms_eps / rope_theta out of range");
  if (c->n_heads < 1) return fail(MK_E_INVAL, "n_heads must be positive");
  if (c->attn_kind == MK_ATTN_GQA) {
    if (c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads) return fail(MK_E_INVAL, "n_heads must be a multiple of n_kv_heads");
    if (c->head_dim < 32 || c->head_dim % 32 || c->head_dim > 128)
      return fail(MK_E_UNSUPPORTED, "head_dim must be 32, 64, 96 or 128 (matrix-core attention)");
    // the attention tile: bf16 keys (rows padded by 8) and values (by 16) of kGSub positions, then
    // per query row (new token x head of the group, in tiles of 16) the query's bf16 high and low
    // parts (padded by 8), the rotated query, the scores (padded by 4) and three statistics; the
    // value sums of row tiles x 16-column tiles stay in registers, at most kGqaTiles per wave
    const int nr = c->max_new_tokens * (c->n_heads / c->n_kv_heads), nrp = (nr + 15) / 16 * 16;
    const int d = c->head_dim;
    if (kGSub * (2 * d + 24) / 2 + nrp * (d + 8) + nrp * d + nrp * (kGSub + 4) + 3 * nrp > kLdsFloats ||
        (nrp / 16) * (d / 16) > kWaves * kGqaTiles)
      return fail(MK_E_UNSUPPORTED, "GQA group too large for the attention tile");
  } else {
    if (c->kv_lora < 8 || c->kv_lora % 8 || c->q_lora < 8 || c->q_lora % 8 || c->nope_dim < 8 || c->nope_dim % 8 ||
        c->v_dim < 8 || c->v_dim % 8 || c->rope_dim < 2 || c->rope_dim % 2 || c->rope_dim > 2 * kMaxRopePairs)
      return fail(MK_E_UNSUPPORTED, "MLA dims must be multiples of 8 (rope_dim even, <= %d)", 2 * kMaxRopePairs);
    const int lat = c->kv_lora + c->rope_dim, nh = c->n_heads;
    // the attention tile: up to 16 heads (an even number; padded to 16, the rows of one matrix-core
    // tile) x kv_lora = 512 on the matrix cores (4 K groups x 2 position tiles, 32 value column tiles
    // over 8 waves)
    if (nh > 16 || nh % 2 || c->kv_lora != 512 || lat % 32 || c->rope_dim % 8)
      return fail(MK_E_UNSUPPORTED, "MLA attention supports an even number of heads up to 16, kv_lora 512 and "
                  "kv_lora + rope_dim a multiple of 32");
    if (kSub * (lat + 8) / 2 + 16 * lat + c->max_new_tokens * lat + 5 * 16 * kSub + 16 * 4 + 8 + c->kv_lora / 2 > kLdsFloats)
      return fail(MK_E_UNSUPPORTED, "MLA heads / latent too wide for the attention tile");
    if (c->attn_kind == MK_ATTN_HYBRID) {
      if (c->hybrid_period < 1) return fail(MK_E_INVAL, "hybrid_period must be positive");
      if (c->kda_dk % 64 || c->kda_dk < 64 || c->kda_dk > 128 || c->kda_dv < 8 || c->kda_dv % 8)
        return fail(MK_E_UNSUPPORTED, "kda_dk must be 64 or 128 and kda_dv a multiple of 8");
    }
  }
  // cache rows are addressed through 32-bit buffer ranges of one (layer, sequence) each
  if (c->kv_capacity > MK_MAX_KV_CAPACITY)
    return fail(MK_E_UNSUPPORTED, "kv_capacity %d above %d", c->kv_capacity, MK_MAX_KV_CAPACITY);
  // the split-KV merge holds in LDS, for one task, the statistics of every split of two (m, head)
  // units (4 floats each) and 32 values per split
  if (40LL * max_splits(c->kv_capacity) > kLdsFloats)
    return fail(MK_E_UNSUPPORTED, "kv_capacity %d too large for the split-KV merge", c->kv_capacity);
  return MK_OK;
}

int instance_rows(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// Whether every GEMV phase of a step with M token rows fits the LDS carve-up of the kernel (mf: the
// matrix-core executor): per workgroup share of nloc tasks, the task accumulators (3 x MM floats
// per task) and one partial slot per accumulator tile plus one per wave (MM floats; on the matrix
// cores the S blocks of R x R floats of a 16x16 tile whose row and column segments match, the
// tiles being groups of R = 16 / S tasks, S the instance's column segments) at the end of the buffer; before them the staged input, at least one slab (8 columns;
// 32 S on the matrix cores, rows padded by 4 floats) of each staged row, or the whole window of
// per-head phases.
bool step_fits(const mk_config& c, int M, int nb, bool mf) {
  if (nb < 1) return true;
  const long long MM = instance_rows(M), S = mfma_segments((int)MM), R = 16 / S;
  const long long pslot = mf ? 256 / S : MM, pad = mf ? 4 : 0, minw = mf ? 32 * S : 8;
  auto cap_of = [&](long long nloc, long long nat) {
    return (long long)kLdsFloats - nloc * 3 * MM - (nat + kWaves) * pslot - 8;
  };
  auto groups = [&](long long nloc) { return mf ? (nloc + R - 1) / R : nloc; };
  // pairs: weight-row kinds per task; down: the down projection (one accumulator tile per group)
  auto ok = [&](long long ntasks, long long rows, long long pairs, bool norm, bool down = false) {
    const long long nloc = (ntasks + nb - 1) / nb, ng = groups(nloc);
    return cap_of(nloc, down ? ng : ng * pairs) >= rows * (minw + pad) + (norm ? minw / 2 : 0);
  };
  auto ok_off = [&](long long ntasks, long long rph, long long seg) {
    const long long nloc = mf ? R * ((ntasks / R + nb - 1) / nb) : (ntasks + nb - 1) / nb;
    const long long window = ((nloc + rph - 1) / rph + 1) * seg;
    return cap_of(nloc, groups(nloc)) >= M * (window + pad);
  };
  const long long E = c.n_experts, F = c.ffn, SF = c.shared_ffn, H = c.hidden, nh = c.n_heads;
  const long long np = (long long)M * c.top_k;
  bool good = ok(c.vocab, M, 1, true) && ok(E + SF, M, SF > 0 ? 2 : 1, true) &&
              ok(std::min(E, np) * F, M, 2, true) && ok(H, np + M, 1, false, true) && ok(H, M, 1, false);
  if (c.attn_kind == MK_ATTN_GQA) {
    good = good && ok(nh * c.head_dim + 2LL * c.n_kv_heads * c.head_dim, M, 1, true);
  } else {
    const long long lat = c.kv_lora + c.rope_dim, qd = c.nope_dim + c.rope_dim;
    good = good && ok(c.q_lora + lat, M, 1, true) && ok(nh * qd, M, 1, true) &&
           ok_off(nh * c.kv_lora, c.kv_lora, c.nope_dim) && ok_off(nh * c.v_dim, c.v_dim, c.kv_lora);
    if (c.attn_kind == MK_ATTN_HYBRID) good = good && ok(2 * nh * c.kda_dk + nh * c.kda_dv, M, 1, true);
  }
  return good;
}

// Whether the matrix-core GEMV executor can run every GEMV phase of this model in the instance for
// M token rows: row lengths in whole units of 32 S columns (S the instance's column segments),
// per-head rows in whole groups of 16 inside one head.
bool mfma_shapes(const mk_config& c, int M) {
  const long long H = c.hidden, F = c.ffn, SF = c.shared_ffn, nh = c.n_heads;
  const long long u = 32LL * mfma_segments(instance_rows(M));
  bool ok = H % u == 0 && F % u == 0 && SF % u == 0;
  if (c.attn_kind == MK_ATTN_GQA) {
    ok = ok && (nh * c.head_dim) % u == 0;
  } else {
    ok = ok && c.q_lora % u == 0 && c.nope_dim % u == 0 && c.kv_lora % u == 0 && (nh * c.v_dim) % u == 0 &&
         c.kv_lora % 16 == 0 && c.v_dim % 16 == 0;
    if (c.attn_kind == MK_ATTN_HYBRID) ok = ok && (nh * c.kda_dv) % u == 0;
  }
  return ok;
}

WsLayout ws_layout(const mk_config& c, uint64_t M, uint64_t nsplit, bool trace);

// input width of layer l's attention output projection
uint64_t wo_width(const mk_config& c, int l) {
  const int k = layer_kind(c, l);
  return (uint64_t)c.n_heads * (k == kGqa ? c.head_dim : k == kMla ? c.v_dim : c.kda_dv);
}

// Whether a step of M token rows folds the router onto the attention output projection (see
// Params::rfuse): a MoE model, at most two rows on the vector executor or eight on the matrix
// cores, and the output projection's LDS carve-up fits every layer. Per workgroup: its task accumulators
// (and on the matrix cores the partial-tile slots) at the end; before them the staged input (one
// slab; rows padded by 4 floats on the matrix cores), the layer input's M rows and the router rows
// of its part.
bool router_fusion(const mk_config& c, int M, int nb, bool mf) {
  if (c.n_experts <= 0 || nb < 1 || M > (mf ? 8 : 2)) return false;
  const long long E = c.n_experts, MM = instance_rows(M), H = c.hidden, S = mfma_segments((int)MM), R = 16 / S;
  const long long P = std::max(1LL, std::min(8LL, nb / E)), nr = P > 1 ? 1 : (E + nb - 1) / nb;
  const long long nloc = (H + nb - 1) / nb, ngrp = (nloc + R - 1) / R;
  for (int l = 0; l < c.n_layers; ++l) {
    const long long K = (long long)wo_width(c, l), span = 4 * (((H + K) / 4 + P - 1) / P);
    long long cap = (long long)kLdsFloats - nloc * 3 * MM;
    if (mf) cap -= (ngrp + kWaves) * (256 / S);
    cap &= ~7LL;
    if (M * (K + (mf ? 4 : 0)) + M * span + nr * span > cap) return false;
  }
  return true;
}

Layout make_layout(const mk_config& c) {
  Layout Lt;
  const uint64_t H = c.hidden, V = c.vocab, E = c.n_experts, F = c.ffn, SF = c.shared_ffn;
  uint64_t off = align_up(sizeof(LayerDev) * (uint64_t)c.n_layers);
  // packed: the next tensor follows without padding (the experts of one pool block are indexed as
  // one [E][rows][cols] array)
  auto put = [&](int kind, int layer, int expert, uint64_t bytes, int repack = 0, bool packed = false) {
    Slot s;
    s.off = off;
    s.bytes = bytes;
    s.repack = repack;
    Lt.tensors[Key(kind, layer, expert)] = s;
    off = packed ? off + bytes : align_up(off + bytes);
    return s.off;
  };
  put(MK_W_EMBED, -1, -1, V * H * 2);
  put(MK_W_FINAL_NORM, -1, -1, H * 2);
  put(MK_W_LM_HEAD, -1, -1, V * H * 2);
  Lt.layers.resize(c.n_layers);
  auto rel = [](uint64_t o) { return reinterpret_cast<const uint16_t*>(o); };
  for (int l = 0; l < c.n_layers; ++l) {
    LayerDev& d = Lt.layers[l];
    std::memset(&d, 0, sizeof d);
    d.kind = layer_kind(c, l);
    d.slot = c.expert_pool_layers ? l % c.expert_pool_layers : l;
    d.attn_norm = rel(put(MK_W_ATTN_NORM, l, -1, H * 2));
    if (d.kind == kGqa) {
      d.ord = Lt.n_gqa++;
      const uint64_t dq = (uint64_t)c.n_heads * c.head_dim, dkv = (uint64_t)c.n_kv_heads * c.head_dim;
      d.wq = rel(put(MK_W_WQ, l, -1, dq * H * 2));
      d.wk = rel(put(MK_W_WK, l, -1, dkv * H * 2));
      d.wv = rel(put(MK_W_WV, l, -1, dkv * H * 2));
      d.wo = rel(put(MK_W_WO, l, -1, H * dq * 2));
    } else if (d.kind == kMla) {
      d.ord = Lt.n_mla++;
      const uint64_t nh = c.n_heads, ql = c.q_lora, kvl = c.kv_lora, rd = c.rope_dim, nd = c.nope_dim, vd = c.v_dim;
      d.w_dq = rel(put(MK_W_W_DQ, l, -1, ql * H * 2));
      d.q_norm = rel(put(MK_W_Q_NORM, l, -1, ql * 2));
      d.w_uq = rel(put(MK_W_W_UQ, l, -1, nh * (nd + rd) * ql * 2));
      d.w_dkv = rel(put(MK_W_W_DKV, l, -1, (kvl + rd) * H * 2));
      d.kv_norm = rel(put(MK_W_KV_NORM, l, -1, kvl * 2));
      d.w_ukT = rel(put(MK_W_W_UK, l, -1, nh * nd * kvl * 2, 1));
      d.w_uv = rel(put(MK_W_W_UV, l, -1, nh * vd * kvl * 2));
      d.wo = rel(put(MK_W_WO, l, -1, H * nh * vd * 2));
    } else {
      d.ord = Lt.n_kda++;
      const uint64_t nh = c.n_heads, dk = c.kda_dk, dv = c.kda_dv;
      d.kwq = rel(put(MK_W_KDA_WQ, l, -1, nh * dk * H * 2));
      d.kwk = rel(put(MK_W_KDA_WK, l, -1, nh * dk * H * 2));
      d.kwv = rel(put(MK_W_KDA_WV, l, -1, nh * dv * H * 2));
      d.alpha = reinterpret_cast<const float*>(put(MK_W_KDA_ALPHA, l, -1, nh * dk * 4));
      d.beta = reinterpret_cast<const float*>(put(MK_W_KDA_BETA, l, -1, nh * 4));
      d.wo = rel(put(MK_W_WO, l, -1, H * nh * dv * 2));
    }
    d.moe_norm = rel(put(MK_W_MOE_NORM, l, -1, H * 2));
    if (E) {
      d.router = rel(put(MK_W_ROUTER, l, -1, E * H * 2));
      // derived, not loaded (no slot of the tensor map): the router folded onto W_o
      const uint64_t rb = E * (H + wo_width(c, l)) * 4;
      d.rwx = reinterpret_cast<const float*>(off);
      off = align_up(off + rb);
      Lt.derived += align_up(rb);
    }
    if (SF) {
      d.sh_gate = rel(put(MK_W_SH_GATE, l, -1, SF * H * 2));
      d.sh_up = rel(put(MK_W_SH_UP, l, -1, SF * H * 2));
      d.sh_down = rel(put(MK_W_SH_DOWN, l, -1, H * SF * 2));
    }
  }
  // expert pool: per slot three contiguous blocks [E][F][H], [E][F][H], [E][H][F]
  const int nslot = c.expert_pool_layers ? c.expert_pool_layers : c.n_layers;
  std::vector<uint64_t> gbase(nslot), ubase(nslot), dbase(nslot);
  for (int s = 0; s < nslot; ++s) {
    gbase[s] = off;
    for (int e = 0; e < c.n_experts; ++e) put(MK_W_EXP_GATE, s, e, F * H * 2, 0, e + 1 < c.n_experts);
    ubase[s] = off;
    for (int e = 0; e < c.n_experts; ++e) put(MK_W_EXP_UP, s, e, F * H * 2, 0, e + 1 < c.n_experts);
    dbase[s] = off;
    for (int e = 0; e < c.n_experts; ++e) put(MK_W_EXP_DOWN, s, e, H * F * 2, 0, e + 1 < c.n_experts);
  }
  for (int l = 0; l < c.n_layers; ++l) {
    LayerDev& d = Lt.layers[l];
    d.exp_gate = rel(gbase[d.slot]);
    d.exp_up = rel(ubase[d.slot]);
    d.exp_down = rel(dbase[d.slot]);
  }
  Lt.arena = off;

  // caches
  const uint64_t Bm = c.max_batch, cap = c.kv_capacity;
  if (c.attn_kind == MK_ATTN_GQA)
    Lt.kv = 2ull * c.n_layers * Bm * c.n_kv_heads * cap * c.head_dim * 2;
  else
    Lt.kv = (uint64_t)Lt.n_mla * Bm * cap * (c.kv_lora + c.rope_dim) * 2;
  Lt.state = (uint64_t)Lt.n_kda * Bm * c.n_heads * c.kda_dk * c.kda_dv * 4;

  // workspace: sized for the largest step of the model
  Lt.nsplit_max = max_splits(c.kv_capacity);
  Lt.ws = ws_layout(c, (uint64_t)std::min(MK_MAX_M, c.max_batch * c.max_new_tokens), Lt.nsplit_max, true);
  return Lt;
}

// The workspace carve-up for steps of at most M token rows and nsplit split-KV partials per
// (row, head); trace: room for the per-barrier wall-clock stamps.
WsLayout ws_layout(const mk_config& c, uint64_t M, uint64_t nsplit, bool trace) {
  const uint64_t H = c.hidden, E = c.n_experts, F = c.ffn, SF = c.shared_ffn;
  const uint64_t nh = c.n_heads;
  uint64_t w1 = 0, w2 = 0, w3 = 0, dmax = 0, w4 = 0, wo2 = 0;
  if (c.attn_kind == MK_ATTN_GQA) {
    w1 = nh * c.head_dim;
    w2 = w3 = (uint64_t)c.n_kv_heads * c.head_dim;
    dmax = c.head_dim;
  } else {
    w1 = std::max<uint64_t>(c.q_lora, nh * c.kda_dk);
    w2 = std::max<uint64_t>(c.kv_lora + c.rope_dim, nh * c.kda_dk);
    w3 = std::max<uint64_t>(nh * (c.nope_dim + c.rope_dim), nh * c.kda_dv);
    w4 = nh * c.kv_lora;
    wo2 = nh * c.v_dim;
    dmax = std::max<uint64_t>(c.kv_lora, c.kda_dv);
  }
  uint64_t part = M * nh * nsplit * (dmax + kPartPad);
  if (c.attn_kind != MK_ATTN_GQA && trace) {
    // the W_uk repack stages a host tensor here (the context's workspace only)
    const uint64_t uk = nh * c.nope_dim * c.kv_lora * 2 / 4 + 64;
    part = std::max(part, uk);
  }
  WsLayout w{};
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.flags = take(kMaxBlocks * 4);
  w.status = take(kStatusWords * 4);
  w.trace_slots = trace ? (uint64_t)(3 + 10 * c.n_layers) * kMaxBlocks : 0;
  w.trace = take(w.trace_slots * kTraceStamps * 8);
  w.rope = take((uint64_t)MK_MAX_NEW_TOKENS * kMaxRopePairs * 2 * 4);
  w.x = take(M * H * 4);
  w.x2 = take(M * H * 4);
  w.ssq = take(M * kMaxBlocks * 4);
  w.a1 = take(M * w1 * 4);
  w.a2 = take(M * w2 * 4);
  w.a3 = take(M * w3 * 4);
  w.a4 = take(M * std::max<uint64_t>(w4, 1) * 4);
  w.att = take(M * nh * dmax * 4);
  w.o2 = take(M * std::max<uint64_t>(wo2, 1) * 4);
  w.part = take(part * 4);
  w.part_floats = part;
  // router logits; with router fusion up to 8 partial logits per (row, expert), E * 8 <= 8 * grid
  w.rlog = take(M * std::max<uint64_t>(E * 8, kMaxBlocks) * 4);
  w.sact = take(M * std::max<uint64_t>(SF, 1) * 4);
  w.eact = take(M * c.top_k * F * 4);
  w.amax = take(M * 8);
  w.scratch = w.part;
  w.total = o;
  return w;
}

}  // namespace

struct mk_ctx {
  mk_config cfg;
  Layout lt;
  int device;
  uint8_t* arena;
  uint8_t* ws;
  int nblocks;
  uint64_t launches;
  uint64_t watchdog_ticks;
  bool poisoned;
  bool trace;
  int mfma_min_rows;  // GEMV phases of steps with at least this many rows on the matrix cores
  int last_barriers;
  const uint8_t* last_status;  // status words of the last step (the workspace's, or the static scratch's)
  std::vector<uint8_t> loaded;  // per tensor slot, in map order
  std::map<Key, size_t> index;
  size_t n_loaded;
};

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

int mk_config_preset(int id, mk_config* out) {
  if (!out) return fail(MK_E_INVAL, "config output is NULL");
  mk_config c;
  std::memset(&c, 0, sizeof c);
  c.max_batch = 8;
  c.max_new_tokens = 8;
  c.rms_eps = 1e-6f;
  c.rope_theta = 1e4f;
  switch (id) {
    case 1:  // tiny MoE decoder
      c.n_layers = 2; c.hidden = 256; c.vocab = 1024; c.attn_kind = MK_ATTN_GQA;
      c.n_heads = 4; c.n_kv_heads = 4; c.head_dim = 64;
      c.n_experts = 8; c.top_k = 2; c.ffn = 512; c.shared_ffn = 0;
      c.kv_capacity = 136;
      break;
    case 2:  // mid-size MoE decoder
      c.n_layers = 8; c.hidden = 2048; c.vocab = 32000; c.attn_kind = MK_ATTN_GQA;
      c.n_heads = 16; c.n_kv_heads = 4; c.head_dim = 128;
      c.n_experts = 64; c.top_k = 8; c.ffn = 768; c.shared_ffn = 768;
      c.max_batch = 4; c.kv_capacity = 2056;
      break;
    case 3:  // K3-scale one-GPU share (and its verify step, preset 4; hybrid variant, preset 5)
    case 4:
    case 5:
      c.n_layers = 92; c.hidden = 7168; c.vocab = 40960; c.attn_kind = id == 5 ? MK_ATTN_HYBRID : MK_ATTN_MLA;
      c.n_heads = 16; c.q_lora = 1536; c.kv_lora = 512; c.rope_dim = 64; c.nope_dim = 128; c.v_dim = 128;
      if (id == 5) {
        c.kda_dk = 128; c.kda_dv = 128; c.hybrid_period = 4;
      }
      c.n_experts = 48; c.top_k = 1; c.ffn = 2048; c.shared_ffn = 512; c.expert_pool_layers = 46;
      c.kv_capacity = 4104;
      break;
    case 6:  // dense second model
      c.n_layers = 64; c.hidden = 5120; c.vocab = 151936; c.attn_kind = MK_ATTN_GQA;
      c.n_heads = 40; c.n_kv_heads = 8; c.head_dim = 128;
      c.n_experts = 0; c.top_k = 0; c.ffn = 0; c.shared_ffn = 21504;
      c.kv_capacity = 4104; c.rope_theta = 1e6f;
      break;
    default:
      return fail(MK_E_INVAL, "unknown preset %d (1..6)", id);
  }
  c.preset = id;
  *out = c;
  g_err.clear();
  return MK_OK;
}

int mk_query_sizes(const mk_config* cfg, mk_sizes* out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(MK_E_INVAL, "sizes output is NULL");
  Layout lt = make_layout(*cfg);
  out->arena_bytes = lt.arena;
  out->workspace_bytes = lt.ws.total;
  out->kv_bytes = lt.kv;
  out->kda_state_bytes = lt.state;
  g_err.clear();
  return MK_OK;
}

int mk_create(const mk_config* cfg, int device, void* d_arena, uint64_t arena_bytes, void* d_workspace,
              uint64_t workspace_bytes, mk_ctx** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(MK_E_INVAL, "context output is NULL");
  *out = nullptr;
  Layout lt = make_layout(*cfg);
  // a device context without a workspace (NULL, 0 bytes) steps only through mk_decode_step_static
  const bool no_ws = device != MK_DEVICE_NONE && !d_workspace && workspace_bytes == 0;
  if (device != MK_DEVICE_NONE) {
    if (!d_arena || (!d_workspace && !no_ws)) return fail(MK_E_INVAL, "arena and workspace must be device pointers");
    if ((reinterpret_cast<uintptr_t>(d_arena) | reinterpret_cast<uintptr_t>(d_workspace)) & (kAlign - 1))
      return fail(MK_E_INVAL, "arena and workspace must be 256-byte aligned");
  }
  if (arena_bytes < lt.arena) return fail(MK_E_NOMEM, "arena has %llu bytes, needs %llu", (unsigned long long)arena_bytes, (unsigned long long)lt.arena);
  if (lt.ws.total >= (1ull << 31)) return fail(MK_E_UNSUPPORTED, "workspace above 2 GiB");
  if (!no_ws && workspace_bytes < lt.ws.total)
    return fail(MK_E_NOMEM, "workspace has %llu bytes, needs %llu", (unsigned long long)workspace_bytes, (unsigned long long)lt.ws.total);
  mk_ctx* c = new mk_ctx();
  c->cfg = *cfg;
  c->lt = lt;
  c->device = device;
  c->arena = static_cast<uint8_t*>(d_arena);
  c->ws = static_cast<uint8_t*>(d_workspace);
  c->launches = 0;
  c->poisoned = false;
  c->trace = false;
  c->mfma_min_rows = cfg->n_experts > 0 ? kMfmaMinRows : MK_MFMA_MIN_ROWS_DENSE;
  c->last_barriers = 0;
  c->last_status = nullptr;
  c->n_loaded = 0;
  size_t i = 0;
  for (auto& kv : c->lt.tensors) c->index[kv.first] = i++;
  c->loaded.assign(i, 0);
  c->nblocks = 0;
  if (device != MK_DEVICE_NONE) {
    hipError_t e = hipSetDevice(device);
    int cus = 0, rate_khz = 0, per_cu = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, device);
    if (e == hipSuccess) e = occupancy(&per_cu);
    if (e != hipSuccess) {
      delete c;
      return fail(MK_E_HIP, "device query failed: %s", hipGetErrorString(e));
    }
    if (per_cu < 1) {
      delete c;
      return fail(MK_E_UNSUPPORTED, "the megakernel does not fit on a CU (LDS %zu bytes)", kernel_lds_bytes());
    }
    c->nblocks = std::min(cus, max_grid());
    double ms = 2000.0;
    if (const char* env = std::getenv("MK_WATCHDOG_MS")) ms = std::max(1.0, std::atof(env));
    c->watchdog_ticks = (uint64_t)(ms * (rate_khz > 0 ? rate_khz : 100000));
    // write the layer table (pointers rebased onto the arena) and clear the workspace
    std::vector<LayerDev> tab = c->lt.layers;
    const uintptr_t base = reinterpret_cast<uintptr_t>(c->arena);
    for (auto& d : tab) {
      const uint16_t** ps[] = {&d.attn_norm, &d.moe_norm, &d.router, &d.sh_gate, &d.sh_up, &d.sh_down, &d.wo,
                               &d.wq, &d.wk, &d.wv, &d.w_dq, &d.q_norm, &d.w_uq, &d.w_dkv, &d.kv_norm, &d.w_ukT,
                               &d.w_uv, &d.kwq, &d.kwk, &d.kwv, &d.exp_gate, &d.exp_up, &d.exp_down};
      for (auto p : ps)
        if (*p) *p = reinterpret_cast<const uint16_t*>(base + reinterpret_cast<uintptr_t>(*p));
      if (d.alpha) d.alpha = reinterpret_cast<const float*>(base + reinterpret_cast<uintptr_t>(d.alpha));
      if (d.rwx) d.rwx = reinterpret_cast<const float*>(base + reinterpret_cast<uintptr_t>(d.rwx));
      if (d.beta) d.beta = reinterpret_cast<const float*>(base + reinterpret_cast<uintptr_t>(d.beta));
    }
    e = hipMemcpy(c->arena, tab.data(), sizeof(LayerDev) * tab.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && c->ws) e = hipMemset(c->ws, 0, c->lt.ws.total);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      delete c;
      return fail(MK_E_HIP, "context set-up failed: %s", hipGetErrorString(e));
    }
  }
  *out = c;
  g_err.clear();
  return MK_OK;
}

int mk_load_weights(mk_ctx* c, const mk_tensor_desc* d, int n, void* stream) {
  if (!c) return fail(MK_E_INVAL, "context is NULL");
  if (n < 0 || (n > 0 && !d)) return fail(MK_E_INVAL, "bad descriptor list");
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) {
    const mk_tensor_desc& t = d[i];
    const bool global = t.kind == MK_W_EMBED || t.kind == MK_W_FINAL_NORM || t.kind == MK_W_LM_HEAD;
    const bool expert = t.kind == MK_W_EXP_GATE || t.kind == MK_W_EXP_UP || t.kind == MK_W_EXP_DOWN;
    Key k(t.kind, global ? -1 : t.layer, expert ? t.expert : -1);
    auto it = c->lt.tensors.find(k);
    if (t.kind < 0 || t.kind >= MK_W_N_KINDS || it == c->lt.tensors.end())
      return fail(MK_E_INVAL, "tensor %d: no tensor of kind %d, layer %d, expert %d in this model", i, t.kind, t.layer, t.expert);
    if (t.bytes != it->second.bytes)
      return fail(MK_E_INVAL, "tensor %d (kind %d layer %d): %llu bytes given, %llu expected", i, t.kind, t.layer,
                  (unsigned long long)t.bytes, (unsigned long long)it->second.bytes);
    if (!t.src) return fail(MK_E_INVAL, "tensor %d: NULL source", i);
    if (c->device != MK_DEVICE_NONE) {
      uint8_t* dst = c->arena + it->second.off;
      hipError_t e;
      if (it->second.repack == 1) {
        const void* src = t.src;
        if (!t.src_on_device && !c->ws)
          return fail(MK_E_INVAL, "tensor %d: a context without a workspace takes W_uk from device memory only", i);
        if (!t.src_on_device) {
          e = hipMemcpyAsync(c->ws + c->lt.ws.scratch, t.src, t.bytes, hipMemcpyHostToDevice, st);
          if (e != hipSuccess) return fail(MK_E_HIP, "copy of tensor %d failed: %s", i, hipGetErrorString(e));
          src = c->ws + c->lt.ws.scratch;
        }
        e = launch_transpose_uk(static_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst), c->cfg.n_heads,
                                c->cfg.nope_dim, c->cfg.kv_lora, st);
      } else {
        e = hipMemcpyAsync(dst, t.src, t.bytes, t.src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, st);
      }
      if (e != hipSuccess) return fail(MK_E_HIP, "load of tensor %d failed: %s", i, hipGetErrorString(e));
    }
    size_t idx = c->index[k];
    if (!c->loaded[idx]) {
      c->loaded[idx] = 1;
      c->n_loaded++;
    }
    // a MoE layer's folded router, once its three factors are in the arena (again whenever one of
    // them is replaced)
    if ((t.kind == MK_W_ROUTER || t.kind == MK_W_MOE_NORM || t.kind == MK_W_WO) && c->cfg.n_experts > 0 &&
        c->device != MK_DEVICE_NONE) {
      const int l = t.layer;
      const Key kr(MK_W_ROUTER, l, -1), kg(MK_W_MOE_NORM, l, -1), ko(MK_W_WO, l, -1);
      if (c->loaded[c->index[kr]] && c->loaded[c->index[kg]] && c->loaded[c->index[ko]]) {
        const LayerDev& d = c->lt.layers[l];
        auto at = [&](const void* rel) { return c->arena + reinterpret_cast<uintptr_t>(rel); };
        const hipError_t e = launch_fold_router(
            reinterpret_cast<const uint16_t*>(at(d.router)), reinterpret_cast<const uint16_t*>(at(d.moe_norm)),
            reinterpret_cast<const uint16_t*>(at(d.wo)), reinterpret_cast<float*>(at(d.rwx)), c->cfg.n_experts,
            c->cfg.hidden, (int)wo_width(c->cfg, l), st);
        if (e != hipSuccess) return fail(MK_E_HIP, "folded router of layer %d failed: %s", l, hipGetErrorString(e));
      }
    }
  }
  g_err.clear();
  return MK_OK;
}

// One decode step (both entry points): validation, parameters, the launch.
// A sampling step: temperature, top_p and the caller's uniform numbers in, tokens out.
struct SampleArgs {
  float temperature, top_p;
  const float* uniform;
  int32_t* sampled;
};

// use_static: the step's workspace is the library's static scratch array on the context's device
// (sized for this step), instead of the context's workspace.
static int decode_step(mk_ctx* c, int B, int T, int kv_len, const int32_t* d_tokens, void* d_kv, float* d_kda_state,
                       float* d_logits, int32_t* d_route, int32_t* d_argmax, int32_t* d_accepted, void* stream,
                       const SampleArgs* smp = nullptr, bool use_static = false) {
  if (!c) return fail(MK_E_INVAL, "context is NULL");
  const bool greedy = d_argmax != nullptr;
  if (smp) {
    if (!(smp->temperature > 0.f) || !std::isfinite(smp->temperature))
      return fail(MK_E_INVAL, "temperature must be positive and finite");
    if (!(smp->top_p > 0.f && smp->top_p <= 1.f)) return fail(MK_E_INVAL, "top_p must be in (0, 1]");
    if (!smp->uniform || !smp->sampled || !d_logits)
      return fail(MK_E_INVAL, "a sampling step needs logits, uniform and sampled buffers");
  }
  const mk_config& g = c->cfg;
  if (B < 1 || B > g.max_batch) return fail(MK_E_INVAL, "batch %d outside 1..%d", B, g.max_batch);
  if (T < 1 || T > g.max_new_tokens) return fail(MK_E_INVAL, "n_new_tokens %d outside 1..%d", T, g.max_new_tokens);
  if (B * T > MK_MAX_M) return fail(MK_E_UNSUPPORTED, "batch * n_new_tokens = %d exceeds %d", B * T, MK_MAX_M);
  if (kv_len < 0) return fail(MK_E_INVAL, "kv_len %d is negative", kv_len);
  if ((long long)kv_len + T > g.kv_capacity)
    return fail(MK_E_KV_OVERFLOW, "kv_len %d + %d new tokens exceeds capacity %d", kv_len, T, g.kv_capacity);
  if (!d_tokens || !d_kv) return fail(MK_E_INVAL, "tokens and kv must be non-NULL");
  if (!greedy && !d_logits) return fail(MK_E_INVAL, "logits must be non-NULL");
  if (g.attn_kind == MK_ATTN_HYBRID && !d_kda_state) return fail(MK_E_INVAL, "hybrid model needs the delta-rule state");
  const int M = B * T;
  const bool mf = M >= c->mfma_min_rows && mfma_shapes(g, M) && step_fits(g, M, c->nblocks, true);
  if (!mf && !step_fits(g, M, c->nblocks, false))
    return fail(MK_E_UNSUPPORTED, "a phase of this step does not fit the workgroup's LDS");
  // split-KV: chunks (at least kChunk positions) sized so that the tasks of the step about fill the grid
  const int npos = kv_len + T;
  // merge and W_uv in one phase: MLA layers with v_dim 128 and kv_lora 512, 1 or 2 rows on the
  // vector executor or 3 to 8 on the matrix cores. A workgroup per (row, head, latent block, block
  // of W_uv rows): 4 latent blocks at 1 row, 2 at 2 rows, 1 at 3-8 rows (64-row blocks in the 8-row
  // instance), at most 256 workgroups at 16 heads, with a counter per (row, head, row block) in the
  // last 128 flag words where a head's latent values are split. With whole heads
  // per workgroup at 1 row, each one's read of the head's split-KV partials (266 KB over 4096
  // positions) cost what the phase saved.
  const bool mfuse = g.attn_kind != MK_ATTN_GQA && (mf ? M >= 3 && M <= 8 : M <= 2) && g.v_dim == 128 &&
                     g.kv_lora == 512 && g.n_heads <= 16 && g.n_heads * (M <= 2 ? 16 : M <= 4 ? 4 * M : 2 * M) <= c->nblocks &&
                     !std::getenv("MK_NO_MERGE_FUSION");
  int chunk = kChunk;
  if (g.attn_kind != MK_ATTN_GQA && c->nblocks > 0) {  // whole kSub-position tiles per task
    const int even = (int)(((long long)B * npos + c->nblocks - 1) / c->nblocks);
    chunk = (std::max(kChunk, even) + kSub - 1) / kSub * kSub;
  } else if (c->nblocks > 0) {  // GQA: tasks (sequence, kv head, split) about fill the grid
    const int even = (int)(((long long)B * g.n_kv_heads * npos + c->nblocks - 1) / c->nblocks);
    chunk = (std::max(kChunk, even) + kChunk - 1) / kChunk * kChunk;
  }
  const int nsplit = (npos + chunk - 1) / chunk;
  WsLayout w = c->lt.ws;
  if (use_static) {
    w = ws_layout(g, (uint64_t)M, (uint64_t)nsplit, false);
    if (w.total > kStaticScratchBytes)
      return fail(MK_E_UNSUPPORTED, "this step needs %llu bytes of workspace; the static scratch holds %llu",
                  (unsigned long long)w.total, (unsigned long long)kStaticScratchBytes);
  }
  if (c->n_loaded != c->loaded.size())
    return fail(MK_E_STATE, "%zu of %zu weight tensors loaded", c->n_loaded, c->loaded.size());
  if (c->poisoned) return fail(MK_E_STATE, "context poisoned by an earlier device error");
  if (c->device == MK_DEVICE_NONE) return fail(MK_E_STATE, "host-only context cannot launch");
  if (!use_static && !c->ws) return fail(MK_E_STATE, "context has no workspace: steps go through mk_decode_step_static");
  uint8_t* ws = c->ws;
  if (use_static) {
    void* base = nullptr;
    hipError_t e = static_scratch(c->device, &base);
    if (e != hipSuccess) return fail(MK_E_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    ws = static_cast<uint8_t*>(base);
  }

  Params p{};
  p.L = g.n_layers; p.H = g.hidden; p.V = g.vocab; p.nh = g.n_heads; p.nkv = g.n_kv_heads; p.hd = g.head_dim;
  p.ql = g.q_lora; p.kvl = g.attn_kind == MK_ATTN_GQA ? 0 : g.kv_lora; p.rd = g.rope_dim; p.nd = g.nope_dim;
  p.vd = g.v_dim; p.dk = g.kda_dk; p.dv = g.kda_dv; p.E = g.n_experts; p.topk = g.top_k; p.F = g.ffn;
  p.SF = g.shared_ffn; p.norm_topk = g.norm_topk; p.cap = g.kv_capacity; p.Bmax = g.max_batch;
  // the MLA family's kernels are built for rope_dim 64; an MLA model with another runs on the
  // hybrid family's kernels (the same MLA code with the rope dimension as a parameter)
  p.family = g.attn_kind == MK_ATTN_MLA && g.rope_dim != 64 ? MK_ATTN_HYBRID : g.attn_kind;
  p.eps = g.rms_eps; p.rope_theta = g.rope_theta;
  p.B = B; p.T = T; p.M = M; p.kv_len = kv_len;
  p.chunk = chunk;
  p.nsplit = nsplit;
  // the context's flags count up across its steps; the static scratch's are cleared before each step
  p.epoch = use_static ? 0u : (uint32_t)(c->launches * 65536ull);
  p.tokens = d_tokens; p.logits = d_logits; p.route = d_route;
  p.layers = reinterpret_cast<const LayerDev*>(c->arena);
  auto wt = [&](int kind) { return reinterpret_cast<const uint16_t*>(c->arena + c->lt.tensors.at(Key(kind, -1, -1)).off); };
  p.embed = wt(MK_W_EMBED); p.final_norm = wt(MK_W_FINAL_NORM); p.lm_head = wt(MK_W_LM_HEAD);
  p.kv = static_cast<uint16_t*>(d_kv);
  p.kda_state = d_kda_state;
  p.flags = reinterpret_cast<uint32_t*>(ws + w.flags);
  p.status = reinterpret_cast<uint32_t*>(ws + w.status);
  auto f = [&](uint64_t o) { return reinterpret_cast<float*>(ws + o); };
  p.rope = f(w.rope); p.x = f(w.x); p.a1 = f(w.a1); p.a2 = f(w.a2); p.a3 = f(w.a3); p.a4 = f(w.a4);
  p.att = f(w.att); p.o2 = f(w.o2); p.part = f(w.part); p.rlog = f(w.rlog); p.sact = f(w.sact); p.eact = f(w.eact);
  p.x2 = f(w.x2); p.ssq = f(w.ssq);
  p.rfuse = router_fusion(g, M, c->nblocks, mf) && !std::getenv("MK_NO_ROUTER_FUSION") ? 1 : 0;
  p.mfuse = mfuse ? 1 : 0;
  p.wsb = reinterpret_cast<const char*>(ws);
  p.ws_bytes = (uint32_t)w.total;
  p.watchdog_ticks = c->watchdog_ticks;
  p.trace = c->trace && !use_static ? reinterpret_cast<uint64_t*>(ws + w.trace) : nullptr;
  p.greedy = greedy ? 1 : 0;
  p.amax = reinterpret_cast<unsigned long long*>(ws + w.amax);
  p.argmax = d_argmax;
  p.accepted = d_accepted;
  if (smp) {
    p.sample = 1;
    p.temperature = smp->temperature;
    p.top_p = smp->top_p;
    p.uniform = smp->uniform;
    p.sampled = smp->sampled;
  }
  const int nh = g.n_heads;
  const uint64_t dmax = g.attn_kind == MK_ATTN_GQA ? g.head_dim : std::max(g.kv_lora, g.kda_dv);
  if ((uint64_t)M * nh * p.nsplit * (dmax + kPartPad) > w.part_floats)
    return fail(MK_E_UNSUPPORTED, "attention partials exceed the workspace");
  if (p.nsplit > c->lt.nsplit_max) return fail(MK_E_UNSUPPORTED, "%d split-KV chunks, at most %d", p.nsplit, c->lt.nsplit_max);
  hipError_t e = hipSetDevice(c->device);
  if (e == hipSuccess && use_static)  // barrier flags and status words start at zero
    e = launch_clear_words(p.flags, (int)((w.status + kStatusWords * 4 - w.flags) / 4),
                           static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = launch_decode(p, c->nblocks, mf, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MK_E_HIP, "launch failed: %s", hipGetErrorString(e));
  if (!use_static) c->launches++;
  c->last_status = ws + w.status;
  int nb = (greedy || smp) ? 2 : 1;  // the LM head's barrier, and the one before greedy or sampled tokens
  for (int l = 0; l < g.n_layers; ++l) {  // attention phases, then 3 MoE phases (router fusion, dense: 2)
    const int k = layer_kind(g, l);
    nb += (k == kGqa ? 4 : k == kMla ? 7 - p.mfuse : 3) + (g.n_experts && !p.rfuse ? 3 : 2);
  }
  c->last_barriers = use_static ? 0 : nb;  // a static step records no trace
  g_err.clear();
  return MK_OK;
}

int mk_decode_step(mk_ctx* c, int B, int T, int kv_len, const int32_t* d_tokens, void* d_kv, float* d_kda_state,
                   float* d_logits, int32_t* d_route, void* stream) {
  return decode_step(c, B, T, kv_len, d_tokens, d_kv, d_kda_state, d_logits, d_route, nullptr, nullptr, stream);
}

int mk_decode_step_greedy(mk_ctx* c, int B, int T, int kv_len, const int32_t* d_tokens, void* d_kv,
                          float* d_kda_state, float* d_logits, int32_t* d_argmax, int32_t* d_accepted, void* stream) {
  if (c && !d_argmax) return fail(MK_E_INVAL, "argmax output must be non-NULL");
  return decode_step(c, B, T, kv_len, d_tokens, d_kv, d_kda_state, d_logits, nullptr, d_argmax, d_accepted, stream);
}

int mk_decode_step_sample(mk_ctx* c, int B, int T, int kv_len, const int32_t* d_tokens, void* d_kv,
                          float* d_kda_state, float* d_logits, float temperature, float top_p, const float* d_uniform,
                          int32_t* d_sampled, void* stream) {
  const SampleArgs smp{temperature, top_p, d_uniform, d_sampled};
  return decode_step(c, B, T, kv_len, d_tokens, d_kv, d_kda_state, d_logits, nullptr, nullptr, nullptr, stream, &smp);
}

int mk_decode_step_static(mk_ctx* c, int B, int T, int kv_len, const int32_t* d_tokens, void* d_kv, float* d_kda_state,
                          float* d_logits, int32_t* d_route, void* stream) {
  return decode_step(c, B, T, kv_len, d_tokens, d_kv, d_kda_state, d_logits, d_route, nullptr, nullptr, stream, nullptr,
                     true);
}

int mk_set_trace(mk_ctx* c, int enable) {
  if (!c) return fail(MK_E_INVAL, "context is NULL");
  if (enable && !device_trace_built())
    return fail(MK_E_UNSUPPORTED, "this build has no device tracing: libmk_trace.so (the same sources built with "
                "MK_DEVICE_TRACE) records it");
  c->trace = enable != 0;
  g_err.clear();
  return MK_OK;
}

int mk_set_matrix_cores(mk_ctx* c, int min_rows) {
  if (!c) return fail(MK_E_INVAL, "context is NULL");
  if (min_rows < 2) return fail(MK_E_INVAL, "min_rows %d below 2", min_rows);
  c->mfma_min_rows = min_rows;
  g_err.clear();
  return MK_OK;
}

int mk_read_trace(mk_ctx* c, uint64_t* out, uint64_t capacity, int* n_barriers, int* n_blocks) {
  if (!c || !n_barriers || !n_blocks) return fail(MK_E_INVAL, "NULL argument");
  if (c->device == MK_DEVICE_NONE) return fail(MK_E_STATE, "host-only context has no trace");
  if (!c->trace || c->last_barriers == 0 || !c->ws) return fail(MK_E_STATE, "no traced step since tracing was enabled");
  const uint64_t n = (uint64_t)(c->last_barriers + 1) * c->nblocks * kTraceStamps;
  *n_barriers = c->last_barriers;
  *n_blocks = c->nblocks;
  if (!out) return MK_OK;
  if (capacity < n) return fail(MK_E_NOMEM, "trace needs %llu slots", (unsigned long long)n);
  hipError_t e = hipMemcpy(out, c->ws + c->lt.ws.trace, n * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MK_E_HIP, "trace read failed: %s", hipGetErrorString(e));
  g_err.clear();
  return MK_OK;
}

int mk_poll(mk_ctx* c) {
  if (!c) return fail(MK_E_INVAL, "context is NULL");
  if (c->device == MK_DEVICE_NONE) return c->poisoned ? fail(MK_E_DEVICE, "context poisoned") : MK_OK;
  uint32_t st[4] = {0, 0, 0, 0};
  if (!c->last_status) {  // no step yet
    if (c->poisoned) return fail(MK_E_DEVICE, "context poisoned");
    g_err.clear();
    return MK_OK;
  }
  hipError_t e = hipMemcpy(st, c->last_status, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MK_E_HIP, "status read failed: %s", hipGetErrorString(e));
  if (st[0] != 0 || c->poisoned) {
    c->poisoned = true;
    if (st[3]) return fail(MK_E_DEVICE, "token %u of the step is outside the vocabulary", st[3] - 1);
    return fail(MK_E_DEVICE, "device watchdog fired at grid barrier %u", st[2]);
  }
  g_err.clear();
  return MK_OK;
}

void mk_destroy(mk_ctx* c) { delete c; }

}  // extern "C"
