// mk_internal.h -- layouts shared by the host front end (mk_api.cpp) and the megakernel
// (mk_kernel.hip). Not part of the public ABI.
#pragma once
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

constexpr int kThreads = 512;            // threads per workgroup (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 1024;         // barrier flag slots
constexpr int kLdsFloats = 36 * 1024;    // 144 KiB of LDS per workgroup
constexpr int kChunk = 16;               // minimum cache positions per split-KV task
constexpr int kStatusWords = 64;        // status words: [0] error code, [1] abort flag, [2] detail, [3] token
constexpr int kSub = 32;                 // cache positions an MLA task stages at once
constexpr int kGSub = 64;                // cache positions a GQA task stages at once (one per lane)
constexpr int kGqaTiles = 3;             // GQA value-sum tiles (16 rows x 16 columns) per wave
constexpr int kPartPad = 4;              // a partial is [max, sum, pad, pad, values...]: values 16-byte aligned
constexpr int kMaxExperts = 256;
constexpr int kTraceStamps = MK_TRACE_STAMPS;
constexpr int kMaxRopePairs = 64;
constexpr int kMaxQueue = MK_MAX_M * 8;  // token-expert pairs per step (top_k <= 8)
// Column segments of a matrix-core tile in the instance for at most mm token rows: a 16x16x32
// multiply takes 16 / S weight rows x S consecutive 32-column segments as its 16 A rows and
// 16 / S token rows x the same S segments as its 16 B columns (only the products of matching
// segments are used), so that one load instruction reads 16 / S rows x 64 S contiguous bytes.
constexpr int mfma_segments(int mm) { return mm <= 4 ? 4 : mm <= 8 ? 2 : 1; }
// The allocation-free step's workspace: a device array of the library, one per GPU, held until the
// process ends (mk_decode_step_static). 64 MiB covers every step of the preset models.
constexpr uint64_t kStaticScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;

enum LayerKind : int32_t { kGqa = 0, kMla = 1, kKda = 2 };

// Device-side pointers of one layer, stored in a table at the start of the arena.
struct alignas(16) LayerDev {
  int32_t kind, ord, slot, pad;
  const uint16_t *attn_norm, *moe_norm, *router, *sh_gate, *sh_up, *sh_down, *wo;
  const uint16_t *wq, *wk, *wv;                                     // GQA
  const uint16_t *w_dq, *q_norm, *w_uq, *w_dkv, *kv_norm, *w_ukT, *w_uv;  // MLA (w_ukT: [h][kv_lora][nope])
  const uint16_t *kwq, *kwk, *kwv;                                  // KDA
  const float *alpha, *beta;
  const uint16_t *exp_gate, *exp_up, *exp_down;                     // pool slot base, [E][F][H] / [E][H][F]
  // MoE layers: the router folded onto the attention block's output projection, derived from router,
  // moe_norm and wo when all three are loaded. Row e: [W_r[e][t] g[t] for t < H | sum over t of
  // W_r[e][t] g[t] W_o[t][j] for j < K] (fp32; K the output projection's input width), so that the
  // router logit of x + W_o o before the norm's 1/rms factor is row e . [x | o].
  const float* rwx;
};
static_assert(sizeof(LayerDev) % 16 == 0, "layer table rows are copied in 16-byte units");

// Workspace carve-up (byte offsets from the workspace base).
struct WsLayout {
  uint64_t flags, status, trace, rope, x, x2, ssq, a1, a2, a3, a4, att, o2, part, rlog, sact, eact, amax, scratch, total;
  uint64_t part_floats;  // capacity of the partials buffer in floats
  uint64_t trace_slots;  // barriers x blocks the trace region holds
};

// Everything the kernel needs, passed by value.
struct Params {
  // model
  int32_t L, H, V, nh, nkv, hd, ql, kvl, rd, nd, vd, dk, dv, E, topk, F, SF, norm_topk, cap, Bmax;
  int32_t family;  // attention family: MK_ATTN_GQA, MK_ATTN_MLA or MK_ATTN_HYBRID (the kernel instance)
  float eps, rope_theta;
  // step
  int32_t B, T, M, kv_len, nsplit, chunk;  // chunk: cache positions per split
  uint32_t epoch;
  const int32_t* tokens;
  float* logits;
  int32_t* route;
  // weights
  const LayerDev* layers;
  const uint16_t *embed, *final_norm, *lm_head;
  // caches
  uint16_t* kv;  // GQA: K block then V block; MLA: latent
  float* kda_state;
  // workspace
  uint32_t* flags;   // [kMaxBlocks]: barrier flags, then (the last 128) the merge counters
  uint32_t* status;  // [0] error code, [1] abort flag, [2] detail, [3] token
  float *rope, *x, *a1, *a2, *a3, *a4, *att, *o2, *part, *rlog, *sact, *eact;
  // router fusion (1- and 2-row vector instances of MoE models): the output projection also computes
  // the router logits from the layer's input and its own input (rows rwx of the layer table), and the
  // shared expert's gate/up rows run in the routed-expert phase, one phase fewer per layer. The
  // hidden state then alternates between x (input of even layers) and x2 (input of odd layers).
  int32_t rfuse;
  // split-KV merge and W_uv in one phase (the 1- and 2-row vector instances of MLA layers)
  int32_t mfuse;
  float* x2;
  float* ssq;  // [grid][M] per-workgroup sums of squares of the MoE input (router fusion)
  const char* wsb;    // workspace base: activations are addressed by byte offsets from here
  uint32_t ws_bytes;  // workspace size (< 2^31)
  uint64_t watchdog_ticks;  // wall-clock ticks a barrier may wait
  uint64_t* trace;          // optional [barrier][block][kTraceStamps] wall-clock stamps
  // greedy steps: per-row argmax keys (workspace), the argmax tokens and accepted draft counts
  int32_t greedy;
  unsigned long long* amax;  // [M] (value, index) keys, largest logit then lowest index
  int32_t* argmax;           // [M]
  int32_t* accepted;         // [B] or nullptr
  // sampling steps: temperature / nucleus sampling of every row after the LM head
  int32_t sample;
  float temperature, top_p;
  const float* uniform;  // [M] the caller's uniform numbers in [0, 1)
  int32_t* sampled;      // [M]
};

}  // namespace mk
