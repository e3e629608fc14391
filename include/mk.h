/*
 * mk.h -- C ABI of the one-launch MoE decode megakernel for AMD MI355X (gfx950).
 *
 * One call to mk_decode_step runs a whole decode step of a deep MoE transformer
 * -- every layer's RMSNorm, attention (GQA, multi-head latent attention over a
 * compressed cache, or the gated delta rule of the hybrid model), router top-k,
 * SwiGLU routed and shared experts, residuals, and the final norm plus LM head --
 * as a single persistent kernel launch. This is the method of
 * "700 TPS on Kimi K3: A Case for TPU Megakernels" (tpu-megakernels README, FAQ
 * on why to build a custom megakernel: the whole decode step -- attention, MoE,
 * normalisation, residuals -- fused into one kernel; the weights of layer n+1
 * fetched while layer n computes: news digest "TPU 巨核:同样是 16 块芯片,Kimi K3
 * 快 57%", section 差距从哪里来, and the video description "700 tok/s on a 2.8
 * Trillion Model: The 92-Layer TPU Megakernel", timestamp "The Choreography: Layer
 * n+1 Loads While Layer n Computes"), built for one MI355X.
 *
 * The pages describe no kernel-level API (only the servers and their launch scripts:
 * tpu-megakernels README, section "OpenAI-compatible servers"). The calls below are
 * this library's boundary: the model described once, its weights loaded once into
 * device memory the caller owns, then one call per decode step.
 *
 * Ownership: the caller owns every device buffer (weight arena, workspace, KV
 * cache, recurrent state, tokens, logits). The library allocates no device
 * memory; it owns only the host context.
 * Errors: every function returns MK_OK (0) or a negative mk_status; argument
 * errors are detected on the host before anything is launched, and
 * mk_last_error() then describes the failure (thread-local string).
 * Threading: a context may be used by one host thread and one stream at a time
 * (its workspace holds the grid-barrier flags of the running step).
 */
#ifndef MK_H
#define MK_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_MAX_M 16          /* batch * new tokens per step */
#define MK_MAX_BATCH 8
#define MK_MAX_NEW_TOKENS 8
#define MK_MAX_KV_CAPACITY (1 << 20)  /* cache positions per sequence */
#define MK_DEVICE_NONE (-1)  /* host-only context: validates and lays out, never launches */
#define MK_TRACE_STAMPS 16   /* wall-clock stamps per trace record */

typedef enum {
  MK_OK = 0,
  MK_E_INVAL = -1,        /* bad argument: batch, T, kv_len, token pointer, config field, tensor id */
  MK_E_STATE = -2,        /* weights not loaded, host-only context, or context poisoned by a device error */
  MK_E_KV_OVERFLOW = -3,  /* kv_len + n_new_tokens > kv_capacity */
  MK_E_NOMEM = -4,        /* a caller buffer is smaller than mk_query_sizes requires */
  MK_E_HIP = -5,          /* a HIP runtime call failed (message in mk_last_error) */
  MK_E_DEVICE = -6,       /* the device reported an error (watchdog timeout or bad token id); see mk_poll */
  MK_E_UNSUPPORTED = -7   /* valid but not supported by this library (e.g. shape limits) */
} mk_status;

typedef enum { MK_ATTN_GQA = 0, MK_ATTN_MLA = 1, MK_ATTN_HYBRID = 2 } mk_attn_kind;

/* Model and capacity description (a deep MoE decoder whose attention is MLA, or MLA combined with
 * delta-rule linear attention, or GQA: German news article, section "Auf dem Papier liegt der
 * GB200 vorn", on Kimi K3's 92 MoE layers and its mix of delta-rule and latent attention).
 * Matrices are bf16, stored [out][in] (row = output feature).
 * attn_kind GQA: n_heads query heads and n_kv_heads key/value heads of head_dim (32, 64, 96 or
 *   128: the attention runs on the matrix cores), RoPE over the whole head. MLA: n_heads heads, q_lora / kv_lora latent ranks, rope_dim + nope_dim query-key
 *   width per head, v_dim value width. HYBRID: layer l is MLA when l % hybrid_period ==
 *   hybrid_period - 1, otherwise a gated delta-rule layer with n_heads heads of kda_dk x kda_dv.
 * Every layer has a MoE block: n_experts routed SwiGLU experts of width ffn, top_k chosen by a
 * softmax router (weights are the chosen probabilities; renormalised over the chosen set when
 * norm_topk != 0), plus a shared SwiGLU expert of width shared_ffn (0 = none).
 * n_experts = 0 (with top_k = 0, ffn ignored, shared_ffn > 0) describes a dense decoder: its
 * feed-forward block is the shared SwiGLU block alone and there is no router ("tpu-megakernels
 * README", FAQ: the dense BF16 decoder served beside the MoE model). Its layers have one grid
 * phase fewer (no routed-expert phase).
 * expert_pool_layers > 0: layer l uses the expert weights of pool slot l % expert_pool_layers.
 * kv_capacity is at most MK_MAX_KV_CAPACITY positions (larger returns MK_E_UNSUPPORTED). A step
 * splits each sequence's positions into at most one split-KV chunk per workgroup of the grid
 * (at most 256), whatever the length, so the merge of the chunks' partial softmax results and
 * the workspace that holds them do not grow with kv_capacity. */
typedef struct {
  int32_t preset;  /* informational: the mk_config_preset id this description came from, 0 for a custom model */
  int32_t n_layers, hidden, vocab, attn_kind;
  int32_t n_heads, n_kv_heads, head_dim;
  int32_t q_lora, kv_lora, rope_dim, nope_dim, v_dim;
  int32_t kda_dk, kda_dv, hybrid_period;
  int32_t n_experts, top_k, ffn, shared_ffn, norm_topk;
  int32_t expert_pool_layers;
  int32_t max_batch, max_new_tokens, kv_capacity;
  float rms_eps, rope_theta;
} mk_config;

typedef struct {
  uint64_t arena_bytes;      /* weights and the folded router rows derived from them (device, caller-allocated, 256-byte aligned) */
  uint64_t workspace_bytes;  /* activations, attention partials, barrier flags, status (device) */
  uint64_t kv_bytes;         /* KV cache (device), layout below */
  uint64_t kda_state_bytes;  /* recurrent state of delta-rule layers (device, fp32), 0 if none */
} mk_sizes;

/* Weight kinds. Shapes (row-major) for mk_load_weights:
 *   EMBED [vocab][hidden]  FINAL_NORM [hidden]  LM_HEAD [vocab][hidden]
 *   per layer: ATTN_NORM, MOE_NORM [hidden]; ROUTER [n_experts][hidden] (none when n_experts = 0);
 *     SH_GATE, SH_UP [shared_ffn][hidden]; SH_DOWN [hidden][shared_ffn]
 *     GQA: WQ [n_heads*head_dim][hidden], WK, WV [n_kv_heads*head_dim][hidden], WO [hidden][n_heads*head_dim]
 *     MLA: W_DQ [q_lora][hidden], Q_NORM [q_lora], W_UQ [n_heads*(nope_dim+rope_dim)][q_lora]
 *          (per head: nope part first, then rope part), W_DKV [kv_lora+rope_dim][hidden]
 *          (latent first, then the shared rope key), KV_NORM [kv_lora], W_UK [n_heads][nope_dim][kv_lora],
 *          W_UV [n_heads][v_dim][kv_lora], WO [hidden][n_heads*v_dim]
 *     KDA: KDA_WQ, KDA_WK [n_heads*kda_dk][hidden], KDA_WV [n_heads*kda_dv][hidden],
 *          KDA_ALPHA [n_heads][kda_dk] fp32, KDA_BETA [n_heads] fp32, WO [hidden][n_heads*kda_dv]
 *   per pool slot and expert: EXP_GATE, EXP_UP [ffn][hidden]; EXP_DOWN [hidden][ffn]
 * Everything is bf16 except KDA_ALPHA/KDA_BETA. */
typedef enum {
  MK_W_EMBED = 0, MK_W_FINAL_NORM, MK_W_LM_HEAD,
  MK_W_ATTN_NORM, MK_W_WQ, MK_W_WK, MK_W_WV, MK_W_WO,
  MK_W_W_DQ, MK_W_Q_NORM, MK_W_W_UQ, MK_W_W_DKV, MK_W_KV_NORM, MK_W_W_UK, MK_W_W_UV,
  MK_W_KDA_WQ, MK_W_KDA_WK, MK_W_KDA_WV, MK_W_KDA_ALPHA, MK_W_KDA_BETA,
  MK_W_MOE_NORM, MK_W_ROUTER, MK_W_SH_GATE, MK_W_SH_UP, MK_W_SH_DOWN,
  MK_W_EXP_GATE, MK_W_EXP_UP, MK_W_EXP_DOWN,
  MK_W_N_KINDS
} mk_weight_kind;

typedef struct {
  int32_t kind;           /* mk_weight_kind */
  int32_t layer;          /* layer index; pool slot for EXP_*; ignored for global tensors */
  int32_t expert;         /* expert index for EXP_*, otherwise ignored */
  int32_t src_on_device;  /* 1: src is device memory, 0: host memory */
  const void* src;        /* tensor data in the layout above */
  uint64_t bytes;         /* must equal the tensor's size */
} mk_tensor_desc;

typedef struct mk_ctx mk_ctx;

/* Preset model descriptions of the measured and tested workloads. The pages give the deployed model
 * only in outline (92 MoE layers; 2.8 T parameters, 104 B active; tensor-parallel 4 x expert-parallel
 * 8 over 16 chips: video description "700 tok/s on a 2.8 Trillion Model", key takeaways; German news
 * article, section "Auf dem Papier liegt der GB200 vorn"); the dimensions below are synthetic choices.
 *   1  tiny MoE decoder: 2 layers, hidden 256, 4 GQA heads of 64, 8 experts top-2 (ffn 512), vocab 1024
 *   2  mid-size MoE decoder: 8 layers, hidden 2048, GQA 16 / 4 heads of 128, 64 experts top-8 (ffn 768)
 *      plus a shared expert of 768, vocab 32000
 *   3  K3-scale one-GPU share: 92 layers, hidden 7168, MLA 16 heads (q_lora 1536, kv_lora 512, rope 64,
 *      nope 128, v 128), 48 local experts top-1 (ffn 2048) in a 46-layer pool, shared expert 512,
 *      vocabulary slice 40960
 *   4  the same model as 3: the speculative-verify workload differs only in the step (7 new tokens)
 *   5  the hybrid variant of 3: delta-rule layers (16 heads, dk = dv = 128) at positions 1-3 of every
 *      group of 4 layers, MLA at the fourth
 *   6  the dense second model: 64 layers, hidden 5120, GQA 40 / 8 heads of 128, SwiGLU 21504, vocab
 *      151936, RoPE theta 1e6 (the dense BF16 decoder served beside the MoE model: tpu-megakernels
 *      README, FAQ on DSpark and DFlash2)
 * Every preset has max_new_tokens 8, rms_eps 1e-6, max_batch 8 (preset 2: 4), and a cache capacity
 * of the workload's kv_len plus 8 (presets 1 and 2: 136 and 2056; 3-6: 4104). out->preset is set to id.
 * MK_E_INVAL for an unknown id or a NULL out. */
int mk_config_preset(int id, mk_config* out);

/* Sizes of the caller-owned buffers for cfg (the weights stay resident in device memory and are
 * streamed again every step: news digest "TPU 巨核:同样是 16 块芯片,Kimi K3 快 57%", section
 * 差距从哪里来, on every token reading the weights from high-bandwidth memory). Returns MK_E_INVAL / MK_E_UNSUPPORTED for bad configs.
 * KV cache layout (bf16):
 *   GQA:    K block then V block, each [n_layers][max_batch][n_kv_heads][kv_capacity][head_dim]
 *   MLA:    [n_mla_layers][max_batch][kv_capacity][kv_lora + rope_dim]   (normed latent, then
 *           the RoPE'd shared key); MLA layers numbered by their ordinal among MLA layers
 * Delta-rule state (fp32): [n_kda_layers][max_batch][n_heads][kda_dk][kda_dv]. */
int mk_query_sizes(const mk_config* cfg, mk_sizes* out);

/* Create a context on HIP device `device` (or MK_DEVICE_NONE) over caller buffers of at least the
 * queried sizes. The workspace is cleared here (once); the arena is filled by mk_load_weights.
 * A barrier that waits longer than MK_WATCHDOG_MS milliseconds (environment, default 2000) ends
 * the step with MK_E_DEVICE instead of hanging.
 * (The pages' program likewise runs over buffers laid out ahead of time, with static shapes:
 * video description "700 tok/s on a 2.8 Trillion Model", timestamp "What It Costs: Static Shapes,
 * Cold Compiles, and Tradeoffs".) arena and workspace must be 256-byte aligned device pointers;
 * MK_E_NOMEM when a buffer is smaller than queried, MK_E_HIP when a device call fails. */
int mk_create(const mk_config* cfg, int device, void* d_arena, uint64_t arena_bytes, void* d_workspace,
              uint64_t workspace_bytes, mk_ctx** out);

/* Copy (and, where the kernel wants another layout, repack) n tensors into the arena, in stream
 * order on hip_stream. Every tensor of the model must have been loaded once before the first step.
 * Once a MoE layer's ROUTER, MOE_NORM and WO are all in the arena (and again whenever one of them is
 * loaded anew), a kernel on hip_stream derives that layer's folded router rows, which the arena also
 * holds (fp32 [n_experts][hidden + W_o's input width]: ROUTER times MOE_NORM's gain, then that
 * product times WO, summed in fp64): the router logit of x + W_o o is linear in [x | o] before the
 * norm's 1/rms factor, so steps of 1-2 token rows (up to 8 on the matrix cores) compute it in the
 * attention output projection's phase and route right after it. Setting the environment variable
 * MK_NO_ROUTER_FUSION makes every step use the separate router phase instead (for comparisons);
 * MK_NO_MERGE_FUSION likewise keeps the split-KV merge and W_uv in separate phases at 1 to 8 token rows.
 * (The pages' demos likewise prepare their kernel layouts from the checkpoints before serving:
 * tpu-megakernels README, section "Setup".) The source of each descriptor must stay valid until the
 * stream reaches the copy. MK_E_INVAL for an unknown tensor, a wrong byte count or a NULL source. */
int mk_load_weights(mk_ctx* ctx, const mk_tensor_desc* descs, int n, void* hip_stream);

/* One decode step, a single kernel launch, asynchronous on hip_stream (the whole decode step as
 * one program: tpu-megakernels README, FAQ on why to build a custom megakernel; German news
 * article, section "Der Trick: 92 Schichten zu einem Programm verschmelzen").
 * d_tokens [batch][n_new_tokens] int32 (device); new tokens take positions kv_len .. kv_len+T-1 of
 * each sequence, attend causally to positions 0 .. their own, and their cache entries are written
 * (rounded to bf16) at those positions; d_kv holds entries 0 .. kv_len-1 on entry. kv_len is
 * owned by the caller (the step never advances it), so rejected speculative tokens roll back for
 * free. d_kda_state (hybrid only, else NULL) is updated in place. d_logits [batch][n_new_tokens][vocab]
 * fp32 (device). d_route (optional, may be NULL): [n_layers][batch*n_new_tokens][top_k] int32, the
 * selected experts in descending probability. Device-side errors surface through mk_poll. */
int mk_decode_step(mk_ctx* ctx, int batch, int n_new_tokens, int kv_len, const int32_t* d_tokens, void* d_kv,
                   float* d_kda_state, float* d_logits, int32_t* d_route, void* hip_stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc -- mk_decode_step without the context's workspace: the
 * step's activations, split-KV partials, barrier flags and status words live in a device array of
 * the library instead (one per GPU, 64 MiB, held until the process ends; its address on each GPU
 * is looked up once). The call allocates nothing. It launches two kernels on hip_stream: a fill
 * kernel that zeroes the array's barrier flags and status words, then the step. Arguments, outputs
 * and errors are those of mk_decode_step, plus MK_E_UNSUPPORTED when the step needs more workspace
 * than the array holds (activations of batch * n_new_tokens rows and split-KV partials over kv_len +
 * n_new_tokens positions; every step of the preset models fits). The context may have been created
 * without a workspace (NULL, 0 bytes). Every static step on one GPU uses the same array, which
 * keeps the last step's contents: static steps that overlap in time on one GPU (other streams,
 * other threads, other contexts) race, and must not be issued. mk_poll reports the device status
 * of the context's last step as long as no other static step has run on that GPU since. Static
 * steps record no trace. */
int mk_decode_step_static(mk_ctx* ctx, int batch, int n_new_tokens, int kv_len, const int32_t* d_tokens, void* d_kv,
                          float* d_kda_state, float* d_logits, int32_t* d_route, void* hip_stream);

/* The same step with greedy selection fused after the LM head (the pages' serving loop picks the
 * next token on the device: tpu-megakernels README, section on the servers' generation modes;
 * drafts verified in one step: news summary "谷歌TPU v7推理Kimi K3性能超英伟达GB200 57%", background
 * section). d_argmax [batch][n_new_tokens] int32 (device, required) receives, for every new
 * position, the index of its largest logit (the lowest such index on ties). d_logits may be NULL:
 * the logits are then not written. d_accepted [batch] int32 (device, may be NULL) receives, for
 * each sequence, the number of draft tokens accepted by greedy verification: tokens[b][1..T-1] are
 * drafts, and draft j is accepted while tokens[b][j] == argmax[b][j-1] for every j up to it. The
 * step then yields accepted + 1 tokens for the sequence -- the accepted drafts and
 * argmax[b][accepted] -- and the caller continues from kv_len + accepted + 1 (the cache entries of
 * the accepted positions are already written; later ones are overwritten by the next step). One
 * kernel launch, asynchronous on hip_stream; same errors as mk_decode_step, plus MK_E_INVAL for a
 * NULL d_argmax. */
int mk_decode_step_greedy(mk_ctx* ctx, int batch, int n_new_tokens, int kv_len, const int32_t* d_tokens, void* d_kv,
                          float* d_kda_state, float* d_logits, int32_t* d_argmax, int32_t* d_accepted,
                          void* hip_stream);

/* mk_decode_step followed, in the same launch, by temperature / nucleus (top-p) sampling of every
 * position's next token (the MoE model's server offers greedy or temperature/top-p generation:
 * "tpu-megakernels README", section "OpenAI-compatible servers"). With p = softmax(logits /
 * temperature) per position, the kept set is every token whose p is at least tau, tau the largest
 * value at which the kept probability mass reaches top_p (tokens tied with tau are all kept); the
 * sampled token is the first, in index order, at which the running sum of kept probabilities
 * exceeds u times their total, u = d_uniform[b][t]. The library draws no random numbers:
 * d_uniform [batch][n_new_tokens] fp32 in [0, 1) (device) is the caller's. d_logits is required
 * (written as by mk_decode_step, then read back by the sampler); d_sampled [batch][n_new_tokens]
 * int32 (device). One workgroup samples each position: logits in registers, the threshold by
 * bisection on its bits, every sum in a fixed order (the tokens do not vary from run to run).
 * MK_E_INVAL for temperature <= 0 or not finite, top_p outside (0, 1], or a NULL d_logits,
 * d_uniform or d_sampled; otherwise as mk_decode_step. */
int mk_decode_step_sample(mk_ctx* ctx, int batch, int n_new_tokens, int kv_len, const int32_t* d_tokens, void* d_kv,
                          float* d_kda_state, float* d_logits, float temperature, float top_p,
                          const float* d_uniform, int32_t* d_sampled, void* hip_stream);

/* After the caller synchronised the step's stream: MK_OK, or MK_E_DEVICE if the kernel reported a
 * watchdog timeout or an out-of-range token (the context is then poisoned, and later steps return
 * MK_E_STATE). The pages report no device errors; a persistent kernel whose workgroups wait on
 * each other must never hang the GPU, so every wait is bounded by the device clock and an
 * expired wait or an invalid token ends the step with this status instead. */
int mk_poll(mk_ctx* ctx);

/* Profiling (the per-phase view of the step behind the pages' claim that fused phases leave no
 * idle gaps between kernels: news digest "TPU 巨核:同样是 16 块芯片,Kimi K3 快 57%", section
 * 差距从哪里来): while enabled, every step records, for each grid barrier and workgroup,
 * MK_TRACE_STAMPS stamps of the device wall clock (wall_clock64, 100 MHz on MI355X): 0 arrival at
 * the barrier (flag published), 1 departure, then marks of the phase that follows it (0 where a
 * phase has none):
 * 2 input staged (GEMV) or query and first cache rows staged (attention), 3 dot products done
 * (GEMV) or values accumulated (attention), 4 first weight loads issued (GEMV), 5 epilogue written
 * (GEMV), 6 routing done (routed-expert phase), 7 phase entered (the first wave past the barrier),
 * 8 the phase's stores drained, 9 the phase prepared while waiting at its barrier (descriptor,
 * plan, first loads issued), 10 descriptor built, 11 plan built, 12-15 reserved (0). One extra
 * record per workgroup holds the time it finished the step. Tracing is compiled into the library
 * built with MK_DEVICE_TRACE (libmk_trace.so) only: the default build returns MK_E_UNSUPPORTED for
 * enable != 0 (its kernels carry no stamp code, which is 2.4% faster). */
int mk_set_trace(mk_ctx* ctx, int enable);

/* Where the GEMV phases (projections, router, experts, LM head) run. Steps with at least min_rows
 * token rows (batch * n_new_tokens; default MK_MFMA_MIN_ROWS, or MK_MFMA_MIN_ROWS_DENSE for a
 * model without routed experts, where every weight row meets every token row: a 2-row step of the
 * dense preset runs 14% faster on the matrix cores, a 2-row step of the K3-scale share 1.5% slower,
 * its experts seeing about one token each) run them on the matrix cores
 * (16x16x32 bf16 multiplies of 16 weight rows by up to 16 token rows; inputs split into bf16 high
 * and low parts, fp32 accumulation) whenever every row length of the model is a multiple of 32 and
 * every per-head projection comes in whole groups of 16 rows; other steps, and every step when
 * min_rows > MK_MAX_M, run them on the vector units. Batched rows are what a speculative verify
 * step checks at once (the draft tokens are verified together by the large model: news summary
 * "谷歌TPU v7推理Kimi K3性能超英伟达GB200 57%", background section), and the compute share of a step
 * grows with the batch (German news article, section "Der Trick: 92 Schichten zu einem Programm
 * verschmelzen"). Both paths compute the same products in fp32 and differ only in summation
 * order. Takes effect from the next step. MK_E_INVAL for a NULL context or min_rows < 2. */
#define MK_MFMA_MIN_ROWS 3
#define MK_MFMA_MIN_ROWS_DENSE 2
int mk_set_matrix_cores(mk_ctx* ctx, int min_rows);

/* Copy the last traced step (recorded while mk_set_trace is on, for the per-phase view above):
 * out[((barrier * n_blocks) + block) * MK_TRACE_STAMPS + stamp] for
 * barrier < *n_barriers + 1 (the last record is the end of the step). Call with out == NULL to get
 * the counts; capacity is the number of uint64_t slots in out. Synchronous (after the step's stream
 * has finished). */
int mk_read_trace(mk_ctx* ctx, uint64_t* out, uint64_t capacity, int* n_barriers, int* n_blocks);

/* Message of the last failing call on this thread ("" if none). Part of this library's error
 * reporting; the pages define none. */
const char* mk_last_error(void);

/* Release the host context (NULL is ignored). Device buffers stay the caller's; the stream must
 * have finished every step of the context first. */
void mk_destroy(mk_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif
