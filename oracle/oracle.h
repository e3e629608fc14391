/*
 * oracle.h -- plain, slow, fp64 CPU reference of one decode step of a deep MoE
 * transformer (test infrastructure only: it is called by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the product path).
 *
 * What it computes is the plain definition of the step the megakernel runs
 * ("700 TPS on Kimi K3: A Case for TPU Megakernels" README, Results and CPU
 * correctness tests; the megakernel fuses attention, MoE, normalization and
 * residual of the whole decode step into one program, FAQ of the same page):
 *
 *   x = E[tok]
 *   for every layer l:
 *     h = RMSNorm(x; g_attn)
 *     x += attention(h)      GQA with RoPE, MLA over a latent cache, or the
 *                            gated delta rule (KDA) of the hybrid model
 *     h = RMSNorm(x; g_moe)
 *     x += sum_{e in topk(softmax(W_r h))} p_e * SwiGLU_e(h) + SwiGLU_shared(h)
 *   logits = W_lm RMSNorm(x; g_final)
 *
 * Every value is carried in double. Weights and caches arrive as bf16 and are
 * widened exactly; new cache entries are rounded to bf16 when appended, then
 * read back (the cache is bf16 by definition). Router logits are rounded to
 * fp32 before ranking, the precision in which the GPU takes that decision.
 *
 * Parity pins: tests/test_oracle_*.py (closed forms, invariants, brute force,
 * absorbed == explicit MLA, incremental == one-shot). No function here is
 * unpinned.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_ATTN_GQA = 0, ORC_ATTN_MLA = 1, ORC_ATTN_HYBRID = 2 };

enum {
  ORC_EMBED = 0, ORC_FINAL_NORM, ORC_LM_HEAD,
  ORC_ATTN_NORM, ORC_WQ, ORC_WK, ORC_WV, ORC_WO,
  ORC_W_DQ, ORC_Q_NORM, ORC_W_UQ, ORC_W_DKV, ORC_KV_NORM, ORC_W_UK, ORC_W_UV,
  ORC_KDA_WQ, ORC_KDA_WK, ORC_KDA_WV, ORC_KDA_ALPHA, ORC_KDA_BETA,
  ORC_MOE_NORM, ORC_ROUTER, ORC_SH_GATE, ORC_SH_UP, ORC_SH_DOWN,
  ORC_EXP_GATE, ORC_EXP_UP, ORC_EXP_DOWN,
  ORC_N_KINDS
};

typedef struct {
  int32_t n_layers, hidden, vocab, attn_kind;
  int32_t n_heads, n_kv_heads, head_dim;
  int32_t q_lora, kv_lora, rope_dim, nope_dim, v_dim;
  int32_t kda_dk, kda_dv, hybrid_period;
  int32_t n_experts, top_k, ffn, shared_ffn, norm_topk; /* n_experts = 0: dense (shared block only) */
  int32_t expert_pool_layers; /* 0: every layer has its own experts */
  int32_t kv_capacity;        /* positions per cache row */
  int32_t mla_explicit;       /* 1: MLA in the explicit (non-absorbed) form */
  double rms_eps, rope_theta;
} orc_config;

/* Weight provider: write the n elements of tensor (kind, layer, expert) to out.
 * Matrices and gains are bf16 bit patterns (uint16_t); KDA alpha/beta are float.
 * For experts `layer` is the pool slot. Layouts are row-major as in the tensor list. */
typedef void (*orc_fill_fn)(void* user, int kind, int layer, int expert, size_t n, void* out);

typedef struct {
  /* caches (caller-owned, updated in place at positions kv_len .. kv_len+T-1):
   *  GQA:   kcache, vcache  [n_layers][cache_batch][n_kv][kv_capacity][head_dim] bf16
   *  MLA:   latent          [n_mla_layers][cache_batch][kv_capacity][kv_lora+rope] bf16
   *  KDA:   kda_state       [n_kda_layers][cache_batch][n_heads][dk][dv] float (in place)
   * MLA/KDA layers are numbered by their ordinal among layers of the same kind. */
  uint16_t* kcache;
  uint16_t* vcache;
  uint16_t* latent;
  float* kda_state;
  int32_t cache_batch;
  /* optional outputs (NULL to skip) */
  int32_t* sel;         /* [n_layers][B*T][top_k] selected experts, descending probability */
  double* probs;        /* [n_layers][B*T][n_experts] router probabilities */
  double* x_trace;      /* [n_layers+1][B*T][hidden] residual after the embedding and each layer */
  const int32_t* force_sel; /* [n_layers][B*T][top_k]: use these experts instead of top-k */
} orc_io;

/* One decode step. tokens [B][T]; logits out [B][T][vocab] (double).
 * Returns 0, or -1 on invalid arguments. */
int orc_decode_step(const orc_config* cfg, orc_fill_fn fill, void* user, int B, int T, int kv_len,
                    const int32_t* tokens, orc_io* io, double* logits);

/* Building blocks, exported for the pins. */
void orc_rmsnorm(const double* x, const uint16_t* gain, int n, double eps, double* y);
void orc_rope(double* x, int d, int pos, double theta);
void orc_softmax(const double* s, int n, double* p);
void orc_topk(const double* p, int n, int k, int32_t* idx);
double orc_silu(double z);
uint16_t orc_round_bf16(double x);
/* bf16 matvec: y[r] = sum_k W[r][k] x[k], W [rows][K] bf16 */
void orc_matvec(const uint16_t* W, int rows, int K, const double* x, double* y);
/* delta-rule update of one head for one token (S [dk][dv] in place), o [dv] */
void orc_kda_head(double* S, int dk, int dv, const float* alpha, double beta, const double* k,
                  const double* v, const double* q, double* o);

#ifdef __cplusplus
}
#endif
#endif
