/*
 * oracle.c -- fp64 CPU reference of one decode step (test infrastructure; see oracle.h).
 *
 * Written from the plain definitions of each block: RMSNorm, rotary position
 * embedding (rotate-half pairing), scaled dot-product attention with a causal
 * mask, multi-head latent attention over a compressed KV cache, the gated
 * delta rule, a softmax router with top-k, and SwiGLU experts. Loops are in the
 * textbook order; each output element is summed by one thread in index order,
 * so results do not depend on the thread count.
 *
 * A model with n_experts = 0 is a dense decoder: its feed-forward block is the
 * one SwiGLU block of width shared_ffn, applied to every token with weight 1
 * (the dense BF16 decoder the pages serve beside the MoE model:
 * "tpu-megakernels README", FAQ on DSpark and DFlash2).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf(uint16_t u) {
  uint32_t v = (uint32_t)u << 16;
  float f;
  memcpy(&f, &v, 4);
  return (double)f;
}

/* nearest bf16 to x, ties to even, rounded once from double */
uint16_t orc_round_bf16(double x) {
  float f;
  uint32_t u;
  if (x == 0.0 || !isfinite(x)) {
    f = (float)x;
  } else {
    int e;
    double m = frexp(x, &e);            /* x = m * 2^e, 0.5 <= |m| < 1 */
    double r = nearbyint(ldexp(m, 8));  /* keep 8 significant bits */
    f = (float)ldexp(r, e - 8);         /* exact */
  }
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void orc_rmsnorm(const double* x, const uint16_t* gain, int n, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv * bf(gain[i]);
}

/* rotate-half RoPE: pairs (j, j + d/2), frequency theta^(-2j/d) */
void orc_rope(double* x, int d, int pos, double theta) {
  int h = d / 2;
  for (int j = 0; j < h; ++j) {
    double inv_freq = pow(theta, -2.0 * j / d);
    double a = pos * inv_freq;
    double c = cos(a), s = sin(a);
    double x0 = x[j], x1 = x[j + h];
    x[j] = x0 * c - x1 * s;
    x[j + h] = x1 * c + x0 * s;
  }
}

void orc_softmax(const double* s, int n, double* p) {
  double mx = -INFINITY;
  for (int i = 0; i < n; ++i) mx = s[i] > mx ? s[i] : mx;
  double sum = 0.0;
  for (int i = 0; i < n; ++i) {
    p[i] = exp(s[i] - mx);
    sum += p[i];
  }
  for (int i = 0; i < n; ++i) p[i] /= sum;
}

/* k largest of p in descending order; equal values keep the lower index first */
void orc_topk(const double* p, int n, int k, int32_t* idx) {
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int i = 0; i < n; ++i) {
      int taken = 0;
      for (int q = 0; q < j; ++q) taken |= (idx[q] == i);
      if (taken) continue;
      if (best < 0 || p[i] > p[best]) best = i;
    }
    idx[j] = best;
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

void orc_matvec(const uint16_t* W, int rows, int K, const double* x, double* y) {
#pragma omp parallel for schedule(static) if ((long)rows * K > 65536)
  for (int r = 0; r < rows; ++r) {
    const uint16_t* w = W + (size_t)r * K;
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += bf(w[k]) * x[k];
    y[r] = acc;
  }
}

/* Y[m][r] = sum_k W[r][k] X[m][k] for m < M (rows of X and Y strided by ldx / ldy) */
static void matmat(const uint16_t* W, int rows, int K, const double* X, int ldx, int M, double* Y, int ldy) {
#pragma omp parallel for schedule(static) if ((long)rows * K * M > 65536)
  for (int r = 0; r < rows; ++r) {
    const uint16_t* w = W + (size_t)r * K;
    for (int m = 0; m < M; ++m) {
      const double* x = X + (size_t)m * ldx;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += bf(w[k]) * x[k];
      Y[(size_t)m * ldy + r] = acc;
    }
  }
}

void orc_kda_head(double* S, int dk, int dv, const float* alpha, double beta, const double* k,
                  const double* v, const double* q, double* o) {
  /* S <- diag(alpha) S */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= (double)alpha[i];
  /* S <- S - beta k (k^T S) + beta k v^T */
  double* kS = (double*)malloc(sizeof(double) * dv);
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += k[i] * S[(size_t)i * dv + j];
    kS[j] = acc;
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += -beta * k[i] * kS[j] + beta * k[i] * v[j];
  free(kS);
  /* o = S^T q */
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
    o[j] = acc;
  }
}

/* ------------------------------------------------------------------------------------ */

typedef struct {
  orc_fill_fn fill;
  void* user;
} provider;

static uint16_t* get_bf16(const provider* P, int kind, int layer, int expert, size_t n) {
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  P->fill(P->user, kind, layer, expert, n, p);
  return p;
}

static float* get_f32(const provider* P, int kind, int layer, size_t n) {
  float* p = (float*)malloc(n * sizeof(float));
  P->fill(P->user, kind, layer, -1, n, p);
  return p;
}

static int layer_kind(const orc_config* c, int l) {
  if (c->attn_kind != ORC_ATTN_HYBRID) return c->attn_kind;
  return (l % c->hybrid_period == c->hybrid_period - 1) ? ORC_ATTN_MLA : 2; /* 2 = KDA */
}

static int ordinal_of(const orc_config* c, int l) {
  int n = 0, k = layer_kind(c, l);
  for (int i = 0; i < l; ++i) n += (layer_kind(c, i) == k);
  return n;
}

/* ---- GQA attention block: out[M][H] ---- */
static void gqa_block(const orc_config* c, const provider* P, int l, int B, int T, int kv_len, const double* h,
                      orc_io* io, double* out) {
  const int H = c->hidden, nq = c->n_heads, nkv = c->n_kv_heads, d = c->head_dim, M = B * T;
  const int cap = c->kv_capacity;
  uint16_t* Wq = get_bf16(P, ORC_WQ, l, -1, (size_t)nq * d * H);
  uint16_t* Wk = get_bf16(P, ORC_WK, l, -1, (size_t)nkv * d * H);
  uint16_t* Wv = get_bf16(P, ORC_WV, l, -1, (size_t)nkv * d * H);
  uint16_t* Wo = get_bf16(P, ORC_WO, l, -1, (size_t)H * nq * d);
  double* q = (double*)malloc(sizeof(double) * M * nq * d);
  double* k = (double*)malloc(sizeof(double) * M * nkv * d);
  double* v = (double*)malloc(sizeof(double) * M * nkv * d);
  double* o = (double*)malloc(sizeof(double) * M * nq * d);
  matmat(Wq, nq * d, H, h, H, M, q, nq * d);
  matmat(Wk, nkv * d, H, h, H, M, k, nkv * d);
  matmat(Wv, nkv * d, H, h, H, M, v, nkv * d);
  size_t layer_stride = (size_t)io->cache_batch * nkv * cap * d;
  uint16_t* Kc = io->kcache + (size_t)l * layer_stride;
  uint16_t* Vc = io->vcache + (size_t)l * layer_stride;
  /* RoPE, then append all T new entries rounded to bf16 */
  for (int m = 0; m < M; ++m) {
    int b = m / T, t = m % T, pos = kv_len + t;
    for (int i = 0; i < nq; ++i) orc_rope(q + (size_t)m * nq * d + i * d, d, pos, c->rope_theta);
    for (int g = 0; g < nkv; ++g) {
      double* kg = k + (size_t)m * nkv * d + g * d;
      orc_rope(kg, d, pos, c->rope_theta);
      size_t base = (((size_t)b * nkv + g) * cap + pos) * d;
      for (int j = 0; j < d; ++j) {
        Kc[base + j] = orc_round_bf16(kg[j]);
        Vc[base + j] = orc_round_bf16(v[(size_t)m * nkv * d + g * d + j]);
      }
    }
  }
  /* causal attention over the cache */
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int m = 0; m < M; ++m) {
    for (int i = 0; i < nq; ++i) {
      int b = m / T, t = m % T, n = kv_len + t + 1, g = i * nkv / nq;
      const double* qi = q + (size_t)m * nq * d + i * d;
      double* s = (double*)malloc(sizeof(double) * n);
      double* a = (double*)malloc(sizeof(double) * n);
      for (int p = 0; p < n; ++p) {
        const uint16_t* kp = Kc + (((size_t)b * nkv + g) * cap + p) * d;
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += qi[j] * bf(kp[j]);
        s[p] = acc / sqrt((double)d);
      }
      orc_softmax(s, n, a);
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int p = 0; p < n; ++p) acc += a[p] * bf(Vc[(((size_t)b * nkv + g) * cap + p) * d + j]);
        o[(size_t)m * nq * d + i * d + j] = acc;
      }
      free(s);
      free(a);
    }
  }
  matmat(Wo, H, nq * d, o, nq * d, M, out, H);
  free(Wq); free(Wk); free(Wv); free(Wo); free(q); free(k); free(v); free(o);
}

/* ---- MLA block: out[M][H] ---- */
static void mla_block(const orc_config* c, const provider* P, int l, int B, int T, int kv_len, const double* h,
                      orc_io* io, double* out) {
  const int H = c->hidden, nh = c->n_heads, ql = c->q_lora, kvl = c->kv_lora, rd = c->rope_dim;
  const int nd = c->nope_dim, vd = c->v_dim, M = B * T, qd = nd + rd, lat = kvl + rd, cap = c->kv_capacity;
  uint16_t* Wdq = get_bf16(P, ORC_W_DQ, l, -1, (size_t)ql * H);
  uint16_t* gq = get_bf16(P, ORC_Q_NORM, l, -1, ql);
  uint16_t* Wuq = get_bf16(P, ORC_W_UQ, l, -1, (size_t)nh * qd * ql);
  uint16_t* Wdkv = get_bf16(P, ORC_W_DKV, l, -1, (size_t)lat * H);
  uint16_t* gkv = get_bf16(P, ORC_KV_NORM, l, -1, kvl);
  uint16_t* Wuk = get_bf16(P, ORC_W_UK, l, -1, (size_t)nh * nd * kvl);
  uint16_t* Wuv = get_bf16(P, ORC_W_UV, l, -1, (size_t)nh * vd * kvl);
  uint16_t* Wo = get_bf16(P, ORC_WO, l, -1, (size_t)H * nh * vd);
  double* qa = (double*)malloc(sizeof(double) * M * ql);
  double* cq = (double*)malloc(sizeof(double) * M * ql);
  double* q = (double*)malloc(sizeof(double) * M * nh * qd);
  double* kva = (double*)malloc(sizeof(double) * M * lat);
  double* o = (double*)malloc(sizeof(double) * M * nh * vd);
  matmat(Wdq, ql, H, h, H, M, qa, ql);
  for (int m = 0; m < M; ++m) orc_rmsnorm(qa + (size_t)m * ql, gq, ql, c->rms_eps, cq + (size_t)m * ql);
  matmat(Wuq, nh * qd, ql, cq, ql, M, q, nh * qd);
  matmat(Wdkv, lat, H, h, H, M, kva, lat);
  int ord = ordinal_of(c, l);
  uint16_t* Lc = io->latent + (size_t)ord * io->cache_batch * cap * lat;
  double* cnew = (double*)malloc(sizeof(double) * lat);
  for (int m = 0; m < M; ++m) {
    int b = m / T, t = m % T, pos = kv_len + t;
    orc_rmsnorm(kva + (size_t)m * lat, gkv, kvl, c->rms_eps, cnew);
    for (int r = 0; r < rd; ++r) cnew[kvl + r] = kva[(size_t)m * lat + kvl + r];
    orc_rope(cnew + kvl, rd, pos, c->rope_theta);
    uint16_t* dst = Lc + ((size_t)b * cap + pos) * lat;
    for (int j = 0; j < lat; ++j) dst[j] = orc_round_bf16(cnew[j]);
    for (int i = 0; i < nh; ++i) orc_rope(q + (size_t)m * nh * qd + i * qd + nd, rd, pos, c->rope_theta);
  }
  free(cnew);
  const double scale = 1.0 / sqrt((double)qd);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int m = 0; m < M; ++m) {
    for (int i = 0; i < nh; ++i) {
      int b = m / T, t = m % T, n = kv_len + t + 1;
      const double* qn = q + (size_t)m * nh * qd + i * qd;
      const double* qp = qn + nd;
      const uint16_t* wk = Wuk + (size_t)i * nd * kvl;
      const uint16_t* wv = Wuv + (size_t)i * vd * kvl;
      double* s = (double*)malloc(sizeof(double) * n);
      double* a = (double*)malloc(sizeof(double) * n);
      double* oi = o + (size_t)m * nh * vd + i * vd;
      if (!c->mla_explicit) {
        /* absorbed: qt = W_uk^T q_nope, scores against the latent directly */
        double* qt = (double*)malloc(sizeof(double) * kvl);
        double* u = (double*)malloc(sizeof(double) * kvl);
        for (int j = 0; j < kvl; ++j) {
          double acc = 0.0;
          for (int r = 0; r < nd; ++r) acc += bf(wk[(size_t)r * kvl + j]) * qn[r];
          qt[j] = acc;
        }
        for (int p = 0; p < n; ++p) {
          const uint16_t* cp = Lc + ((size_t)b * cap + p) * lat;
          double acc = 0.0;
          for (int j = 0; j < kvl; ++j) acc += qt[j] * bf(cp[j]);
          for (int r = 0; r < rd; ++r) acc += qp[r] * bf(cp[kvl + r]);
          s[p] = acc * scale;
        }
        orc_softmax(s, n, a);
        for (int j = 0; j < kvl; ++j) {
          double acc = 0.0;
          for (int p = 0; p < n; ++p) acc += a[p] * bf(Lc[((size_t)b * cap + p) * lat + j]);
          u[j] = acc;
        }
        for (int v = 0; v < vd; ++v) {
          double acc = 0.0;
          for (int j = 0; j < kvl; ++j) acc += bf(wv[(size_t)v * kvl + j]) * u[j];
          oi[v] = acc;
        }
        free(qt);
        free(u);
      } else {
        /* explicit: reconstruct per-head keys and values from the latent, then plain attention */
        double* kn = (double*)malloc(sizeof(double) * nd);
        double* vv = (double*)malloc(sizeof(double) * (size_t)n * vd);
        for (int p = 0; p < n; ++p) {
          const uint16_t* cp = Lc + ((size_t)b * cap + p) * lat;
          for (int r = 0; r < nd; ++r) {
            double acc = 0.0;
            for (int j = 0; j < kvl; ++j) acc += bf(wk[(size_t)r * kvl + j]) * bf(cp[j]);
            kn[r] = acc;
          }
          for (int v = 0; v < vd; ++v) {
            double acc = 0.0;
            for (int j = 0; j < kvl; ++j) acc += bf(wv[(size_t)v * kvl + j]) * bf(cp[j]);
            vv[(size_t)p * vd + v] = acc;
          }
          double acc = 0.0;
          for (int r = 0; r < nd; ++r) acc += qn[r] * kn[r];
          for (int r = 0; r < rd; ++r) acc += qp[r] * bf(cp[kvl + r]);
          s[p] = acc * scale;
        }
        orc_softmax(s, n, a);
        for (int v = 0; v < vd; ++v) {
          double acc = 0.0;
          for (int p = 0; p < n; ++p) acc += a[p] * vv[(size_t)p * vd + v];
          oi[v] = acc;
        }
        free(kn);
        free(vv);
      }
      free(s);
      free(a);
    }
  }
  matmat(Wo, H, nh * vd, o, nh * vd, M, out, H);
  free(Wdq); free(gq); free(Wuq); free(Wdkv); free(gkv); free(Wuk); free(Wuv); free(Wo);
  free(qa); free(cq); free(q); free(kva); free(o);
}

/* ---- gated delta-rule block: out[M][H] ---- */
static void kda_block(const orc_config* c, const provider* P, int l, int B, int T, const double* h, orc_io* io,
                      double* out) {
  const int H = c->hidden, nh = c->n_heads, dk = c->kda_dk, dv = c->kda_dv, M = B * T;
  uint16_t* Wq = get_bf16(P, ORC_KDA_WQ, l, -1, (size_t)nh * dk * H);
  uint16_t* Wk = get_bf16(P, ORC_KDA_WK, l, -1, (size_t)nh * dk * H);
  uint16_t* Wv = get_bf16(P, ORC_KDA_WV, l, -1, (size_t)nh * dv * H);
  float* alpha = get_f32(P, ORC_KDA_ALPHA, l, (size_t)nh * dk);
  float* beta = get_f32(P, ORC_KDA_BETA, l, nh);
  uint16_t* Wo = get_bf16(P, ORC_WO, l, -1, (size_t)H * nh * dv);
  double* q = (double*)malloc(sizeof(double) * M * nh * dk);
  double* k = (double*)malloc(sizeof(double) * M * nh * dk);
  double* v = (double*)malloc(sizeof(double) * M * nh * dv);
  double* o = (double*)malloc(sizeof(double) * M * nh * dv);
  matmat(Wq, nh * dk, H, h, H, M, q, nh * dk);
  matmat(Wk, nh * dk, H, h, H, M, k, nh * dk);
  matmat(Wv, nh * dv, H, h, H, M, v, nh * dv);
  int ord = ordinal_of(c, l);
  float* St = io->kda_state + (size_t)ord * io->cache_batch * nh * dk * dv;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < nh; ++i) {
      float* Sf = St + ((size_t)b * nh + i) * dk * dv;
      double* S = (double*)malloc(sizeof(double) * dk * dv);
      double* kn = (double*)malloc(sizeof(double) * dk);
      for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = (double)Sf[e];
      for (int t = 0; t < T; ++t) {
        int m = b * T + t;
        const double* kk = k + (size_t)m * nh * dk + i * dk;
        double nrm = 0.0;
        for (int r = 0; r < dk; ++r) nrm += kk[r] * kk[r];
        nrm = sqrt(nrm);
        for (int r = 0; r < dk; ++r) kn[r] = kk[r] / nrm;
        orc_kda_head(S, dk, dv, alpha + (size_t)i * dk, (double)beta[i], kn, v + (size_t)m * nh * dv + i * dv,
                     q + (size_t)m * nh * dk + i * dk, o + (size_t)m * nh * dv + i * dv);
        /* the recurrent state is stored in fp32 */
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = (double)(float)S[e];
      }
      for (size_t e = 0; e < (size_t)dk * dv; ++e) Sf[e] = (float)S[e];
      free(S);
      free(kn);
    }
  }
  matmat(Wo, H, nh * dv, o, nh * dv, M, out, H);
  free(Wq); free(Wk); free(Wv); free(alpha); free(beta); free(Wo); free(q); free(k); free(v); free(o);
}

/* ---- MoE block: out[M][H] = sum_e p_e SwiGLU_e(h) + SwiGLU_shared(h) ---- */
static void swiglu(const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, int H, int F, const double* h,
                   double* y /* [H] */) {
  double* g = (double*)malloc(sizeof(double) * F);
  double* u = (double*)malloc(sizeof(double) * F);
  orc_matvec(Wg, F, H, h, g);
  orc_matvec(Wu, F, H, h, u);
  for (int j = 0; j < F; ++j) g[j] = orc_silu(g[j]) * u[j];
  orc_matvec(Wd, H, F, g, y);
  free(g);
  free(u);
}

/* router (softmax over fp32 logits, top-k) and the selected experts, each weighted by its
 * probability (renormalised over the chosen ones when norm_topk), added into out */
static void routed_experts(const orc_config* c, const provider* P, int l, int M, const double* h, orc_io* io,
                           double* y, double* out) {
  const int H = c->hidden, E = c->n_experts, K = c->top_k, F = c->ffn;
  uint16_t* Wr = get_bf16(P, ORC_ROUTER, l, -1, (size_t)E * H);
  double* r = (double*)malloc(sizeof(double) * M * E);
  double* p = (double*)malloc(sizeof(double) * M * E);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * M * K);
  double* w = (double*)malloc(sizeof(double) * M * K);
  matmat(Wr, E, H, h, H, M, r, E);
  for (int m = 0; m < M; ++m) {
    double* rm = r + (size_t)m * E;
    for (int e = 0; e < E; ++e) rm[e] = (double)(float)rm[e]; /* decision taken on fp32 logits */
    orc_softmax(rm, E, p + (size_t)m * E);
    if (io->force_sel)
      memcpy(sel + (size_t)m * K, io->force_sel + ((size_t)l * M + m) * K, sizeof(int32_t) * K);
    else
      orc_topk(p + (size_t)m * E, E, K, sel + (size_t)m * K);
    double tot = 0.0;
    for (int j = 0; j < K; ++j) tot += p[(size_t)m * E + sel[m * K + j]];
    for (int j = 0; j < K; ++j) {
      double pe = p[(size_t)m * E + sel[m * K + j]];
      w[m * K + j] = c->norm_topk ? pe / tot : pe;
    }
  }
  if (io->sel) memcpy(io->sel + (size_t)l * M * K, sel, sizeof(int32_t) * M * K);
  if (io->probs) memcpy(io->probs + (size_t)l * M * E, p, sizeof(double) * M * E);
  int slot = c->expert_pool_layers ? l % c->expert_pool_layers : l;
  for (int e = 0; e < E; ++e) {
    int used = 0;
    for (int q = 0; q < M * K; ++q) used |= (sel[q] == e);
    if (!used) continue;
    uint16_t* Wg = get_bf16(P, ORC_EXP_GATE, slot, e, (size_t)F * H);
    uint16_t* Wu = get_bf16(P, ORC_EXP_UP, slot, e, (size_t)F * H);
    uint16_t* Wd = get_bf16(P, ORC_EXP_DOWN, slot, e, (size_t)H * F);
    for (int m = 0; m < M; ++m)
      for (int j = 0; j < K; ++j)
        if (sel[m * K + j] == e) {
          swiglu(Wg, Wu, Wd, H, F, h + (size_t)m * H, y);
          for (int i = 0; i < H; ++i) out[(size_t)m * H + i] += w[m * K + j] * y[i];
        }
    free(Wg); free(Wu); free(Wd);
  }
  free(Wr); free(r); free(p); free(sel); free(w);
}

/* the feed-forward block: routed experts (none in a dense model) plus the shared SwiGLU block */
static void moe_block(const orc_config* c, const provider* P, int l, int M, const double* h, orc_io* io,
                      double* out) {
  const int H = c->hidden;
  double* y = (double*)malloc(sizeof(double) * H);
  memset(out, 0, sizeof(double) * M * H);
  if (c->n_experts > 0) routed_experts(c, P, l, M, h, io, y, out);
  if (c->shared_ffn) {
    const int S = c->shared_ffn;
    uint16_t* Wg = get_bf16(P, ORC_SH_GATE, l, -1, (size_t)S * H);
    uint16_t* Wu = get_bf16(P, ORC_SH_UP, l, -1, (size_t)S * H);
    uint16_t* Wd = get_bf16(P, ORC_SH_DOWN, l, -1, (size_t)H * S);
    for (int m = 0; m < M; ++m) {
      swiglu(Wg, Wu, Wd, H, S, h + (size_t)m * H, y);
      for (int i = 0; i < H; ++i) out[(size_t)m * H + i] += y[i];
    }
    free(Wg); free(Wu); free(Wd);
  }
  free(y);
}

int orc_decode_step(const orc_config* c, orc_fill_fn fill, void* user, int B, int T, int kv_len,
                    const int32_t* tokens, orc_io* io, double* logits) {
  if (!c || !fill || !io || !tokens || !logits || B < 1 || T < 1 || kv_len < 0) return -1;
  if (kv_len + T > c->kv_capacity || B > io->cache_batch) return -1;
  provider P = {fill, user};
  const int H = c->hidden, M = B * T, V = c->vocab;
  for (int m = 0; m < M; ++m)
    if (tokens[m] < 0 || tokens[m] >= V) return -1;
  double* x = (double*)malloc(sizeof(double) * M * H);
  double* h = (double*)malloc(sizeof(double) * M * H);
  double* d = (double*)malloc(sizeof(double) * M * H);
  uint16_t* row = (uint16_t*)malloc(sizeof(uint16_t) * H);
  /* embedding rows: fetch the whole table once */
  uint16_t* E = get_bf16(&P, ORC_EMBED, -1, -1, (size_t)V * H);
  for (int m = 0; m < M; ++m)
    for (int i = 0; i < H; ++i) x[(size_t)m * H + i] = bf(E[(size_t)tokens[m] * H + i]);
  free(E);
  if (io->x_trace) memcpy(io->x_trace, x, sizeof(double) * M * H);
  for (int l = 0; l < c->n_layers; ++l) {
    uint16_t* g = get_bf16(&P, ORC_ATTN_NORM, l, -1, H);
    for (int m = 0; m < M; ++m) orc_rmsnorm(x + (size_t)m * H, g, H, c->rms_eps, h + (size_t)m * H);
    free(g);
    int kind = layer_kind(c, l);
    if (kind == ORC_ATTN_GQA)
      gqa_block(c, &P, l, B, T, kv_len, h, io, d);
    else if (kind == ORC_ATTN_MLA)
      mla_block(c, &P, l, B, T, kv_len, h, io, d);
    else
      kda_block(c, &P, l, B, T, h, io, d);
    for (size_t i = 0; i < (size_t)M * H; ++i) x[i] += d[i];
    g = get_bf16(&P, ORC_MOE_NORM, l, -1, H);
    for (int m = 0; m < M; ++m) orc_rmsnorm(x + (size_t)m * H, g, H, c->rms_eps, h + (size_t)m * H);
    free(g);
    moe_block(c, &P, l, M, h, io, d);
    for (size_t i = 0; i < (size_t)M * H; ++i) x[i] += d[i];
    if (io->x_trace) memcpy(io->x_trace + (size_t)(l + 1) * M * H, x, sizeof(double) * M * H);
  }
  uint16_t* g = get_bf16(&P, ORC_FINAL_NORM, -1, -1, H);
  for (int m = 0; m < M; ++m) orc_rmsnorm(x + (size_t)m * H, g, H, c->rms_eps, h + (size_t)m * H);
  free(g);
  uint16_t* Wlm = get_bf16(&P, ORC_LM_HEAD, -1, -1, (size_t)V * H);
  matmat(Wlm, V, H, h, H, M, logits, V);
  free(Wlm);
  free(x); free(h); free(d); free(row);
  return 0;
}
