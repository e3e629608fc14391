// mk_kernel.hip -- the persistent decode-step megakernel for gfx950.
//
// One launch runs a whole decode step: embedding, every layer's attention block (GQA, MLA over
// a compressed latent cache, or the gated delta rule) and MoE block, the final norm and the
// LM head ("700 TPS on Kimi K3: A Case for TPU Megakernels", README and FAQ: the whole decode
// step as one kernel). The grid is one workgroup per CU; dependent phases are separated by a
// grid barrier built from one flag per workgroup (no same-address atomics), polled by one wave
// with a clock-bounded watchdog so a lost workgroup can never hang the GPU.
//
// Weights stream from HBM with 16-byte loads; each workgroup stages the phase's input
// activations (RMS-normalised on the fly where the block starts with a norm) in LDS and
// computes dot products of its rows against them with fp32 FMAs. Nothing uses float atomics:
// every output element is owned by exactly one lane, so results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

using namespace mk;

namespace {

constexpr int kInFloats = 24576;   // staged input slab
constexpr int kAccFloats = 12288;  // per-task accumulators
static_assert(kInFloats + kAccFloats <= kLdsFloats, "LDS carve-up");

// ----------------------------------------------------------------------------------------------
// small helpers
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void unpack8(const uint4& w, float (&f)[8]) {
  f[0] = lo_bf(w.x); f[1] = hi_bf(w.x); f[2] = lo_bf(w.y); f[3] = hi_bf(w.y);
  f[4] = lo_bf(w.z); f[5] = hi_bf(w.z); f[6] = lo_bf(w.w); f[7] = hi_bf(w.w);
}

__device__ __forceinline__ uint4 ldw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float wave_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ----------------------------------------------------------------------------------------------
// grid barrier: one monotonically increasing flag per workgroup; wave 0 polls all flags
// ----------------------------------------------------------------------------------------------
struct Sync {
  uint32_t gen = 0;
};

__device__ bool grid_sync(const Params& p, Sync& s, int* s_abort) {
  s.gen += 1;
  const uint32_t target = p.epoch + s.gen;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x < 64) {
    if (threadIdx.x == 0) __hip_atomic_store(p.flags + blockIdx.x, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t0 = wall_clock64();
    int abort = 0;
    while (true) {
      int ok = 1;
      for (int i = threadIdx.x; i < (int)gridDim.x; i += 64) {
        uint32_t f = __hip_atomic_load(p.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok &= ((int32_t)(f - target) >= 0);
      }
      if (__all(ok)) break;
      uint32_t ab = __hip_atomic_load(p.status + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ab) {
        abort = 1;
        break;
      }
      if (wall_clock64() - t0 > p.watchdog_ticks) {
        if (threadIdx.x == 0) {
          __hip_atomic_store(p.status + 0, (uint32_t)(-MK_E_DEVICE), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p.status + 2, s.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        abort = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (threadIdx.x == 0) *s_abort = abort;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *s_abort == 0;
}

// ----------------------------------------------------------------------------------------------
// block-wide helpers
// ----------------------------------------------------------------------------------------------
// inv[m] = 1/sqrt(mean(src[m][:K]^2) + eps) for m < M, written to LDS; uses red[] (>= kWaves*16 floats)
__device__ void block_inv_rms(const float* src, int ld, int M, int K, float eps, float* inv, float* red) {
  for (int m = 0; m < M; ++m) {
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += kThreads) {
      float v = src[(size_t)m * ld + k];
      ss += v * v;
    }
    ss = wave_sum(ss, 64);
    if (lane_id() == 0) red[m * kWaves + wave_id()] = ss;
  }
  __syncthreads();
  if (threadIdx.x < M) {
    float t = 0.f;
    for (int w = 0; w < kWaves; ++w) t += red[threadIdx.x * kWaves + w];
    inv[threadIdx.x] = 1.0f / sqrtf(t / (float)K + eps);
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------------------------
// GEMV executor
//
// A phase is a set of tasks; a task is one or two weight rows of length K (two for SwiGLU gate/up
// pairs) dotted with the staged input rows of a list of tokens. The task space is split into
// contiguous ranges per workgroup; within a workgroup lane groups of LPR lanes take tasks. The
// staged input (rows of width Wst) is processed in slabs that fit LDS; partial dot products are
// reduced across the lane group and accumulated in LDS, and the phase's epilogue consumes them.
// ----------------------------------------------------------------------------------------------
struct TaskRows {
  const uint16_t* w0;
  const uint16_t* w1;  // nullptr for single-row tasks
  int xoff;            // offset of the task's input inside a staged row (offset phases)
  int ntok;            // tokens to compute (<= MM)
  const int* tok;      // token slots (indices of staged rows); nullptr = 0..ntok-1
};

template <int MM>
__device__ __forceinline__ void dot_task(const TaskRows& tr, const float* xin, int ldx, int c_begin, int nch, int sub,
                                         int LPR, float (&a0)[MM], float (&a1)[MM]) {
  constexpr int U = 4;
  const bool two = tr.w1 != nullptr;
  int tk[MM];
#pragma unroll
  for (int q = 0; q < MM; ++q) tk[q] = tr.tok ? tr.tok[q < tr.ntok ? q : 0] : q;
  for (int c0 = sub; c0 < nch; c0 += LPR * U) {
    uint4 v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int c = c0 + u * LPR;
      if (c < nch) {
        v0[u] = ldw(tr.w0 + (size_t)(c_begin + c) * 8);
        if (two) v1[u] = ldw(tr.w1 + (size_t)(c_begin + c) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int c = c0 + u * LPR;
      if (c < nch) {
        float f0[8], f1[8];
        unpack8(v0[u], f0);
        if (two) unpack8(v1[u], f1);
#pragma unroll
        for (int q = 0; q < MM; ++q) {
          if (q < tr.ntok) {
            const float* xp = xin + (size_t)tk[q] * ldx + tr.xoff + c * 8;
            float4 xa = *reinterpret_cast<const float4*>(xp);
            float4 xb = *reinterpret_cast<const float4*>(xp + 4);
            a0[q] += f0[0] * xa.x + f0[1] * xa.y + f0[2] * xa.z + f0[3] * xa.w + f0[4] * xb.x + f0[5] * xb.y +
                     f0[6] * xb.z + f0[7] * xb.w;
            if (two)
              a1[q] += f1[0] * xa.x + f1[1] * xa.y + f1[2] * xa.z + f1[3] * xa.w + f1[4] * xb.x + f1[5] * xb.y +
                       f1[6] * xb.z + f1[7] * xb.w;
          }
        }
      }
    }
  }
}

__device__ __forceinline__ int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Ph must provide:
//   int ntasks() const; int K() const; int stage_rows() const; int stage_width() const; bool offsets() const;
//   void stage(float* dst, int k0, int ks) const   (all threads; writes stage_rows() rows of ks floats)
//   TaskRows rows(int t) const;
//   void epilogue(int t, const float* acc0, const float* acc1, int ntok) const   (one lane)
template <int MM, class Ph>
__device__ void gemv_phase(const Ph& ph, float* smem) {
  float* xin = smem;
  float* acc = smem + kInFloats;
  const int nt = ph.ntasks();
  const int t0 = (int)(((long long)nt * blockIdx.x) / gridDim.x);
  const int t1 = (int)(((long long)nt * (blockIdx.x + 1)) / gridDim.x);
  const int nloc = t1 - t0;
  const int R = ph.stage_rows();
  // offset phases stage only the window of input columns their tasks read
  int wbase = 0, Wst = ph.stage_width();
  if (ph.offsets() && nloc > 0) {
    wbase = ph.rows(t0).xoff;
    Wst = ph.rows(t1 - 1).xoff + ph.K() - wbase;
  }
  int KS = Wst;
  if (!ph.offsets()) {
    int cap = (kInFloats / (R > 0 ? R : 1)) & ~511;
    if (cap < 512) cap = 512;
    if (KS > cap) KS = cap;
  }
  const int Kt = ph.K();
  const int nch_full = (ph.offsets() ? Kt : KS) >> 3;
  const int LPR = nch_full >= 64 ? 64 : pow2ceil(nch_full);
  const int G = 64 / LPR;
  const int sub = lane_id() % LPR;
  const int grp = lane_id() / LPR;
  const int per_iter = kWaves * G;
  const int iters = (nloc + per_iter - 1) / per_iter;

  for (int k0 = 0; k0 < Wst; k0 += KS) {
    const int ks = min(KS, Wst - k0);
    __syncthreads();
    ph.stage(xin, wbase + k0, ks);
    __syncthreads();
    const int c_begin = ph.offsets() ? 0 : (k0 >> 3);
    const int nch = ph.offsets() ? (Kt >> 3) : (ks >> 3);
    const int ldx = ks;
    for (int it = 0; it < iters; ++it) {
      const int i = (it * kWaves + wave_id()) * G + grp;
      float a0[MM], a1[MM];
#pragma unroll
      for (int q = 0; q < MM; ++q) a0[q] = a1[q] = 0.f;
      TaskRows tr{nullptr, nullptr, 0, 0, nullptr};
      if (i < nloc) {
        tr = ph.rows(t0 + i);
        tr.xoff -= wbase;
        dot_task<MM>(tr, xin, ldx, c_begin, nch, sub, LPR, a0, a1);
      }
#pragma unroll
      for (int q = 0; q < MM; ++q) {
        a0[q] = wave_sum(a0[q], LPR);
        a1[q] = wave_sum(a1[q], LPR);
      }
      if (i < nloc && sub == 0) {
        float* ac = acc + (size_t)i * 2 * MM;
#pragma unroll
        for (int q = 0; q < MM; ++q) {
          if (k0 == 0) {
            ac[q] = a0[q];
            ac[MM + q] = a1[q];
          } else {
            ac[q] += a0[q];
            ac[MM + q] += a1[q];
          }
        }
      }
    }
  }
  // epilogue: each task by the lane that accumulated it
  for (int it = 0; it < iters; ++it) {
    const int i = (it * kWaves + wave_id()) * G + grp;
    if (i < nloc && sub == 0) {
      TaskRows tr = ph.rows(t0 + i);
      const float* ac = acc + (size_t)i * 2 * MM;
      ph.epilogue(t0 + i, ac, ac + MM, tr.ntok);
    }
  }
}

// ----------------------------------------------------------------------------------------------
// staging sources
// ----------------------------------------------------------------------------------------------
// normalised rows: dst[m][k-k0] = src[m][k] * inv[m] * gain[k]
struct NormSrc {
  const float* src;
  int ld;
  const float* inv;
  const uint16_t* gain;
  int M;
  __device__ void stage(float* dst, int k0, int ks) const {
    const int n = M * ks;
    for (int e = threadIdx.x; e < n; e += kThreads) {
      int m = e / ks, k = e - m * ks;
      dst[e] = src[(size_t)m * ld + k0 + k] * inv[m] * bf2f(gain[k0 + k]);
    }
  }
};

struct PlainSrc {
  const float* src;
  int ld;
  int off;  // column offset inside a source row
  int M;
  __device__ void stage(float* dst, int k0, int ks) const {
    const int n = M * ks;
    for (int e = threadIdx.x; e < n; e += kThreads) {
      int m = e / ks, k = e - m * ks;
      dst[e] = src[(size_t)m * ld + off + k0 + k];
    }
  }
};

// ----------------------------------------------------------------------------------------------
// phases
// ----------------------------------------------------------------------------------------------
// A list of up to three stacked matrices sharing one input: rows [0,n0) of W0 -> out0, ...
struct StackedPhase {
  NormSrc in;
  int K_;
  const uint16_t* W[3];
  int n[3];
  float* out[3];
  int ldo[3];
  int M;
  __device__ int ntasks() const { return n[0] + n[1] + n[2]; }
  __device__ int K() const { return K_; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return K_; }
  __device__ bool offsets() const { return false; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const {
    int s = 0;
    while (t >= n[s]) t -= n[s++];
    return TaskRows{W[s] + (size_t)t * K_, nullptr, 0, M, nullptr};
  }
  __device__ void epilogue(int t, const float* a0, const float*, int ntok) const {
    int s = 0;
    while (t >= n[s]) t -= n[s++];
    for (int q = 0; q < ntok; ++q) out[s][(size_t)q * ldo[s] + t] = a0[q];
  }
};

// rows of one matrix with a plain (already normalised or raw) input; epilogue: store or residual add
struct SimplePhase {
  PlainSrc in;
  int K_;
  const uint16_t* W;
  int n;
  float* out;
  int ldo;
  int resid;  // 1: out += acc
  int M;
  __device__ int ntasks() const { return n; }
  __device__ int K() const { return K_; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return K_; }
  __device__ bool offsets() const { return false; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const { return TaskRows{W + (size_t)t * K_, nullptr, 0, M, nullptr}; }
  __device__ void epilogue(int t, const float* a0, const float*, int ntok) const {
    for (int q = 0; q < ntok; ++q) {
      float* o = out + (size_t)q * ldo + t;
      *o = resid ? *o + a0[q] : a0[q];
    }
  }
};

// per-head GEMV with the input row segment selected by the head: rows (h, j), j < rows_per_head,
// K = seg; input = staged row at offset h * seg. Used for the MLA absorb (W_uk^T) and W_uv.
struct HeadPhase {
  PlainSrc in;
  int width;  // staged row width = heads * seg
  int seg;
  const uint16_t* W;
  int rows_per_head, heads;
  float* out;
  int ldo;
  int M;
  __device__ int ntasks() const { return rows_per_head * heads; }
  __device__ int K() const { return seg; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return width; }
  __device__ bool offsets() const { return true; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const {
    int h = t / rows_per_head;
    return TaskRows{W + (size_t)t * seg, nullptr, h * seg, M, nullptr};
  }
  __device__ void epilogue(int t, const float* a0, const float*, int ntok) const {
    for (int q = 0; q < ntok; ++q) out[(size_t)q * ldo + t] = a0[q];
  }
};

// router logits + shared-expert gate/up pairs (SwiGLU), one input (normalised x)
struct RouterSharedPhase {
  NormSrc in;
  int H, E, SF;
  const uint16_t *Wr, *Wg, *Wu;
  float *rlog, *sact;
  int M;
  __device__ int ntasks() const { return E + SF; }
  __device__ int K() const { return H; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return H; }
  __device__ bool offsets() const { return false; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const {
    if (t < E) return TaskRows{Wr + (size_t)t * H, nullptr, 0, M, nullptr};
    t -= E;
    return TaskRows{Wg + (size_t)t * H, Wu + (size_t)t * H, 0, M, nullptr};
  }
  __device__ void epilogue(int t, const float* a0, const float* a1, int ntok) const {
    if (t < E) {
      for (int q = 0; q < ntok; ++q) rlog[(size_t)q * E + t] = a0[q];
    } else {
      t -= E;
      for (int q = 0; q < ntok; ++q) sact[(size_t)q * SF + t] = silu(a0[q]) * a1[q];
    }
  }
};

// stage the nope parts of every head contiguously: [M][nh*nd] gathered from [M][nh*qd]
struct NopeSrc {
  const float* q;
  int nh, nd, qd, M;
  __device__ void stage(float* dst, int k0, int ks) const {
    const int n = M * ks;
    for (int e = threadIdx.x; e < n; e += kThreads) {
      const int m = e / ks, k = k0 + e - m * ks, h = k / nd, i = k - h * nd;
      dst[e] = q[(size_t)m * nh * qd + h * qd + i];
    }
  }
};
struct AbsorbPhase {
  NopeSrc in;
  const uint16_t* W;
  int nh, nd, kvl;
  float* out;
  int M;
  __device__ int ntasks() const { return nh * kvl; }
  __device__ int K() const { return nd; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return nh * nd; }
  __device__ bool offsets() const { return true; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const {
    return TaskRows{W + (size_t)t * nd, nullptr, (t / kvl) * nd, M, nullptr};
  }
  __device__ void epilogue(int t, const float* a0, const float*, int ntok) const {
    for (int q = 0; q < ntok; ++q) out[(size_t)q * nh * kvl + t] = a0[q];
  }
};

// routing state of one layer, recomputed identically by every workgroup
struct Route {
  int nu;                    // unique experts
  int uexp[kMaxQueue];       // expert id, ascending
  int ustart[kMaxQueue + 1]; // pair range per unique expert
  int ptok[kMaxQueue];       // token of each pair
  float pw[kMaxQueue];       // router weight of each pair
};

struct ExpertUpPhase {
  NormSrc in;
  int H, F;
  const uint16_t *Wg, *Wu;  // pool slot base [E][F][H]
  const Route* rt;
  float* eact;  // [pair][F]
  int M;
  __device__ int ntasks() const { return rt->nu * F; }
  __device__ int K() const { return H; }
  __device__ int stage_rows() const { return M; }
  __device__ int stage_width() const { return H; }
  __device__ bool offsets() const { return false; }
  __device__ void stage(float* d, int k0, int ks) const { in.stage(d, k0, ks); }
  __device__ TaskRows rows(int t) const {
    int u = t / F, j = t - u * F;
    size_t off = ((size_t)rt->uexp[u] * F + j) * H;
    int s = rt->ustart[u];
    return TaskRows{Wg + off, Wu + off, 0, rt->ustart[u + 1] - s, rt->ptok + s};
  }
  __device__ void epilogue(int t, const float* a0, const float* a1, int ntok) const {
    int u = t / F, j = t - u * F;
    int s = rt->ustart[u];
    for (int q = 0; q < ntok; ++q) eact[(size_t)(s + q) * F + j] = silu(a0[q]) * a1[q];
  }
};

// ----------------------------------------------------------------------------------------------
// routing (every workgroup): softmax over the experts of each token, top-k by logit with ties to
// the lower index, then the unique experts in ascending order with their token lists
// ----------------------------------------------------------------------------------------------
__device__ void compute_route(const Params& p, int layer, Route* rt, int* sel_lds, float* w_lds) {
  const int M = p.M, E = p.E, K = p.topk;
  if (threadIdx.x < M) {
    const int m = threadIdx.x;
    const float* r = p.rlog + (size_t)m * E;
    float mx = -INFINITY;
    for (int e = 0; e < E; ++e) mx = fmaxf(mx, r[e]);
    float sum = 0.f;
    for (int e = 0; e < E; ++e) sum += __expf(r[e] - mx);
    int chosen[8];
    float tot = 0.f;
    for (int j = 0; j < K; ++j) {
      int best = -1;
      float bv = 0.f;
      for (int e = 0; e < E; ++e) {
        bool taken = false;
        for (int q = 0; q < j; ++q) taken |= (chosen[q] == e);
        if (taken) continue;
        if (best < 0 || r[e] > bv) {
          best = e;
          bv = r[e];
        }
      }
      chosen[j] = best;
      float pe = __expf(bv - mx) / sum;
      w_lds[m * K + j] = pe;
      sel_lds[m * K + j] = best;
      tot += pe;
    }
    if (p.norm_topk)
      for (int j = 0; j < K; ++j) w_lds[m * K + j] /= tot;
    if (p.route != nullptr && blockIdx.x == 0)
      for (int j = 0; j < K; ++j) p.route[((size_t)layer * M + m) * K + j] = chosen[j];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int nu = 0, np = 0;
    for (int e = 0; e < E; ++e) {
      int start = np;
      for (int m = 0; m < M; ++m)
        for (int j = 0; j < K; ++j)
          if (sel_lds[m * K + j] == e) {
            rt->ptok[np] = m;
            rt->pw[np] = w_lds[m * K + j];
            ++np;
          }
      if (np > start) {
        rt->uexp[nu] = e;
        rt->ustart[nu] = start;
        ++nu;
      }
    }
    rt->ustart[nu] = np;
    rt->nu = nu;
  }
  __syncthreads();
}

// down projections of the routed experts plus the shared expert, weighted and added to x
__device__ void moe_down_phase(const Params& p, const LayerDev& ly, const Route* rt, float* smem) {
  const int H = p.H, F = p.F, SF = p.SF, M = p.M;
  const int np = rt->ustart[rt->nu];
  float* eact = smem;                    // [np][F]
  float* sact = smem + (size_t)np * F;   // [M][SF]
  for (int e = threadIdx.x; e < np * F; e += kThreads) eact[e] = p.eact[e];
  for (int e = threadIdx.x; e < M * SF; e += kThreads) sact[e] = p.sact[e];
  __syncthreads();
  const int r0 = (int)(((long long)H * blockIdx.x) / gridDim.x);
  const int r1 = (int)(((long long)H * (blockIdx.x + 1)) / gridDim.x);
  const int lane = lane_id();
  for (int r = r0 + wave_id(); r < r1; r += kWaves) {
    float acc[MK_MAX_M];
#pragma unroll
    for (int m = 0; m < MK_MAX_M; ++m) acc[m] = 0.f;
    for (int u = 0; u < rt->nu; ++u) {
      const uint16_t* w = ly.exp_down + ((size_t)rt->uexp[u] * H + r) * F;
      const int s0 = rt->ustart[u], s1 = rt->ustart[u + 1];
      for (int c = lane; c < (F >> 3); c += 64) {
        float f[8];
        unpack8(ldw(w + (size_t)c * 8), f);
        for (int s = s0; s < s1; ++s) {
          const float* xp = eact + (size_t)s * F + c * 8;
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) d += f[j] * xp[j];
          const int m = rt->ptok[s];
          const float wgt = rt->pw[s];
#pragma unroll
          for (int mm = 0; mm < MK_MAX_M; ++mm)
            if (mm == m) acc[mm] += wgt * d;
        }
      }
    }
    if (SF > 0) {
      const uint16_t* w = ly.sh_down + (size_t)r * SF;
      for (int c = lane; c < (SF >> 3); c += 64) {
        float f[8];
        unpack8(ldw(w + (size_t)c * 8), f);
#pragma unroll
        for (int m = 0; m < MK_MAX_M; ++m) {
          if (m < M) {
            const float* xp = sact + (size_t)m * SF + c * 8;
            float d = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) d += f[j] * xp[j];
            acc[m] += d;
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MK_MAX_M; ++m) {
      if (m < M) {
        float v = wave_sum(acc[m], 64);
        if (lane == 0) p.x[(size_t)m * H + r] += v;
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// attention
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ void rope_pair(const float* table, int t, int j, float& x0, float& x1) {
  const float c = table[(t * kMaxRopePairs + j) * 2], s = table[(t * kMaxRopePairs + j) * 2 + 1];
  const float a = x0, b = x1;
  x0 = a * c - b * s;
  x1 = b * c + a * s;
}

// GQA split-KV partials. Task (b, g, s): positions [s*C, s*C+C) of sequence b, kv head g, every
// query head of the group and every new token. New positions in the chunk are appended here.
__device__ void gqa_attn_phase(const Params& p, const LayerDev& ly, float* smem) {
  const int d = p.hd, nq = p.nh, nkv = p.nkv, T = p.T, cap = p.cap;
  const int npos = p.kv_len + T;
  const int nsplit = p.nsplit;
  const int qg = nq / nkv;
  const int ntask = p.B * nkv * nsplit;
  float* Ks = smem;                      // [C][d]
  float* Vs = Ks + kChunk * d;           // [C][d]
  float* Qs = Vs + kChunk * d;           // [T*qg][d]
  float* S = Qs + T * qg * d;            // [T*qg][C]
  const size_t lstride = (size_t)p.Bmax * nkv * cap * d;
  uint16_t* Kc = p.kv + (size_t)ly.ord * lstride;
  uint16_t* Vc = p.kv + (size_t)p.L * lstride + (size_t)ly.ord * lstride;
  const float scale = 1.0f / sqrtf((float)d);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, g = (task / nsplit) % nkv, b = task / (nsplit * nkv);
    const int p0 = s * kChunk, p1 = min(npos, p0 + kChunk), np = p1 - p0;
    __syncthreads();
    // stage keys and values (append the new ones)
    for (int e = threadIdx.x; e < np * (d / 2); e += kThreads) {
      const int pl = e / (d / 2), j = e - pl * (d / 2), pos = p0 + pl;
      const size_t ci = (((size_t)b * nkv + g) * cap + pos) * d;
      float k0, k1, v0, v1;
      if (pos < p.kv_len) {
        k0 = bf2f(Kc[ci + j]);
        k1 = bf2f(Kc[ci + j + d / 2]);
        v0 = bf2f(Vc[ci + j]);
        v1 = bf2f(Vc[ci + j + d / 2]);
      } else {
        const int t = pos - p.kv_len, m = b * T + t;
        k0 = p.a2[(size_t)m * nkv * d + g * d + j];
        k1 = p.a2[(size_t)m * nkv * d + g * d + j + d / 2];
        rope_pair(p.rope, t, j, k0, k1);
        const uint16_t kb0 = f2bf(k0), kb1 = f2bf(k1);
        const uint16_t vb0 = f2bf(p.a3[(size_t)m * nkv * d + g * d + j]);
        const uint16_t vb1 = f2bf(p.a3[(size_t)m * nkv * d + g * d + j + d / 2]);
        Kc[ci + j] = kb0;
        Kc[ci + j + d / 2] = kb1;
        Vc[ci + j] = vb0;
        Vc[ci + j + d / 2] = vb1;
        k0 = bf2f(kb0); k1 = bf2f(kb1); v0 = bf2f(vb0); v1 = bf2f(vb1);
      }
      Ks[pl * d + j] = k0;
      Ks[pl * d + j + d / 2] = k1;
      Vs[pl * d + j] = v0;
      Vs[pl * d + j + d / 2] = v1;
    }
    // stage queries (RoPE at each token's position)
    for (int e = threadIdx.x; e < T * qg * (d / 2); e += kThreads) {
      const int r = e / (d / 2), j = e - r * (d / 2);
      const int t = r / qg, hq = g * qg + (r - t * qg), m = b * T + t;
      float q0 = p.a1[(size_t)m * nq * d + hq * d + j], q1 = p.a1[(size_t)m * nq * d + hq * d + j + d / 2];
      rope_pair(p.rope, t, j, q0, q1);
      Qs[r * d + j] = q0;
      Qs[r * d + j + d / 2] = q1;
    }
    __syncthreads();
    const int nr = T * qg;
    for (int e = threadIdx.x; e < nr * kChunk; e += kThreads) {
      const int r = e / kChunk, pl = e - r * kChunk, t = r / qg;
      float sc = -INFINITY;
      if (pl < np && p0 + pl <= p.kv_len + t) {
        float acc = 0.f;
        for (int j = 0; j < d; ++j) acc += Qs[r * d + j] * Ks[pl * d + j];
        sc = acc * scale;
      }
      S[r * kChunk + pl] = sc;
    }
    __syncthreads();
    // per query row: max, sum and weighted values
    for (int r = wave_id(); r < nr; r += kWaves) {
      const int t = r / qg, hq = g * qg + (r - t * qg), m = b * T + t;
      float mx = -INFINITY;
      for (int pl = 0; pl < kChunk; ++pl) mx = fmaxf(mx, S[r * kChunk + pl]);
      float* dst = p.part + ((size_t)(m * nq + hq) * nsplit + s) * (d + 2);
      float l = 0.f;
      for (int j = lane_id(); j < d; j += 64) {
        float acc = 0.f;
        l = 0.f;
        if (mx != -INFINITY) {
          for (int pl = 0; pl < np; ++pl) {
            const float w = (S[r * kChunk + pl] == -INFINITY) ? 0.f : __expf(S[r * kChunk + pl] - mx);
            l += w;
            acc += w * Vs[pl * d + j];
          }
        }
        dst[2 + j] = acc;
      }
      if (lane_id() == 0) {
        dst[0] = mx;
        dst[1] = l;
      }
    }
  }
}

// merge split-KV partials: out[m][h*dim + j] = sum_s e^{mx_s - M} u_s[j] / sum_s e^{mx_s - M} l_s
__device__ void merge_phase(const Params& p, int heads, int dim, float* out) {
  const int ntask = p.M * heads;
  const int nsplit = p.nsplit;
  const int gw = blockIdx.x * kWaves + wave_id(), tw = gridDim.x * kWaves;
  for (int task = gw; task < ntask; task += tw) {
    const float* src = p.part + (size_t)task * nsplit * (dim + 2);
    float mg = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mg = fmaxf(mg, src[(size_t)s * (dim + 2)]);
    float L = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float mx = src[(size_t)s * (dim + 2)];
      if (mx != -INFINITY) L += src[(size_t)s * (dim + 2) + 1] * __expf(mx - mg);
    }
    for (int j = lane_id(); j < dim; j += 64) {
      float acc = 0.f;
      for (int s = 0; s < nsplit; ++s) {
        const float mx = src[(size_t)s * (dim + 2)];
        if (mx != -INFINITY) acc += src[(size_t)s * (dim + 2) + 2 + j] * __expf(mx - mg);
      }
      out[(size_t)task * dim + j] = acc / L;
    }
  }
}

// MLA split-KV partials over the latent cache. Task (b, s): every head and every new token of
// sequence b against positions [s*C, s*C+C). Scores use the absorbed query (W_uk^T q_nope) on the
// latent part and the RoPE'd query on the shared rope key. New entries are appended here.
__device__ void mla_attn_phase(const Params& p, const LayerDev& ly, float* smem, float* misc) {
  const int nh = p.nh, kvl = p.kvl, rd = p.rd, nd = p.nd, T = p.T, cap = p.cap;
  const int lat = kvl + rd, qd = nd + rd;
  const int npos = p.kv_len + T, nsplit = p.nsplit;
  const int ntask = p.B * nsplit;
  float* Cs = smem;                 // [C][lat]
  float* Qt = Cs + kChunk * lat;    // [nh][lat]  (absorbed query | rope query) for one token
  float* S = Qt + nh * lat;         // [nh][C]
  uint16_t* Lc = p.kv + (size_t)ly.ord * p.Bmax * cap * lat;
  const float scale = 1.0f / sqrtf((float)qd);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, b = task / nsplit;
    const int p0 = s * kChunk, p1 = min(npos, p0 + kChunk), np = p1 - p0;
    __syncthreads();
    // RMS of the new latents in this chunk
    for (int pl = wave_id(); pl < np; pl += kWaves) {
      const int pos = p0 + pl;
      if (pos >= p.kv_len) {
        const int m = b * T + (pos - p.kv_len);
        float ss = 0.f;
        for (int j = lane_id(); j < kvl; j += 64) {
          const float v = p.a2[(size_t)m * lat + j];
          ss += v * v;
        }
        ss = wave_sum(ss, 64);
        if (lane_id() == 0) misc[pl] = 1.0f / sqrtf(ss / (float)kvl + p.eps);
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < np * lat; e += kThreads) {
      const int pl = e / lat, j = e - pl * lat, pos = p0 + pl;
      uint16_t* dst = Lc + ((size_t)b * cap + pos) * lat;
      float v;
      if (pos < p.kv_len) {
        v = bf2f(dst[j]);
      } else {
        const int t = pos - p.kv_len, m = b * T + t;
        const float* src = p.a2 + (size_t)m * lat;
        if (j < kvl) {
          v = src[j] * misc[pl] * bf2f(ly.kv_norm[j]);
        } else {
          const int jj = j - kvl, h2 = rd / 2;
          float x0, x1;
          if (jj < h2) {
            x0 = src[kvl + jj];
            x1 = src[kvl + jj + h2];
            rope_pair(p.rope, t, jj, x0, x1);
            v = x0;
          } else {
            x0 = src[kvl + jj - h2];
            x1 = src[kvl + jj];
            rope_pair(p.rope, t, jj - h2, x0, x1);
            v = x1;
          }
        }
        const uint16_t vb = f2bf(v);
        dst[j] = vb;
        v = bf2f(vb);
      }
      Cs[pl * lat + j] = v;
    }
    for (int t = 0; t < T; ++t) {
      const int m = b * T + t;
      __syncthreads();
      for (int e = threadIdx.x; e < nh * lat; e += kThreads) {
        const int h = e / lat, j = e - h * lat;
        float v;
        if (j < kvl) {
          v = p.a4[((size_t)m * nh + h) * kvl + j];
        } else {
          const int jj = j - kvl, h2 = rd / 2;
          const float* qp = p.a3 + (size_t)m * nh * qd + h * qd + nd;
          float x0, x1;
          if (jj < h2) {
            x0 = qp[jj];
            x1 = qp[jj + h2];
            rope_pair(p.rope, t, jj, x0, x1);
            v = x0;
          } else {
            x0 = qp[jj - h2];
            x1 = qp[jj];
            rope_pair(p.rope, t, jj - h2, x0, x1);
            v = x1;
          }
        }
        Qt[e] = v;
      }
      __syncthreads();
      // scores: wave per head pair, lanes over the latent dimension
      for (int h = wave_id(); h < nh; h += kWaves) {
        for (int pl = 0; pl < kChunk; ++pl) {
          float acc = 0.f;
          if (pl < np) {
            for (int j = lane_id(); j < lat; j += 64) acc += Qt[h * lat + j] * Cs[pl * lat + j];
          }
          acc = wave_sum(acc, 64);
          if (lane_id() == 0) S[h * kChunk + pl] = (pl < np && p0 + pl <= p.kv_len + t) ? acc * scale : -INFINITY;
        }
      }
      __syncthreads();
      for (int h = wave_id(); h < nh; h += kWaves) {
        float mx = -INFINITY;
        for (int pl = 0; pl < kChunk; ++pl) mx = fmaxf(mx, S[h * kChunk + pl]);
        float* dst = p.part + ((size_t)(m * nh + h) * nsplit + s) * (kvl + 2);
        float l = 0.f;
        for (int j = lane_id(); j < kvl; j += 64) {
          float acc = 0.f;
          l = 0.f;
          if (mx != -INFINITY) {
            for (int pl = 0; pl < np; ++pl) {
              const float sv = S[h * kChunk + pl];
              const float w = (sv == -INFINITY) ? 0.f : __expf(sv - mx);
              l += w;
              acc += w * Cs[pl * lat + j];
            }
          }
          dst[2 + j] = acc;
        }
        if (lane_id() == 0) {
          dst[0] = mx;
          dst[1] = l;
        }
      }
    }
  }
}

// gated delta rule, one lane column block: task (b, h, cb) owns columns [8cb, 8cb+8) of S_bh
__device__ void kda_phase(const Params& p, const LayerDev& ly) {
  const int nh = p.nh, dk = p.dk, dv = p.dv, T = p.T;
  const int ncb = dv / 8;
  const int ntask = p.B * nh * ncb;
  const int gw = blockIdx.x * kWaves + wave_id(), tw = gridDim.x * kWaves;
  const int lane = lane_id();
  const int rpl = dk / 64;  // rows per lane (dk multiple of 64, <= 128)
  float* St = p.kda_state + (size_t)ly.ord * p.Bmax * nh * dk * dv;
  for (int task = gw; task < ntask; task += tw) {
    const int cb = task % ncb, h = (task / ncb) % nh, b = task / (ncb * nh);
    float* Sbh = St + ((size_t)b * nh + h) * dk * dv;
    float S[2][8];
    float al[2];
    for (int r = 0; r < rpl; ++r) {
      const int i = lane + r * 64;
      const float4 a = *reinterpret_cast<const float4*>(Sbh + (size_t)i * dv + cb * 8);
      const float4 c = *reinterpret_cast<const float4*>(Sbh + (size_t)i * dv + cb * 8 + 4);
      S[r][0] = a.x; S[r][1] = a.y; S[r][2] = a.z; S[r][3] = a.w;
      S[r][4] = c.x; S[r][5] = c.y; S[r][6] = c.z; S[r][7] = c.w;
      al[r] = ly.alpha[h * dk + i];
    }
    const float beta = ly.beta[h];
    for (int t = 0; t < T; ++t) {
      const int m = b * T + t;
      const float* kv = p.a2 + (size_t)m * nh * dk + h * dk;
      const float* qv = p.a1 + (size_t)m * nh * dk + h * dk;
      const float* vv = p.a3 + (size_t)m * nh * dv + h * dv + cb * 8;
      float kk[2], qq[2];
      float nrm = 0.f;
      for (int r = 0; r < rpl; ++r) {
        kk[r] = kv[lane + r * 64];
        qq[r] = qv[lane + r * 64];
        nrm += kk[r] * kk[r];
      }
      nrm = wave_sum(nrm, 64);
      const float inv = 1.0f / sqrtf(nrm);
      for (int r = 0; r < rpl; ++r) kk[r] *= inv;
      float kS[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = 0.f;
        for (int r = 0; r < rpl; ++r) {
          S[r][j] *= al[r];
          a += kk[r] * S[r][j];
        }
        kS[j] = wave_sum(a, 64);
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float vj = vv[j];
        float a = 0.f;
        for (int r = 0; r < rpl; ++r) {
          S[r][j] = S[r][j] - beta * kk[r] * kS[j] + beta * kk[r] * vj;
          a += S[r][j] * qq[r];
        }
        o[j] = wave_sum(a, 64);
      }
      if (lane == 0)
        for (int j = 0; j < 8; ++j) p.att[(size_t)m * nh * dv + h * dv + cb * 8 + j] = o[j];
    }
    for (int r = 0; r < rpl; ++r) {
      const int i = lane + r * 64;
      *reinterpret_cast<float4*>(Sbh + (size_t)i * dv + cb * 8) = make_float4(S[r][0], S[r][1], S[r][2], S[r][3]);
      *reinterpret_cast<float4*>(Sbh + (size_t)i * dv + cb * 8 + 4) = make_float4(S[r][4], S[r][5], S[r][6], S[r][7]);
    }
  }
}

// ----------------------------------------------------------------------------------------------
// the megakernel
// ----------------------------------------------------------------------------------------------
struct Smem {
  float buf[kLdsFloats];
  float inv[MK_MAX_M];
  float red[kWaves * MK_MAX_M];
  float misc[256];
  float rw[kMaxQueue];
  int rsel[kMaxQueue];
  Route route;
  int abort;
};

template <int MM>
__global__ void __launch_bounds__(kThreads, 1) mk_decode_kernel(Params p) {
  __shared__ Smem sm;
  Sync sync;
  const int M = p.M, H = p.H;

  // ---- embedding rows and the RoPE table ----
  {
    const int n = M * H;
    for (int e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) {
      const int m = e / H, i = e - m * H;
      int tok = p.tokens[m];
      if (tok < 0 || tok >= p.V) {
        if (i == 0) {
          __hip_atomic_store(p.status + 0, (uint32_t)(-MK_E_DEVICE), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p.status + 3, (uint32_t)m + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        tok = 0;
      }
      p.x[e] = bf2f(p.embed[(size_t)tok * H + i]);
    }
    if (blockIdx.x == gridDim.x - 1) {
      const int rdim = (p.kvl > 0) ? p.rd : p.hd;
      const int pairs = rdim / 2;
      for (int e = threadIdx.x; e < p.T * pairs; e += kThreads) {
        const int t = e / pairs, j = e - t * pairs;
        const double inv_freq = pow((double)p.rope_theta, -2.0 * j / rdim);
        const double a = (double)(p.kv_len + t) * inv_freq;
        p.rope[(t * kMaxRopePairs + j) * 2] = (float)cos(a);
        p.rope[(t * kMaxRopePairs + j) * 2 + 1] = (float)sin(a);
      }
    }
  }
  if (!grid_sync(p, sync, &sm.abort)) return;

  for (int l = 0; l < p.L; ++l) {
    const LayerDev ly = p.layers[l];
    // ---------------- attention block ----------------
    block_inv_rms(p.x, H, M, H, p.eps, sm.inv, sm.red);
    const NormSrc xn{p.x, H, sm.inv, ly.attn_norm, M};
    if (ly.kind == kGqa) {
      const int dq = p.nh * p.hd, dkv = p.nkv * p.hd;
      StackedPhase ph{xn, H, {ly.wq, ly.wk, ly.wv}, {dq, dkv, dkv}, {p.a1, p.a2, p.a3}, {dq, dkv, dkv}, M};
      gemv_phase<MM>(ph, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      gqa_attn_phase(p, ly, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      merge_phase(p, p.nh, p.hd, p.att);
      if (!grid_sync(p, sync, &sm.abort)) return;
      SimplePhase wo{PlainSrc{p.att, dq, 0, M}, dq, ly.wo, H, p.x, H, 1, M};
      gemv_phase<MM>(wo, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
    } else if (ly.kind == kMla) {
      const int lat = p.kvl + p.rd, qd = p.nd + p.rd;
      StackedPhase ph{xn, H, {ly.w_dq, ly.w_dkv, nullptr}, {p.ql, lat, 0}, {p.a1, p.a2, nullptr}, {p.ql, lat, 0}, M};
      gemv_phase<MM>(ph, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      // q = W_uq RMSNorm(q_a)
      block_inv_rms(p.a1, p.ql, M, p.ql, p.eps, sm.inv, sm.red);
      StackedPhase uq{NormSrc{p.a1, p.ql, sm.inv, ly.q_norm, M}, p.ql, {ly.w_uq, nullptr, nullptr},
                      {p.nh * qd, 0, 0}, {p.a3, nullptr, nullptr}, {p.nh * qd, 0, 0}, M};
      gemv_phase<MM>(uq, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      // absorbed query: qt[h][j] = sum_i W_uk[h][i][j] q_nope[h][i]
      {
        AbsorbPhase ab{NopeSrc{p.a3, p.nh, p.nd, qd, M}, ly.w_ukT, p.nh, p.nd, p.kvl, p.a4, M};
        gemv_phase<MM>(ab, sm.buf);
      }
      if (!grid_sync(p, sync, &sm.abort)) return;
      mla_attn_phase(p, ly, sm.buf, sm.misc);
      if (!grid_sync(p, sync, &sm.abort)) return;
      merge_phase(p, p.nh, p.kvl, p.att);
      if (!grid_sync(p, sync, &sm.abort)) return;
      HeadPhase uv{PlainSrc{p.att, p.nh * p.kvl, 0, M}, p.nh * p.kvl, p.kvl, ly.w_uv, p.vd, p.nh, p.o2, p.nh * p.vd, M};
      gemv_phase<MM>(uv, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      SimplePhase wo{PlainSrc{p.o2, p.nh * p.vd, 0, M}, p.nh * p.vd, ly.wo, H, p.x, H, 1, M};
      gemv_phase<MM>(wo, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
    } else {
      const int dq = p.nh * p.dk, dvv = p.nh * p.dv;
      StackedPhase ph{xn, H, {ly.kwq, ly.kwk, ly.kwv}, {dq, dq, dvv}, {p.a1, p.a2, p.a3}, {dq, dq, dvv}, M};
      gemv_phase<MM>(ph, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
      kda_phase(p, ly);
      if (!grid_sync(p, sync, &sm.abort)) return;
      SimplePhase wo{PlainSrc{p.att, dvv, 0, M}, dvv, ly.wo, H, p.x, H, 1, M};
      gemv_phase<MM>(wo, sm.buf);
      if (!grid_sync(p, sync, &sm.abort)) return;
    }
    // ---------------- MoE block ----------------
    block_inv_rms(p.x, H, M, H, p.eps, sm.inv, sm.red);
    const NormSrc hn{p.x, H, sm.inv, ly.moe_norm, M};
    {
      RouterSharedPhase rs{hn, H, p.E, p.SF, ly.router, ly.sh_gate, ly.sh_up, p.rlog, p.sact, M};
      gemv_phase<MM>(rs, sm.buf);
    }
    if (!grid_sync(p, sync, &sm.abort)) return;
    compute_route(p, l, &sm.route, sm.rsel, sm.rw);
    {
      ExpertUpPhase eu{hn, H, p.F, ly.exp_gate, ly.exp_up, &sm.route, p.eact, M};
      gemv_phase<MM>(eu, sm.buf);
    }
    if (!grid_sync(p, sync, &sm.abort)) return;
    moe_down_phase(p, ly, &sm.route, sm.buf);
    if (!grid_sync(p, sync, &sm.abort)) return;
  }
  // ---- final norm and LM head ----
  block_inv_rms(p.x, H, M, H, p.eps, sm.inv, sm.red);
  StackedPhase lm{NormSrc{p.x, H, sm.inv, p.final_norm, M}, H, {p.lm_head, nullptr, nullptr}, {p.V, 0, 0},
                  {p.logits, nullptr, nullptr}, {p.V, 0, 0}, M};
  gemv_phase<MM>(lm, sm.buf);
}

// W_uk [h][nope][kv_lora] -> W_ukT [h][kv_lora][nope]
__global__ void transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl) {
  const size_t n = (size_t)nh * nd * kvl;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t h = e / ((size_t)nd * kvl), r = e - h * nd * kvl, i = r / kvl, j = r - i * kvl;
    dst[(h * kvl + j) * nd + i] = src[e];
  }
}

}  // namespace

namespace mk {

size_t kernel_lds_bytes() { return sizeof(Smem); }

hipError_t launch_decode(const Params& p, int nblocks, hipStream_t stream) {
  int mm = p.M <= 1 ? 1 : p.M <= 2 ? 2 : p.M <= 4 ? 4 : p.M <= 8 ? 8 : 16;
  switch (mm) {
    case 1: hipLaunchKernelGGL(mk_decode_kernel<1>, dim3(nblocks), dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(mk_decode_kernel<2>, dim3(nblocks), dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(mk_decode_kernel<4>, dim3(nblocks), dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(mk_decode_kernel<8>, dim3(nblocks), dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL(mk_decode_kernel<16>, dim3(nblocks), dim3(kThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_uk, dim3(256), dim3(256), 0, stream, src, dst, nh, nd, kvl);
  return hipGetLastError();
}

hipError_t occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk_decode_kernel<16>, kThreads, 0);
}

}  // namespace mk
