// mk_kernel.hip -- the persistent decode-step megakernel for gfx950.
//
// One launch runs a whole decode step: embedding, every layer's attention block (GQA, MLA over
// a compressed latent cache, or the gated delta rule) and MoE block, the final norm and the
// LM head ("700 TPS on Kimi K3: A Case for TPU Megakernels", README and FAQ: the whole decode
// step as one kernel). The grid is one workgroup per CU; dependent phases are separated by a
// grid barrier built from one flag per workgroup (no same-address atomics), polled by one wave
// with a clock-bounded watchdog so a lost workgroup can never hang the GPU.
//
// Coherence protocol. The L2 caches of the eight XCDs are not coherent with each other, and the
// memory-model fences that would make them so (an L2 writeback on release, an invalidate on
// acquire) cost ~5 us per barrier on MI355X. Instead, every activation that crosses workgroups
// is written with agent-scope stores (written through to the device coherence point) and read
// with agent-scope loads (served from that point, bypassing the non-coherent caches). A
// workgroup completes its stores (s_waitcnt vmcnt(0)) before its polling wave publishes its
// flag, and consumers issue their loads only after observing every flag, so they see the data.
// Weights, the KV cache entries a workgroup owns, and the recurrent state are read and written
// with ordinary cached accesses: within one step no other workgroup touches them.
//
// Prefetch. The weights of a phase do not depend on activations, so every wave except the
// polling one issues the loads of its first task of the next phase before it arrives at the
// barrier ("layer n+1 loads while layer n computes", the news digests' account of the design);
// the barrier wait and the input staging then overlap the HBM latency.
//
// Nothing uses float atomics: every output element is owned by exactly one lane, so results are
// bitwise reproducible from run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

using namespace mk;

// Pointers into device memory are marked global so that loads and stores compile to global_*
// instructions: flat ones would also count against the LDS counter, and the barrier's LDS wait
// would then wait for prefetched weights.
#define GLOBAL __attribute__((address_space(1)))

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ GLOBAL T* gp(T* p) {
  return (GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ const GLOBAL T* gp(const T* p) {
  return (const GLOBAL T*)p;
}

constexpr int kInFloats = 24576;   // staged input slab
constexpr int kAccFloats = 12288;  // per-task accumulators
constexpr int kPollWave = kWaves - 1;
constexpr int kMaxGrid = 256;      // workgroups the barrier polls (4 flags per lane)
static_assert(kInFloats + kAccFloats <= kLdsFloats, "LDS carve-up");
static_assert(sizeof(Params) % 4 == 0, "Params copied as words");

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

__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  const u32x4 v = *(const GLOBAL u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// coherent (device-scope) accesses for activations shared between workgroups
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load((GLOBAL float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ldc2(const float* p) {  // p 8-byte aligned
  const uint64_t u = __hip_atomic_load((GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store((GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldc_u32(const uint32_t* p) {
  return __hip_atomic_load((GLOBAL uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store((GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// execution barrier of the workgroup that does not wait for outstanding global loads
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
// grid barrier
// Every wave has completed its stores (wait_vm) before calling. The polling wave publishes the
// workgroup's flag and polls all flags with independent loads (four per lane).
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ bool grid_sync(const Params& p, uint32_t& gen, int* s_abort) {
  gen += 1;
  const uint32_t target = p.epoch + gen;
  wg_barrier();
  if (wave_id() == kPollWave) {
    const int lane = lane_id();
    uint64_t* tr = p.trace ? p.trace + ((size_t)(gen - 1) * gridDim.x + blockIdx.x) * 4 : nullptr;
    if (lane == 0) {
      if (tr) gp(tr)[0] = wall_clock64();
      stc_u32(p.flags + blockIdx.x, target);
    }
    const uint64_t t0 = wall_clock64();
    int abort = 0;
    while (true) {
      uint32_t f[kMaxGrid / 64];
#pragma unroll
      for (int k = 0; k < kMaxGrid / 64; ++k) {
        const int i = lane + 64 * k;
        f[k] = i < (int)gridDim.x ? ldc_u32(p.flags + i) : target;
      }
      int ok = 1;
#pragma unroll
      for (int k = 0; k < kMaxGrid / 64; ++k) ok &= ((int32_t)(f[k] - target) >= 0);
      if (__all(ok)) break;
      if (ldc_u32(p.status + 1)) {
        abort = 1;
        break;
      }
      if (wall_clock64() - t0 > p.watchdog_ticks) {
        if (lane == 0) {
          stc_u32(p.status + 0, (uint32_t)(-MK_E_DEVICE));
          stc_u32(p.status + 2, gen);
          stc_u32(p.status + 1, 1u);
        }
        abort = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      *s_abort = abort;
      if (tr) gp(tr)[1] = wall_clock64();
    }
  }
  wg_barrier();
  return *s_abort == 0;
}

// ----------------------------------------------------------------------------------------------
// block-wide helpers
// ----------------------------------------------------------------------------------------------
// inv[m] = 1/sqrt(mean(src[m][:K]^2) + eps) for m < M (coherent loads), written to LDS
__device__ __forceinline__ void block_inv_rms(const float* src, int ld, int M, int K, float eps, float* inv, float* red) {
  for (int m = 0; m < M; ++m) {
    float ss = 0.f;
    for (int k = 2 * threadIdx.x; k < K; k += 2 * kThreads) {
      const float2 v = ldc2(src + (size_t)m * ld + k);
      ss += v.x * v.x + v.y * v.y;
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
// GEMV executor (one copy in the kernel, driven by a per-phase descriptor)
//
// A phase is a set of tasks; a task is one or two weight rows of length K (two for SwiGLU gate/up
// pairs) dotted with the staged input rows of a list of tokens. The task space is split into
// contiguous ranges per workgroup; within a workgroup lane groups of LPR lanes take tasks. Each
// lane group streams its rows through two register buffers -- row r+2 is loaded while row r+1 is
// computed -- so a row of loads is always in flight; the first two rows of a phase are loaded
// before the barrier that precedes it. The staged input (rows of width Wst) is processed in slabs
// that fit LDS; partial dot products are reduced across the lane group and accumulated in LDS,
// and the epilogue writes each task's outputs.
// ----------------------------------------------------------------------------------------------
struct TaskRows {
  const uint16_t* w0;
  const uint16_t* w1;  // nullptr for single-row tasks
  int xoff;            // offset of the task's input inside a staged row (offset phases)
  int ntok;            // tokens to compute (<= MM)
  const int* tok;      // token slots (indices of staged rows); nullptr = 0..ntok-1
};

enum GemvKind : int {
  G_STACK = 0,  // up to three stacked matrices, store
  G_RESID,      // one matrix, residual add into the output
  G_OFF,        // per-head rows: row t reads the staged input at (t / rph) * seg, store
  G_RS,         // router rows (store logits) then shared-expert gate/up pairs (store SwiGLU)
  G_EXP,        // routed-expert gate/up pairs of the unique experts (store SwiGLU per pair)
};
enum StageKind : int { S_NORM = 0, S_PLAIN, S_NOPE };

struct Route {
  int nu;                     // unique experts
  int uexp[kMaxQueue];        // expert id, ascending
  int ustart[kMaxQueue + 1];  // pair range per unique expert
  int ptok[kMaxQueue];        // token of each pair
  float pw[kMaxQueue];        // router weight of each pair
};

struct Gemv {
  int kind, stage;
  int ntasks, K, Wst, pairs, M;
  // staging
  const float* src;
  int ld;
  const uint16_t* gain;
  int nh, nd, qd;  // S_NOPE
  float eps;
  // rows and outputs
  const uint16_t *W0, *W1, *W2;
  int n0, n1;
  float *out0, *out1, *out2;
  int ldo0, ldo1, ldo2;
  int rph, seg;  // G_OFF
  int E, SF, F;  // G_RS / G_EXP
  const uint16_t *Wg, *Wu;
  float *rlog, *sact, *eact;
  const Route* rt;

  __device__ __forceinline__ TaskRows rows(int t) const {
    switch (kind) {
      case G_STACK:
        if (t < n0) return TaskRows{W0 + (size_t)t * K, nullptr, 0, M, nullptr};
        if (t < n0 + n1) return TaskRows{W1 + (size_t)(t - n0) * K, nullptr, 0, M, nullptr};
        return TaskRows{W2 + (size_t)(t - n0 - n1) * K, nullptr, 0, M, nullptr};
      case G_RESID:
        return TaskRows{W0 + (size_t)t * K, nullptr, 0, M, nullptr};
      case G_OFF:
        return TaskRows{W0 + (size_t)t * seg, nullptr, (t / rph) * seg, M, nullptr};
      case G_RS:
        if (t < E) return TaskRows{W0 + (size_t)t * K, nullptr, 0, M, nullptr};
        return TaskRows{Wg + (size_t)(t - E) * K, Wu + (size_t)(t - E) * K, 0, M, nullptr};
      default: {  // G_EXP
        const int u = t / F, j = t - u * F;
        const size_t off = ((size_t)rt->uexp[u] * F + j) * K;
        const int s0 = rt->ustart[u];
        return TaskRows{Wg + off, Wu + off, 0, rt->ustart[u + 1] - s0, rt->ptok + s0};
      }
    }
  }

  __device__ __forceinline__ void epilogue(int t, const float* a0, const float* a1, int ntok) const {
    switch (kind) {
      case G_STACK: {
        float* o = out0;
        int ld_o = ldo0;
        if (t >= n0 + n1) {
          o = out2;
          ld_o = ldo2;
          t -= n0 + n1;
        } else if (t >= n0) {
          o = out1;
          ld_o = ldo1;
          t -= n0;
        }
        for (int k = 0; k < ntok; ++k) stc(o + (size_t)k * ld_o + t, a0[k]);
        break;
      }
      case G_RESID:
        for (int k = 0; k < ntok; ++k) {
          float* o = out0 + (size_t)k * ldo0 + t;
          stc(o, ldc(o) + a0[k]);
        }
        break;
      case G_OFF:
        for (int k = 0; k < ntok; ++k) stc(out0 + (size_t)k * ldo0 + t, a0[k]);
        break;
      case G_RS:
        if (t < E) {
          for (int k = 0; k < ntok; ++k) stc(rlog + (size_t)k * E + t, a0[k]);
        } else {
          for (int k = 0; k < ntok; ++k) stc(sact + (size_t)k * SF + (t - E), silu(a0[k]) * a1[k]);
        }
        break;
      default: {  // G_EXP
        const int u = t / F, j = t - u * F;
        const int s0 = rt->ustart[u];
        for (int k = 0; k < ntok; ++k) stc(eact + (size_t)(s0 + k) * F + j, silu(a0[k]) * a1[k]);
      }
    }
  }

  // stage rows [k0, k0+ks) of the input into LDS (all threads). inv/red: LDS scratch.
  __device__ __forceinline__ void stage_in(float* dst, int k0, int ks, float* inv, float* red) const {
    if (stage == S_NORM) {
      if (k0 == 0 && ks == K) {  // one pass: raw rows and their sums of squares
        for (int m = 0; m < M; ++m) {
          float ss = 0.f;
          for (int k = 2 * threadIdx.x; k < K; k += 2 * kThreads) {
            const float2 v = ldc2(src + (size_t)m * ld + k);
            dst[m * ks + k] = v.x;
            dst[m * ks + k + 1] = v.y;
            ss += v.x * v.x + v.y * v.y;
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
        const int n = M * ks;
        for (int e = threadIdx.x; e < n; e += kThreads) {
          const int m = e / ks, k = e - m * ks;
          dst[e] *= inv[m] * bf2f(gp(gain)[k]);
        }
        return;
      }
      if (k0 == 0) block_inv_rms(src, ld, M, K, eps, inv, red);
      const int n = M * ks;
      for (int e = 2 * threadIdx.x; e < n; e += 2 * kThreads) {
        const int m = e / ks, k = e - m * ks;  // ks even, so a pair never straddles rows
        const float2 v = ldc2(src + (size_t)m * ld + k0 + k);
        dst[e] = v.x * inv[m] * bf2f(gp(gain)[k0 + k]);
        dst[e + 1] = v.y * inv[m] * bf2f(gp(gain)[k0 + k + 1]);
      }
    } else if (stage == S_PLAIN) {
      const int n = M * ks;
      for (int e = 2 * threadIdx.x; e < n; e += 2 * kThreads) {
        const int m = e / ks, k = e - m * ks;
        const float2 v = ldc2(src + (size_t)m * ld + k0 + k);
        dst[e] = v.x;
        dst[e + 1] = v.y;
      }
    } else {  // S_NOPE: the nope parts of every head, contiguous [M][nh*nd] from [M][nh*qd]
      const int n = M * ks;
      for (int e = 2 * threadIdx.x; e < n; e += 2 * kThreads) {
        const int m = e / ks, k = k0 + e - m * ks, h = k / nd, i = k - h * nd;  // nd even
        const float2 v = ldc2(src + (size_t)m * nh * qd + h * qd + i);
        dst[e] = v.x;
        dst[e + 1] = v.y;
      }
    }
  }
};

constexpr int kNC = 8;  // 16-byte chunks of one weight-row block a lane holds in registers

struct RowBuf {
  uint4 v[kNC];
};

// Issue the loads of this lane's chunks of one block of a weight row: chunks c = c0 + sub + u*LPR
// (u < kNC, c < nch), at chunk offset c_begin from w. Every load is issued (out-of-range chunks
// read `safe`, a valid address, and are ignored): branches around individual loads make the
// compiler wait for each load before issuing the next.
__device__ __forceinline__ void load_block(const uint16_t* w, int c_begin, int c0, int nch, int sub, int LPR,
                                           const uint16_t* safe, RowBuf& b) {
  const uint16_t* base = w + (size_t)(c_begin + c0 + sub) * 8;
#pragma unroll
  for (int u = 0; u < kNC; ++u) {
    const bool ok = c0 + sub + u * LPR < nch;
    b.v[u] = ldw(ok ? base + (size_t)u * LPR * 8 : safe);
  }
}

// d[q] = this lane's partial dot product of the block with staged input row tok[q]
template <int MM>
__device__ __forceinline__ void dot_block(const RowBuf& b, const float* xin, int ldx, int xoff, const int* tok,
                                          int ntok, int c0, int nch, int sub, int LPR, float (&d)[MM]) {
  int tk[MM];
#pragma unroll
  for (int q = 0; q < MM; ++q) {
    tk[q] = tok ? tok[q < ntok ? q : 0] : q;
    d[q] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < kNC; ++u) {
    const int c = c0 + sub + u * LPR;
    if (c < nch) {
      float f[8];
      unpack8(b.v[u], f);
#pragma unroll
      for (int q = 0; q < MM; ++q) {
        if (q < ntok) {
          const float* xp = xin + (size_t)tk[q] * ldx + xoff + c * 8;
          const float4 xa = *reinterpret_cast<const float4*>(xp);
          const float4 xb = *reinterpret_cast<const float4*>(xp + 4);
          d[q] += f[0] * xa.x + f[1] * xa.y + f[2] * xa.z + f[3] * xa.w + f[4] * xb.x + f[5] * xb.y + f[6] * xb.z +
                  f[7] * xb.w;
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

// Static distribution of a phase's tasks (identical whenever it is computed for the same phase).
// Each lane group streams elements e = (task it, row which, block blk) in that order.
struct Plan {
  int t0, nloc, wbase, Wst, KS, LPR, G, sub, grp, iters, nblk, nel;
  bool one_slab;
};

__device__ __forceinline__ Plan make_plan(const Gemv& g) {
  Plan q;
  const int nt = g.ntasks;
  q.t0 = (int)(((long long)nt * blockIdx.x) / gridDim.x);
  const int t1 = (int)(((long long)nt * (blockIdx.x + 1)) / gridDim.x);
  q.nloc = t1 - q.t0;
  q.wbase = 0;
  q.Wst = g.Wst;
  const bool offs = g.kind == G_OFF;
  if (offs && q.nloc > 0) {  // offset phases stage only the window of columns their tasks read
    q.wbase = (q.t0 / g.rph) * g.seg;
    q.Wst = ((t1 - 1) / g.rph) * g.seg + g.seg - q.wbase;
  }
  q.KS = q.Wst;
  if (!offs) {
    int cap = (kInFloats / g.M) & ~511;
    if (cap < 512) cap = 512;
    if (q.KS > cap) q.KS = cap;
  }
  const int nch_full = (offs ? g.seg : q.KS) >> 3;
  q.LPR = nch_full >= 64 ? 64 : pow2ceil(nch_full);
  q.G = 64 / q.LPR;
  q.sub = lane_id() % q.LPR;
  q.grp = lane_id() / q.LPR;
  const int per_iter = kWaves * q.G;
  q.iters = (q.nloc + per_iter - 1) / per_iter;
  q.nblk = (nch_full + kNC * q.LPR - 1) / (kNC * q.LPR);
  q.nel = q.iters * g.pairs * q.nblk;
  q.one_slab = q.KS >= q.Wst;
  return q;
}

// Issue the loads of stream element e into b (a wave-uniform decision: elements past the end of
// the stream are skipped as a whole; lanes without a task read a valid dummy row).
__device__ __forceinline__ void load_element(const Gemv& g, const Plan& q, int e, int c_begin, int nch, RowBuf& b) {
  if (e >= q.nel) return;
  const int per_task = g.pairs * q.nblk;
  const int it = e / per_task, rem = e - it * per_task, which = rem / q.nblk, blk = rem - which * q.nblk;
  const int i = (it * kWaves + wave_id()) * q.G + q.grp;
  // a row that exists in every model: the first matrix of the phase (the router for G_RS; the
  // shared expert may be absent), or the expert pool of the layer for G_EXP
  const uint16_t* safe = g.kind == G_EXP ? g.Wg : g.W0;
  const uint16_t* w = safe;
  int nc = 0;
  if (i < q.nloc) {
    const TaskRows tr = g.rows(q.t0 + i);
    const uint16_t* wr = which ? tr.w1 : tr.w0;
    if (wr) {
      w = wr;
      nc = nch;
    }
  }
  load_block(w, c_begin, blk * kNC * q.LPR, nc, q.sub, q.LPR, safe, b);
}

// Load the first two elements of this lane group's stream before the barrier (not the polling
// wave, whose poll would otherwise wait for them). Returns 2 when issued, else 0.
__device__ __forceinline__ int gemv_preload(const Gemv& g, RowBuf& b0, RowBuf& b1) {
  if (wave_id() == kPollWave) return 0;
  const Plan q = make_plan(g);
  if (!q.one_slab) return 0;
  const int nch = (g.kind == G_OFF ? g.seg : q.KS) >> 3;
  load_element(g, q, 0, 0, nch, b0);
  load_element(g, q, 1, 0, nch, b1);
  return 2;
}

template <int MM>
__device__ __forceinline__ void reduce_task(const Plan& q, int i, bool first_slab, float (&a0)[MM], float (&a1)[MM],
                                            float* acc) {
#pragma unroll
  for (int k = 0; k < MM; ++k) {
    a0[k] = wave_sum(a0[k], q.LPR);
    a1[k] = wave_sum(a1[k], q.LPR);
  }
  if (i < q.nloc && q.sub == 0) {
    float* ac = acc + (size_t)i * 2 * MM;
#pragma unroll
    for (int k = 0; k < MM; ++k) {
      ac[k] = first_slab ? a0[k] : ac[k] + a0[k];
      ac[MM + k] = first_slab ? a1[k] : ac[MM + k] + a1[k];
    }
  }
#pragma unroll
  for (int k = 0; k < MM; ++k) a0[k] = a1[k] = 0.f;
}

// Consume stream element e from b, then reuse b for element e + 2.
template <int MM>
__device__ __forceinline__ void step_element(const Gemv& g, const Plan& q, int e, int c_begin, int nch,
                                             const float* xin, int ldx, bool first_slab, RowBuf& b, float (&a0)[MM],
                                             float (&a1)[MM], float* acc) {
  const int per_task = g.pairs * q.nblk;
  const int it = e / per_task, rem = e - it * per_task, which = rem / q.nblk, blk = rem - which * q.nblk;
  const int i = (it * kWaves + wave_id()) * q.G + q.grp;
  if (i < q.nloc) {
    const TaskRows tr = g.rows(q.t0 + i);
    if (which == 0 || tr.w1) {
      float d[MM];
      dot_block<MM>(b, xin, ldx, tr.xoff - q.wbase, tr.tok, tr.ntok, blk * kNC * q.LPR, nch, q.sub, q.LPR, d);
#pragma unroll
      for (int k = 0; k < MM; ++k) {
        a0[k] += which ? 0.f : d[k];
        a1[k] += which ? d[k] : 0.f;
      }
    }
  }
  load_element(g, q, e + 2, c_begin, nch, b);
  if (rem == per_task - 1) reduce_task<MM>(q, i, first_slab, a0, a1, acc);
}

template <int MM>
__device__ __forceinline__ void gemv_phase(const Gemv& g, float* smem, float* inv, float* red, RowBuf& b0,
                                           RowBuf& b1, int npre, uint64_t* trace) {
  float* xin = smem;
  float* acc = smem + kInFloats;
  const Plan q = make_plan(g);
  const bool offs = g.kind == G_OFF;
  for (int k0 = 0; k0 < q.Wst; k0 += q.KS) {
    const int ks = min(q.KS, q.Wst - k0);
    const int c_begin = offs ? 0 : (k0 >> 3);
    const int nch = offs ? (g.seg >> 3) : (ks >> 3);
    if (!(k0 == 0 && npre == 2)) {
      load_element(g, q, 0, c_begin, nch, b0);
      load_element(g, q, 1, c_begin, nch, b1);
    }
    __syncthreads();
    g.stage_in(xin, q.wbase + k0, ks, inv, red);
    __syncthreads();
    if (trace && k0 == 0 && threadIdx.x == 0) gp(trace)[2] = wall_clock64();
    float a0[MM], a1[MM];
#pragma unroll
    for (int k = 0; k < MM; ++k) a0[k] = a1[k] = 0.f;
    for (int e = 0; e < q.nel; e += 2) {
      step_element<MM>(g, q, e, c_begin, nch, xin, ks, k0 == 0, b0, a0, a1, acc);
      if (e + 1 < q.nel) step_element<MM>(g, q, e + 1, c_begin, nch, xin, ks, k0 == 0, b1, a0, a1, acc);
    }
  }
  if (trace && threadIdx.x == 0) gp(trace)[3] = wall_clock64();
  // epilogue: each task by the lane that accumulated it
  for (int it = 0; it < q.iters; ++it) {
    const int i = (it * kWaves + wave_id()) * q.G + q.grp;
    if (i < q.nloc && q.sub == 0) {
      const TaskRows tr = g.rows(q.t0 + i);
      const float* ac = acc + (size_t)i * 2 * MM;
      g.epilogue(q.t0 + i, ac, ac + MM, tr.ntok);
    }
  }
}

// ----------------------------------------------------------------------------------------------
// routing (every workgroup): softmax over the experts of each token, top-k by logit with ties to
// the lower index, then the unique experts in ascending order with their token lists
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ void compute_route(const Params& p, int layer, Route* rt, int* sel_lds, float* w_lds, float* r_lds) {
  const int M = p.M, E = p.E, K = p.topk;
  for (int e = threadIdx.x; e < M * E; e += kThreads) r_lds[e] = ldc(p.rlog + e);
  __syncthreads();
  if (threadIdx.x < M) {
    const int m = threadIdx.x;
    const float* r = r_lds + (size_t)m * E;
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
      const float pe = __expf(bv - mx) / sum;
      w_lds[m * K + j] = pe;
      sel_lds[m * K + j] = best;
      tot += pe;
    }
    if (p.norm_topk)
      for (int j = 0; j < K; ++j) w_lds[m * K + j] /= tot;
    if (p.route != nullptr && blockIdx.x == 0)
      for (int j = 0; j < K; ++j) gp(p.route)[((size_t)layer * M + m) * K + j] = chosen[j];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int nu = 0, np = 0;
    for (int e = 0; e < E; ++e) {
      const int start = np;
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
__device__ __forceinline__ void moe_down_phase(const Params& p, const LayerDev& ly, const Route* rt, float* smem) {
  const int H = p.H, F = p.F, SF = p.SF, M = p.M;
  const int np = rt->ustart[rt->nu];
  float* eact = smem;                   // [np][F]
  float* sact = smem + (size_t)np * F;  // [M][SF]
  const int r0 = (int)(((long long)H * blockIdx.x) / gridDim.x);
  const int r1 = (int)(((long long)H * (blockIdx.x + 1)) / gridDim.x);
  const int lane = lane_id();
  const int nchF = F >> 3;
  // the first 256 chunks of the first row's weights in flight while the activations are staged
  uint4 pre[4];
  const int r_first = r0 + wave_id();
  const bool has_pre = rt->nu > 0 && r_first < r1;
  if (has_pre) {
    const uint16_t* w = ly.exp_down + ((size_t)rt->uexp[0] * H + r_first) * F;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = lane + u * 64;
      if (c < nchF) pre[u] = ldw(w + (size_t)c * 8);
    }
  }
  for (int e = 2 * threadIdx.x; e < np * F; e += 2 * kThreads) {
    const float2 v = ldc2(p.eact + e);
    eact[e] = v.x;
    eact[e + 1] = v.y;
  }
  for (int e = 2 * threadIdx.x; e < M * SF; e += 2 * kThreads) {
    const float2 v = ldc2(p.sact + e);
    sact[e] = v.x;
    sact[e + 1] = v.y;
  }
  __syncthreads();
  for (int r = r_first; r < r1; r += kWaves) {
    float acc[MK_MAX_M];
#pragma unroll
    for (int m = 0; m < MK_MAX_M; ++m) acc[m] = 0.f;
    for (int u = 0; u < rt->nu; ++u) {
      const uint16_t* w = ly.exp_down + ((size_t)rt->uexp[u] * H + r) * F;
      const int s0 = rt->ustart[u], s1 = rt->ustart[u + 1];
      for (int cb = 0; cb < nchF; cb += 256) {
        const bool use_pre = has_pre && r == r_first && u == 0 && cb == 0;
        uint4 wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = cb + lane + k * 64;
          if (c < nchF) wv[k] = use_pre ? pre[k] : ldw(w + (size_t)c * 8);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = cb + lane + k * 64;
          if (c >= nchF) continue;
          float f[8];
          unpack8(wv[k], f);
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
        const float v = wave_sum(acc[m], 64);
        if (lane == 0) stc(p.x + (size_t)m * H + r, ldc(p.x + (size_t)m * H + r) + v);
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// attention
// ----------------------------------------------------------------------------------------------
// RoPE table of the step, copied into LDS: table[(t * kMaxRopePairs + j) * 2 + {cos, sin}]
__device__ __forceinline__ void rope_pair(const float* table, int t, int j, float& x0, float& x1) {
  const float c = table[(t * kMaxRopePairs + j) * 2], s = table[(t * kMaxRopePairs + j) * 2 + 1];
  const float a = x0, b = x1;
  x0 = a * c - b * s;
  x1 = b * c + a * s;
}

// GQA split-KV partials. Task (b, g, s): positions [s*C, s*C+C) of sequence b, kv head g, every
// query head of the group and every new token. New positions in the chunk are appended here.
__device__ __forceinline__ void gqa_attn_phase(const Params& p, const LayerDev& ly, float* smem, const float* rope) {
  const int d = p.hd, nq = p.nh, nkv = p.nkv, T = p.T, cap = p.cap;
  const int npos = p.kv_len + T;
  const int nsplit = p.nsplit;
  const int qg = nq / nkv;
  const int ntask = p.B * nkv * nsplit;
  float* Ks = smem;                 // [C][d]
  float* Vs = Ks + kChunk * d;      // [C][d]
  float* Qs = Vs + kChunk * d;      // [T*qg][d]
  float* S = Qs + T * qg * d;       // [T*qg][C]
  const size_t lstride = (size_t)p.Bmax * nkv * cap * d;
  uint16_t* Kc = p.kv + (size_t)ly.ord * lstride;
  uint16_t* Vc = p.kv + (size_t)p.L * lstride + (size_t)ly.ord * lstride;
  const float scale = 1.0f / sqrtf((float)d);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, g = (task / nsplit) % nkv, b = task / (nsplit * nkv);
    const int p0 = s * kChunk, p1 = min(npos, p0 + kChunk), np = p1 - p0;
    __syncthreads();
    for (int e = threadIdx.x; e < np * (d / 2); e += kThreads) {
      const int pl = e / (d / 2), j = e - pl * (d / 2), pos = p0 + pl;
      const size_t ci = (((size_t)b * nkv + g) * cap + pos) * d;
      float k0, k1, v0, v1;
      if (pos < p.kv_len) {
        k0 = bf2f(gp(Kc)[ci + j]);
        k1 = bf2f(gp(Kc)[ci + j + d / 2]);
        v0 = bf2f(gp(Vc)[ci + j]);
        v1 = bf2f(gp(Vc)[ci + j + d / 2]);
      } else {
        const int t = pos - p.kv_len, m = b * T + t;
        k0 = ldc(p.a2 + (size_t)m * nkv * d + g * d + j);
        k1 = ldc(p.a2 + (size_t)m * nkv * d + g * d + j + d / 2);
        rope_pair(rope, t, j, k0, k1);
        const uint16_t kb0 = f2bf(k0), kb1 = f2bf(k1);
        const uint16_t vb0 = f2bf(ldc(p.a3 + (size_t)m * nkv * d + g * d + j));
        const uint16_t vb1 = f2bf(ldc(p.a3 + (size_t)m * nkv * d + g * d + j + d / 2));
        gp(Kc)[ci + j] = kb0;
        gp(Kc)[ci + j + d / 2] = kb1;
        gp(Vc)[ci + j] = vb0;
        gp(Vc)[ci + j + d / 2] = vb1;
        k0 = bf2f(kb0); k1 = bf2f(kb1); v0 = bf2f(vb0); v1 = bf2f(vb1);
      }
      Ks[pl * d + j] = k0;
      Ks[pl * d + j + d / 2] = k1;
      Vs[pl * d + j] = v0;
      Vs[pl * d + j + d / 2] = v1;
    }
    for (int e = threadIdx.x; e < T * qg * (d / 2); e += kThreads) {
      const int r = e / (d / 2), j = e - r * (d / 2);
      const int t = r / qg, hq = g * qg + (r - t * qg), m = b * T + t;
      float q0 = ldc(p.a1 + (size_t)m * nq * d + hq * d + j), q1 = ldc(p.a1 + (size_t)m * nq * d + hq * d + j + d / 2);
      rope_pair(rope, t, j, q0, q1);
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
        stc(dst + 2 + j, acc);
      }
      if (lane_id() == 0) {
        stc(dst, mx);
        stc(dst + 1, l);
      }
    }
  }
}

// Merge split-KV partials: out[m][h*dim + j] = sum_s e^{mx_s - M} u_s[j] / sum_s e^{mx_s - M} l_s.
// Workgroup task (m, h, 32-wide slice of dims): the split weights are computed once into LDS,
// then 16 groups of 32 threads sum disjoint sets of splits and LDS reduces the groups.
__device__ __forceinline__ void merge_phase(const Params& p, int heads, int dim, float* out, float* smem) {
  const int nsplit = p.nsplit;
  const int nj = (dim + 31) / 32;
  const int ntask = p.M * heads * nj;
  float* w = smem;            // [nsplit]
  float* red = smem + 1024;   // [16][32]
  float* misc = smem + 1600;  // [2 * kWaves]
  const int tid = threadIdx.x, sg = tid >> 5, jj = tid & 31;
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int mh = task / nj, j0 = (task - mh * nj) * 32;
    const float* src = p.part + (size_t)mh * nsplit * (dim + 2);
    float mx = -INFINITY;
    for (int s = tid; s < nsplit; s += kThreads) mx = fmaxf(mx, ldc(src + (size_t)s * (dim + 2)));
    mx = wave_max(mx, 64);
    __syncthreads();
    if (lane_id() == 0) misc[wave_id()] = mx;
    __syncthreads();
    float mg = misc[0];
    for (int i = 1; i < kWaves; ++i) mg = fmaxf(mg, misc[i]);
    float lsum = 0.f;
    for (int s = tid; s < nsplit; s += kThreads) {
      const float2 ml = ldc2(src + (size_t)s * (dim + 2));
      const float ws = (ml.x == -INFINITY) ? 0.f : __expf(ml.x - mg);
      w[s] = ws;
      lsum += ws * ml.y;
    }
    lsum = wave_sum(lsum, 64);
    if (lane_id() == 0) misc[kWaves + wave_id()] = lsum;
    __syncthreads();
    float L = 0.f;
    for (int i = 0; i < kWaves; ++i) L += misc[kWaves + i];
    float acc = 0.f;
    const int j = j0 + jj;
    if (j < dim) {
#pragma unroll 8
      for (int s = sg; s < nsplit; s += 16) acc += w[s] * ldc(src + (size_t)s * (dim + 2) + 2 + j);
    }
    red[sg * 32 + jj] = acc;
    __syncthreads();
    if (tid < 32 && j0 + tid < dim) {
      float t = 0.f;
      for (int g = 0; g < 16; ++g) t += red[g * 32 + tid];
      stc(out + (size_t)mh * dim + j0 + tid, t / L);
    }
  }
}

// MLA split-KV partials over the latent cache. Task (b, s): every head and every new token of
// sequence b against positions [s*C, s*C+C). Scores use the absorbed query (W_uk^T q_nope) on the
// latent part and the RoPE'd query on the shared rope key. New entries are appended here.
__device__ __forceinline__ void mla_attn_phase(const Params& p, const LayerDev& ly, float* smem, float* misc, const float* rope) {
  const int nh = p.nh, kvl = p.kvl, rd = p.rd, nd = p.nd, T = p.T, cap = p.cap;
  const int lat = kvl + rd, qd = nd + rd;
  const int npos = p.kv_len + T, nsplit = p.nsplit;
  const int ntask = p.B * nsplit;
  float* Cs = smem;               // [C][lat]
  float* Qt = Cs + kChunk * lat;  // [nh][lat]  (absorbed query | rope query) for one token
  float* S = Qt + nh * lat;       // [nh][C]
  uint16_t* Lc = p.kv + (size_t)ly.ord * p.Bmax * cap * lat;
  const float scale = 1.0f / sqrtf((float)qd);
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, b = task / nsplit;
    const int p0 = s * kChunk, p1 = min(npos, p0 + kChunk), np = p1 - p0;
    __syncthreads();
    for (int pl = wave_id(); pl < np; pl += kWaves) {
      const int pos = p0 + pl;
      if (pos >= p.kv_len) {
        const int m = b * T + (pos - p.kv_len);
        float ss = 0.f;
        for (int j = lane_id(); j < kvl; j += 64) {
          const float v = ldc(p.a2 + (size_t)m * lat + j);
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
        v = bf2f(gp(dst)[j]);
      } else {
        const int t = pos - p.kv_len, m = b * T + t;
        const float* src = p.a2 + (size_t)m * lat;
        if (j < kvl) {
          v = ldc(src + j) * misc[pl] * bf2f(gp(ly.kv_norm)[j]);
        } else {
          const int jj = j - kvl, h2 = rd / 2;
          float x0, x1;
          if (jj < h2) {
            x0 = ldc(src + kvl + jj);
            x1 = ldc(src + kvl + jj + h2);
            rope_pair(rope, t, jj, x0, x1);
            v = x0;
          } else {
            x0 = ldc(src + kvl + jj - h2);
            x1 = ldc(src + kvl + jj);
            rope_pair(rope, t, jj - h2, x0, x1);
            v = x1;
          }
        }
        const uint16_t vb = f2bf(v);
        gp(dst)[j] = vb;
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
          v = ldc(p.a4 + ((size_t)m * nh + h) * kvl + j);
        } else {
          const int jj = j - kvl, h2 = rd / 2;
          const float* qp = p.a3 + (size_t)m * nh * qd + h * qd + nd;
          float x0, x1;
          if (jj < h2) {
            x0 = ldc(qp + jj);
            x1 = ldc(qp + jj + h2);
            rope_pair(rope, t, jj, x0, x1);
            v = x0;
          } else {
            x0 = ldc(qp + jj - h2);
            x1 = ldc(qp + jj);
            rope_pair(rope, t, jj - h2, x0, x1);
            v = x1;
          }
        }
        Qt[e] = v;
      }
      __syncthreads();
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
          stc(dst + 2 + j, acc);
        }
        if (lane_id() == 0) {
          stc(dst, mx);
          stc(dst + 1, l);
        }
      }
    }
  }
}

// gated delta rule: task (b, h, cb) owns columns [8cb, 8cb+8) of S_bh, one wave per task
__device__ __forceinline__ void kda_phase(const Params& p, const LayerDev& ly) {
  const int nh = p.nh, dk = p.dk, dv = p.dv, T = p.T;
  const int ncb = dv / 8;
  const int ntask = p.B * nh * ncb;
  const int gw = blockIdx.x * kWaves + wave_id(), tw = gridDim.x * kWaves;
  const int lane = lane_id();
  const int rpl = dk / 64;  // rows per lane (dk is 64 or 128)
  float* St = p.kda_state + (size_t)ly.ord * p.Bmax * nh * dk * dv;
  for (int task = gw; task < ntask; task += tw) {
    const int cb = task % ncb, h = (task / ncb) % nh, b = task / (ncb * nh);
    float* Sbh = St + ((size_t)b * nh + h) * dk * dv;
    float S[2][8];
    float al[2];
    for (int r = 0; r < rpl; ++r) {
      const int i = lane + r * 64;
      const f32x4 a = *(const GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8);
      const f32x4 c = *(const GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8 + 4);
      S[r][0] = a.x; S[r][1] = a.y; S[r][2] = a.z; S[r][3] = a.w;
      S[r][4] = c.x; S[r][5] = c.y; S[r][6] = c.z; S[r][7] = c.w;
      al[r] = gp(ly.alpha)[h * dk + i];
    }
    const float beta = gp(ly.beta)[h];
    for (int t = 0; t < T; ++t) {
      const int m = b * T + t;
      const float* kv = p.a2 + (size_t)m * nh * dk + h * dk;
      const float* qv = p.a1 + (size_t)m * nh * dk + h * dk;
      const float* vv = p.a3 + (size_t)m * nh * dv + h * dv + cb * 8;
      float kk[2], qq[2];
      float nrm = 0.f;
      for (int r = 0; r < rpl; ++r) {
        kk[r] = ldc(kv + lane + r * 64);
        qq[r] = ldc(qv + lane + r * 64);
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
        const float vj = ldc(vv + j);
        float a = 0.f;
        for (int r = 0; r < rpl; ++r) {
          S[r][j] = S[r][j] - beta * kk[r] * kS[j] + beta * kk[r] * vj;
          a += S[r][j] * qq[r];
        }
        o[j] = wave_sum(a, 64);
      }
      if (lane == 0)
        for (int j = 0; j < 8; ++j) stc(p.att + (size_t)m * nh * dv + h * dv + cb * 8 + j, o[j]);
    }
    for (int r = 0; r < rpl; ++r) {
      const int i = lane + r * 64;
      *(GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8) = f32x4{S[r][0], S[r][1], S[r][2], S[r][3]};
      *(GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8 + 4) = f32x4{S[r][4], S[r][5], S[r][6], S[r][7]};
    }
  }
}

// ----------------------------------------------------------------------------------------------
// the megakernel: an interpreter over the phases of the step
//
// Every layer is a short sequence of phases (GQA: qkv, attention, merge, W_o; MLA: q_a/kv_a, q_b,
// absorb, attention, merge, W_uv, W_o; delta rule: qkv, recurrence, W_o; then MoE: router +
// shared up, routed experts up, down + residual), followed after the last layer by the LM head.
// The kernel walks that sequence with one copy of each phase's code: a barrier precedes every
// phase, and a GEMV phase's first weight rows are requested before it.
// ----------------------------------------------------------------------------------------------
struct Smem {
  float buf[kLdsFloats];
  float inv[MK_MAX_M];
  float red[kWaves * MK_MAX_M];
  float misc[256];
  float rope[MK_MAX_NEW_TOKENS * kMaxRopePairs * 2];
  float rw[kMaxQueue];
  int rsel[kMaxQueue];
  Route route;
  int abort;
};

enum PhaseType : int { PT_GEMV = 0, PT_ATTN_GQA, PT_ATTN_MLA, PT_MERGE, PT_KDA, PT_EXPERT, PT_DOWN };

__device__ __forceinline__ int attn_phases(int kind) { return kind == kGqa ? 4 : kind == kMla ? 7 : 3; }

__device__ __forceinline__ void norm_input(Gemv& g, const float* src, int ld, int K, const uint16_t* gain) {
  g.stage = S_NORM;
  g.src = src;
  g.ld = ld;
  g.K = K;
  g.Wst = K;
  g.gain = gain;
}
__device__ __forceinline__ void plain_input(Gemv& g, const float* src, int ld, int K) {
  g.stage = S_PLAIN;
  g.src = src;
  g.ld = ld;
  g.K = K;
  g.Wst = K;
}

// Phase i of layer l (l == L: the final norm and LM head). Fills g for GEMV phases.
__device__ __forceinline__ int describe(const Params& p, int l, int i, Gemv& g) {
  g.M = p.M;
  g.eps = p.eps;
  g.pairs = 1;
  g.n1 = 0;
  if (l == p.L) {
    norm_input(g, p.x, p.H, p.H, p.final_norm);
    g.kind = G_STACK;
    g.W0 = p.lm_head;
    g.n0 = p.V;
    g.out0 = p.logits;
    g.ldo0 = p.V;
    g.ntasks = p.V;
    return PT_GEMV;
  }
  const GLOBAL LayerDev* ly = gp(p.layers + l);
  const int kind = ly->kind;
  const int na = attn_phases(kind);
  if (i >= na) {
    norm_input(g, p.x, p.H, p.H, ly->moe_norm);
    if (i == na) {
      g.kind = G_RS;
      g.E = p.E;
      g.SF = p.SF;
      g.W0 = ly->router;
      g.Wg = ly->sh_gate;
      g.Wu = ly->sh_up;
      g.rlog = p.rlog;
      g.sact = p.sact;
      g.ntasks = p.E + p.SF;
      g.pairs = 2;
      return PT_GEMV;
    }
    if (i == na + 1) {
      g.kind = G_EXP;
      g.F = p.F;
      g.Wg = ly->exp_gate;
      g.Wu = ly->exp_up;
      g.eact = p.eact;
      g.pairs = 2;
      g.ntasks = 0;  // known after routing
      return PT_EXPERT;
    }
    return PT_DOWN;
  }
  if (kind == kGqa) {
    const int dq = p.nh * p.hd, dkv = p.nkv * p.hd;
    if (i == 0) {
      norm_input(g, p.x, p.H, p.H, ly->attn_norm);
      g.kind = G_STACK;
      g.W0 = ly->wq; g.W1 = ly->wk; g.W2 = ly->wv;
      g.n0 = dq; g.n1 = dkv;
      g.out0 = p.a1; g.out1 = p.a2; g.out2 = p.a3;
      g.ldo0 = dq; g.ldo1 = dkv; g.ldo2 = dkv;
      g.ntasks = dq + 2 * dkv;
      return PT_GEMV;
    }
    if (i == 1) return PT_ATTN_GQA;
    if (i == 2) return PT_MERGE;
    plain_input(g, p.att, dq, dq);
    g.kind = G_RESID;
    g.W0 = ly->wo;
    g.out0 = p.x;
    g.ldo0 = p.H;
    g.ntasks = p.H;
    return PT_GEMV;
  }
  if (kind == kMla) {
    const int lat = p.kvl + p.rd, qd = p.nd + p.rd;
    switch (i) {
      case 0:
        norm_input(g, p.x, p.H, p.H, ly->attn_norm);
        g.kind = G_STACK;
        g.W0 = ly->w_dq; g.W1 = ly->w_dkv;
        g.n0 = p.ql; g.n1 = lat;
        g.out0 = p.a1; g.out1 = p.a2;
        g.ldo0 = p.ql; g.ldo1 = lat;
        g.ntasks = p.ql + lat;
        return PT_GEMV;
      case 1:
        norm_input(g, p.a1, p.ql, p.ql, ly->q_norm);
        g.kind = G_STACK;
        g.W0 = ly->w_uq;
        g.n0 = p.nh * qd;
        g.out0 = p.a3;
        g.ldo0 = p.nh * qd;
        g.ntasks = p.nh * qd;
        return PT_GEMV;
      case 2:  // absorbed query: rows (h, j) of W_uk^T over each head's nope query
        g.stage = S_NOPE;
        g.src = p.a3;
        g.nh = p.nh; g.nd = p.nd; g.qd = qd;
        g.K = p.nd;
        g.Wst = p.nh * p.nd;
        g.kind = G_OFF;
        g.W0 = ly->w_ukT;
        g.rph = p.kvl;
        g.seg = p.nd;
        g.out0 = p.a4;
        g.ldo0 = p.nh * p.kvl;
        g.ntasks = p.nh * p.kvl;
        return PT_GEMV;
      case 3:
        return PT_ATTN_MLA;
      case 4:
        return PT_MERGE;
      case 5:  // o_h = W_uv,h u_h
        plain_input(g, p.att, p.nh * p.kvl, p.kvl);
        g.Wst = p.nh * p.kvl;
        g.kind = G_OFF;
        g.W0 = ly->w_uv;
        g.rph = p.vd;
        g.seg = p.kvl;
        g.out0 = p.o2;
        g.ldo0 = p.nh * p.vd;
        g.ntasks = p.nh * p.vd;
        return PT_GEMV;
      default:
        plain_input(g, p.o2, p.nh * p.vd, p.nh * p.vd);
        g.kind = G_RESID;
        g.W0 = ly->wo;
        g.out0 = p.x;
        g.ldo0 = p.H;
        g.ntasks = p.H;
        return PT_GEMV;
    }
  }
  // gated delta rule
  const int dq = p.nh * p.dk, dvv = p.nh * p.dv;
  if (i == 0) {
    norm_input(g, p.x, p.H, p.H, ly->attn_norm);
    g.kind = G_STACK;
    g.W0 = ly->kwq; g.W1 = ly->kwk; g.W2 = ly->kwv;
    g.n0 = dq; g.n1 = dq;
    g.out0 = p.a1; g.out1 = p.a2; g.out2 = p.a3;
    g.ldo0 = dq; g.ldo1 = dq; g.ldo2 = dvv;
    g.ntasks = 2 * dq + dvv;
    return PT_GEMV;
  }
  if (i == 1) return PT_KDA;
  plain_input(g, p.att, dvv, dvv);
  g.kind = G_RESID;
  g.W0 = ly->wo;
  g.out0 = p.x;
  g.ldo0 = p.H;
  g.ntasks = p.H;
  return PT_GEMV;
}

// Uniform values read from LDS land in vector registers; move the descriptor into scalar ones.
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float rflf(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
template <class T>
__device__ __forceinline__ T* rflp(T* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = (uint32_t)rfl((int)(uint32_t)u), hi = (uint32_t)rfl((int)(uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void scalarize(Gemv& g) {
  g.kind = rfl(g.kind); g.stage = rfl(g.stage); g.ntasks = rfl(g.ntasks); g.K = rfl(g.K); g.Wst = rfl(g.Wst);
  g.pairs = rfl(g.pairs); g.M = rfl(g.M); g.src = rflp(g.src); g.ld = rfl(g.ld); g.gain = rflp(g.gain);
  g.nh = rfl(g.nh); g.nd = rfl(g.nd); g.qd = rfl(g.qd); g.eps = rflf(g.eps);
  g.W0 = rflp(g.W0); g.W1 = rflp(g.W1); g.W2 = rflp(g.W2); g.n0 = rfl(g.n0); g.n1 = rfl(g.n1);
  g.out0 = rflp(g.out0); g.out1 = rflp(g.out1); g.out2 = rflp(g.out2);
  g.ldo0 = rfl(g.ldo0); g.ldo1 = rfl(g.ldo1); g.ldo2 = rfl(g.ldo2); g.rph = rfl(g.rph); g.seg = rfl(g.seg);
  g.E = rfl(g.E); g.SF = rfl(g.SF); g.F = rfl(g.F); g.Wg = rflp(g.Wg); g.Wu = rflp(g.Wu);
  g.rlog = rflp(g.rlog); g.sact = rflp(g.sact); g.eact = rflp(g.eact);
}

#define MK_SYNC()                                   \
  do {                                              \
    if (!grid_sync(p, gen, &sm.abort)) return;      \
  } while (0)

template <int MM>
__global__ void __launch_bounds__(kThreads, 1) mk_decode_kernel(Params pk) {
  __shared__ Smem sm;
  // the parameters live in LDS: read where needed instead of pinning ~100 scalar registers
  __shared__ Params sp;
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&pk);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&sp);
    for (int i = threadIdx.x; i < (int)(sizeof(Params) / 4); i += kThreads) dst[i] = src[i];
    __syncthreads();
  }
  const Params& p = sp;
  uint32_t gen = 0;
  const int M = p.M, H = p.H;
  const int rpairs = ((p.kvl > 0) ? p.rd : p.hd) / 2;

  // ---- embedding rows and the RoPE table of this step's positions ----
  {
    const int n = M * H;
    for (int e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) {
      const int m = e / H, i = e - m * H;
      int tok = gp(p.tokens)[m];
      if (tok < 0 || tok >= p.V) {
        if (i == 0) {
          stc_u32(p.status + 0, (uint32_t)(-MK_E_DEVICE));
          stc_u32(p.status + 3, (uint32_t)m + 1);
        }
        tok = 0;
      }
      stc(p.x + e, bf2f(gp(p.embed)[(size_t)tok * H + i]));
    }
    // every workgroup computes the table itself (no cross-workgroup dependency)
    for (int e = threadIdx.x; e < p.T * rpairs; e += kThreads) {
      const int t = e / rpairs, j = e - t * rpairs;
      const double inv_freq = pow((double)p.rope_theta, -2.0 * j / (2 * rpairs));
      const double a = (double)(p.kv_len + t) * inv_freq;
      sm.rope[(t * kMaxRopePairs + j) * 2] = (float)cos(a);
      sm.rope[(t * kMaxRopePairs + j) * 2 + 1] = (float)sin(a);
    }
    wait_vm();
  }

  for (int l = 0; l <= p.L; ++l) {
    const int nph = (l == p.L) ? 1 : attn_phases(gp(p.layers + l)->kind) + 3;
    for (int i = 0; i < nph; ++i) {
      Gemv g{};
      RowBuf b0, b1;  // per phase: dead outside GEMV phases
      const int type = rfl(describe(p, l, i, g));
      scalarize(g);
      const int npre = (type == PT_GEMV) ? gemv_preload(g, b0, b1) : 0;
      MK_SYNC();
      // sub-phase stamps of this phase go to the record of the barrier that preceded it
      uint64_t* trec = p.trace ? p.trace + ((size_t)(gen - 1) * gridDim.x + blockIdx.x) * 4 : nullptr;
      switch (type) {
        case PT_GEMV:
          gemv_phase<MM>(g, sm.buf, sm.inv, sm.red, b0, b1, npre, trec);
          break;
        case PT_ATTN_GQA:
          gqa_attn_phase(p, p.layers[l], sm.buf, sm.rope);
          break;
        case PT_ATTN_MLA:
          mla_attn_phase(p, p.layers[l], sm.buf, sm.misc, sm.rope);
          break;
        case PT_MERGE:
          merge_phase(p, p.nh, p.kvl > 0 ? p.kvl : p.hd, p.att, sm.buf);
          break;
        case PT_KDA:
          kda_phase(p, p.layers[l]);
          break;
        case PT_EXPERT:
          compute_route(p, l, &sm.route, sm.rsel, sm.rw, sm.buf);
          g.rt = &sm.route;
          g.ntasks = rfl(sm.route.nu * p.F);
          gemv_phase<MM>(g, sm.buf, sm.inv, sm.red, b0, b1, 0, trec);
          break;
        default:
          moe_down_phase(p, p.layers[l], &sm.route, sm.buf);
          break;
      }
      wait_vm();
    }
  }
  if (p.trace) {
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t* tr = p.trace + ((size_t)gen * gridDim.x + blockIdx.x) * 4;
      gp(tr)[0] = gp(tr)[1] = gp(tr)[2] = gp(tr)[3] = wall_clock64();
    }
  }
}

// W_uk [h][nope][kv_lora] -> W_ukT [h][kv_lora][nope]
__global__ void transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl) {
  const size_t n = (size_t)nh * nd * kvl;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t h = e / ((size_t)nd * kvl), r = e - h * nd * kvl, i = r / kvl, j = r - i * kvl;
    gp(dst)[(h * kvl + j) * nd + i] = gp(src)[e];
  }
}

}  // namespace

namespace mk {

size_t kernel_lds_bytes() { return sizeof(Smem); }
int max_grid() { return kMaxGrid; }

hipError_t launch_decode(const Params& p, int nblocks, hipStream_t stream) {
  const int mm = p.M <= 1 ? 1 : p.M <= 2 ? 2 : p.M <= 4 ? 4 : p.M <= 8 ? 8 : 16;
#ifdef MK_ONLY_MM1
  if (mm != 1) return hipErrorNotSupported;
  hipLaunchKernelGGL(mk_decode_kernel<1>, dim3(nblocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
#endif
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
#ifdef MK_ONLY_MM1
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk_decode_kernel<1>, kThreads, 0);
#endif
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk_decode_kernel<16>, kThreads, 0);
}

}  // namespace mk
