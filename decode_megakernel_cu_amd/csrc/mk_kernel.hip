// mk_kernel.hip -- the persistent decode-step megakernel for gfx950.
//
// One launch runs a whole decode step: embedding, every layer's attention block (GQA, MLA over
// a compressed latent cache, or the gated delta rule) and MoE block, the final norm and the
// LM head (the whole decode step as one kernel: "tpu-megakernels README", FAQ). The grid is one workgroup per CU; dependent phases are separated by a
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
// Latency. Under full weight streaming every dependent round trip to memory costs about a
// microsecond, so activations are moved with 16-byte agent-scope buffer loads issued in batches
// (up to eight per lane in flight before the first is consumed), never one load per loop trip.
//
// Prefetch. The weights of a phase do not depend on activations, so as soon as the workgroup has
// arrived at the barrier before a GEMV phase, every wave (the polling one included) issues the
// loads of its first rows of that phase, and only then waits (the next layer's weights already in
// flight while the current one computes: video description "700 tok/s on a 2.8 Trillion Model: The
// 92-Layer TPU Megakernel", timestamp "The Choreography: Layer n+1 Loads While Layer n Computes");
// the barrier wait and the input staging then overlap the HBM latency.
//
// Nothing uses float atomics: every output element is owned by exactly one lane, so results are
// bitwise reproducible from run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mk_internal.h"

using namespace mk;

// Device tracing (mk_set_trace): per-phase wall-clock stamps. Compiled in only with MK_DEVICE_TRACE
// (the library libmk_trace.so): even when switched off at run time, the stamp code's checks and the
// pointer they test cost about 2.4% of the K3-scale share's batch-1 step.
#ifdef MK_DEVICE_TRACE
constexpr bool kTrace = true;
#else
constexpr bool kTrace = false;
#endif

// Pointers into device memory are marked global so that loads and stores compile to global_*
// instructions: flat ones would also count against the LDS counter, and the barrier's LDS wait
// would then wait for prefetched weights.
#define GLOBAL __attribute__((address_space(1)))

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

template <class T>
__device__ __forceinline__ GLOBAL T* gp(T* p) {
  return (GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ const GLOBAL T* gp(const T* p) {
  return (const GLOBAL T*)p;
}

constexpr int kPollWave = kWaves - 1;
constexpr int kMaxGrid = 256;  // workgroups the barrier polls (4 flags per lane)
constexpr int kQSlots = 5;     // MLA: 16-byte query loads per lane in one batch
constexpr int kCSlots = 5;     // MLA: 16-byte cache loads per lane in one batch
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

// bf16 vectors for the matrix cores
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) { return as_bf16x8(*reinterpret_cast<const u32x4*>(p)); }
// two floats as bf16 high parts (packed) and the bf16 of what the high parts leave (low parts):
// x = hi + lo to about 16 significant bits (hardware round-to-nearest-even conversions)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = {(__bf16)x0, (__bf16)x1};
  hi = __builtin_bit_cast(uint32_t, h);
  const bf16x2 l = {(__bf16)(x0 - __uint_as_float(hi << 16)), (__bf16)(x1 - __uint_as_float(hi & 0xFFFF0000u))};
  lo = __builtin_bit_cast(uint32_t, l);
}

// Weights and cache rows are read once per step: non-temporal loads keep them from evicting the
// kernel's code and the activations from L2.
__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// coherent (device-scope) accesses for activations shared between workgroups
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load((GLOBAL float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// 16-byte coherent accesses through a buffer resource over the workspace. The cache policy is
// sc1, the same bits an agent-scope relaxed atomic access carries; offsets are in bytes.
constexpr int kCoherent = 16;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workspace view: activations addressed by byte offsets from the workspace base.
struct Ws {
  Rsrc r;
  const char* base;
  __device__ __forceinline__ uint32_t off(const float* p) const { return (uint32_t)((const char*)p - base); }
  __device__ __forceinline__ f32x4 ld4(const float* p) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off(p), 0, kCoherent);
    return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
  }
  __device__ __forceinline__ float ld1(const float* p) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off(p), 0, kCoherent));
  }
  __device__ __forceinline__ void st4(float* p, f32x4 v) const {
    const u32x4 u{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, off(p), 0, kCoherent);
  }
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// execution barrier of the workgroup that does not wait for outstanding global loads
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reductions over aligned groups of `width` lanes (a power of two up to 64); every lane of a group
// receives the result. Lane pairs are combined by data-parallel moves inside rows of 16 (swap
// neighbours, swap pairs, mirror half-rows, mirror rows), a swizzle that swaps halves of 32 lanes,
// and, for the whole wave, the sum of lanes 0 and 32 read as scalars: one instruction per step where
// a chain of LDS permutes would wait on each. The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {  // lane l's value, wave-uniform
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float swap16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float wave_sum(float v, int width) {
  if (width >= 2) v += dpp_mov<0xB1>(0.f, v);   // lanes 2i <-> 2i+1
  if (width >= 4) v += dpp_mov<0x4E>(0.f, v);   // pairs of a quad
  if (width >= 8) v += dpp_mov<0x141>(0.f, v);  // mirror within 8 lanes
  if (width >= 16) v += dpp_mov<0x140>(0.f, v); // mirror within 16 lanes
  if (width >= 32) v += swap16(v);
  if (width >= 64) v = lane_f(v, 0) + lane_f(v, 32);
  return v;
}
__device__ __forceinline__ float wave_max(float v, int width) {
  if (width >= 2) v = fmaxf(v, dpp_mov<0xB1>(v, v));
  if (width >= 4) v = fmaxf(v, dpp_mov<0x4E>(v, v));
  if (width >= 8) v = fmaxf(v, dpp_mov<0x141>(v, v));
  if (width >= 16) v = fmaxf(v, dpp_mov<0x140>(v, v));
  if (width >= 32) v = fmaxf(v, swap16(v));
  if (width >= 64) v = fmaxf(lane_f(v, 0), lane_f(v, 32));
  return v;
}


__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// Uniform values read from LDS land in vector registers; these move them into scalar ones.
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The thread index, opaque to the optimiser at each use: values derived from it are then computed
// where they are needed instead of being hoisted to the kernel's entry and kept live (spilled to
// scratch) across every phase of the step.
__device__ __forceinline__ int tid_x() {
  int t = (int)__builtin_amdgcn_workitem_id_x();
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int lane_id() { return tid_x() & 63; }
__device__ __forceinline__ int wave_id() { return rfl(tid_x() >> 6); }
__device__ __forceinline__ float rflf(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
template <class T>
__device__ __forceinline__ T* rflp(T* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = (uint32_t)rfl((int)(uint32_t)u), hi = (uint32_t)rfl((int)(uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

typedef __attribute__((address_space(3))) void* LdsPtr;
// Trace stamps are written to LDS during a phase (a store to memory would count against the
// writing wave's vector-memory counter, and that wave's next wait for its weight loads would then
// also wait for the store to be acknowledged) and copied out by the polling wave at the next barrier.
typedef __attribute__((address_space(3))) uint64_t LdsU64;

// Direct memory-to-LDS copies (buffer_load ... lds): no registers hold the data, so nothing forces
// a wait on earlier loads (prefetched weights) before the copies are issued. Rows r < R of U
// 16-byte units are read at byte offsets off(r, c) of the buffer r_ and land at
// dst + r * DS + 4c (floats); a wave instruction moves up to 64 units of one row (lane l writes
// the block's base + 16 l). Nothing waits here: the caller waits for vmcnt and synchronises.
template <int AUX, class Off>
__device__ __forceinline__ void dma_rows(Rsrc r_, float* dst, int R, int U, int DS, Off off) {
  const int bpr = (U + 63) >> 6, nb = R * bpr, lane = lane_id();
  for (int b = wave_id(); b < nb; b += kWaves) {
    const int r = b / bpr, c0 = (b - r * bpr) << 6, c = c0 + lane;
    if (c < U) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (LdsPtr)(dst + r * DS + 4 * c0), 16, off(r, c), 0, 0, AUX);
  }
}
// the same with row r landing at dst + at(r) (floats)
template <int AUX, class At, class Off>
__device__ __forceinline__ void dma_rows_at(Rsrc r_, float* dst, int R, int U, At at, Off off) {
  const int bpr = (U + 63) >> 6, nb = R * bpr, lane = lane_id();
  for (int b = wave_id(); b < nb; b += kWaves) {
    const int r = b / bpr, c0 = (b - r * bpr) << 6, c = c0 + lane;
    if (c < U) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (LdsPtr)(dst + at(r) + 4 * c0), 16, off(r, c), 0, 0, AUX);
  }
}
// the same with 4-byte units (lane l writes the block's base + 4 l)
template <int AUX, class Off>
__device__ __forceinline__ void dma_rows4(Rsrc r_, float* dst, int R, int U, int DS, Off off) {
  const int bpr = (U + 63) >> 6, nb = R * bpr, lane = lane_id();
  for (int b = wave_id(); b < nb; b += kWaves) {
    const int r = b / bpr, c0 = (b - r * bpr) << 6, c = c0 + lane;
    if (c < U) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, (LdsPtr)(dst + r * DS + c0), 4, off(r, c), 0, 0, AUX);
  }
}

// Copy n 16-byte units of coherent workspace data into LDS, all threads: unit i is read from
// src(i) and written to dst(i). NS loads per lane are in flight before the first is consumed.
template <int NS, class Src, class Dst>
__device__ __forceinline__ void copy_units(const Ws& ws, int n, Src src, Dst dst) {
  for (int b = 0; b < n; b += NS * kThreads) {
    f32x4 v[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (b + u * kThreads < n) v[u] = ws.ld4(src(min(b + u * kThreads + tid_x(), n - 1)));
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int i = b + u * kThreads + tid_x();
      if (b + u * kThreads < n && i < n) *reinterpret_cast<f32x4*>(dst(i)) = v[u];
    }
  }
}

// ----------------------------------------------------------------------------------------------
// grid barrier, in two halves so that a workgroup prepares its next phase while it waits
// arrive: every wave has completed its stores (wait_vm) before calling; the polling wave publishes
//   the workgroup's flag.
// wait: the polling wave polls all flags with independent loads (four per lane) until every
//   workgroup has arrived, or the abort flag or the watchdog ends the step.
// ----------------------------------------------------------------------------------------------
// stamps: [2][kTraceStamps] in LDS, record r in row r % 2 (the row of the previous record is copied
// to memory here: every wave has finished the phase that record covers)
__device__ __forceinline__ void barrier_arrive(const Params& p, uint32_t& gen, LdsU64* stamps) {
  gen += 1;
  wg_barrier();
  if (wave_id() == kPollWave) {
    const int lane = lane_id();
    if (kTrace && p.trace) {  // copy out the previous record and clear its row for the record after this one
      if (lane < kTraceStamps) {
        LdsU64* prev = stamps + (gen & 1) * kTraceStamps;
        if (gen >= 2) gp(p.trace)[((size_t)(gen - 2) * gridDim.x + blockIdx.x) * kTraceStamps + lane] = prev[lane];
        prev[lane] = 0;
      }
      if (lane == 0) stamps[((gen - 1) & 1) * kTraceStamps] = wall_clock64();
    }
    if (lane == 0) stc_u32(p.flags + blockIdx.x, p.epoch + gen);
  }
}

// The polling wave's half of the wait: poll until every workgroup has arrived (or abort).
__device__ __forceinline__ void barrier_poll(const Params& p, uint32_t gen, int* s_abort, LdsU64* stamps) {
  const uint32_t target = p.epoch + gen;
  const int lane = lane_id();
  LdsU64* tr = kTrace && p.trace ? stamps + ((gen - 1) & 1) * kTraceStamps : nullptr;
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
    if (tr) tr[1] = wall_clock64();
  }
}

// Every wave's half: the workgroup leaves together once the polling wave is done.
__device__ __forceinline__ bool barrier_finish(int* s_abort) {
  wg_barrier();
  return *s_abort == 0;
}

// ----------------------------------------------------------------------------------------------
// GEMV executor (one copy in the kernel, driven by a per-phase descriptor)
//
// A phase is a set of tasks (output rows); a task owns one or more weight rows (two for SwiGLU
// gate/up pairs, one per routed expert plus the shared expert for the down projection), each
// dotted with some of the staged input rows. The task space is split into contiguous ranges per
// workgroup; within a workgroup lane groups of LPR lanes take tasks. Each lane group streams its
// rows through two register buffers -- element e+2 is requested while element e+1 is computed --
// so a block of loads is always in flight; the first two elements of a phase are requested
// before the barrier that precedes it. The staged input is processed in column slabs that fit
// LDS; partial dot products are reduced across the lane group and accumulated in LDS, and the
// epilogue writes each task's outputs.
// ----------------------------------------------------------------------------------------------
enum GemvKind : int {
  G_STACK = 0,  // up to three stacked matrices, store
  G_RESID,      // one matrix, residual add into the output
  G_OFF,        // per-head rows: row t reads the staged input at (t / rph) * seg, store
  G_RS,         // router rows (store logits) then shared-expert gate/up pairs (store SwiGLU)
  G_EXP,        // routed-expert gate/up pairs of the unique experts (store SwiGLU per pair)
  G_DOWN,       // routed and shared down projections, router-weighted, residual add
};
enum StageKind : int { S_NORM = 0, S_PLAIN, S_NOPE, S_DOWN };

struct Route {
  int nu;                     // unique experts
  int uexp[kMaxQueue];        // expert id, ascending
  int ustart[kMaxQueue + 1];  // pair range per unique expert
  int ptok[kMaxQueue];        // token of each pair
  float pw[kMaxQueue];        // router weight of each pair
};

// one weight row of a task
struct RowRef {
  const uint16_t* w;  // nullptr: the task has no such row
  int len;            // weights in the row
  int xoff;           // column of the row's input inside a staged row
  int ntok;           // staged rows it is dotted with
  int tbase;          // first of them when tok is nullptr (they are then consecutive)
  const int* tok;     // staged rows, or nullptr
};

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
// Greedy selection key of logit v at vocabulary index i: unsigned order of the keys is the order
// of the logits, ties broken towards the lower index (the float's bits made monotonic, then the
// index complemented in the low word).
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (uint32_t)i);
}
// the value of a key (the inverse of the order-preserving map above)
__device__ __forceinline__ float key_value(unsigned long long k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long k) {
  return ((unsigned long long)dpp_u32<CTRL>((uint32_t)(k >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)k);
}
// the largest key of the wave, in every lane (the same lane moves as wave_max)
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  auto mx = [](unsigned long long a, unsigned long long b) { return a > b ? a : b; };
  k = mx(k, dpp_u64<0xB1>(k));
  k = mx(k, dpp_u64<0x4E>(k));
  k = mx(k, dpp_u64<0x141>(k));
  k = mx(k, dpp_u64<0x140>(k));
  const uint32_t sh = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(k >> 32), 0x401F);
  const uint32_t sl = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)k, 0x401F);
  k = mx(k, ((unsigned long long)sh << 32) | sl);
  const unsigned long long k0 =
      ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(k >> 32), 0) << 32) |
      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 0);
  const unsigned long long k1 =
      ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(k >> 32), 32) << 32) |
      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 32);
  return mx(k0, k1);
}
// by value (a reference-returning min keeps its operands in memory)
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

struct Gemv {
  int kind, stage;
  int ntasks, K, Wst, pairs, M;
  // staging
  const float* src;
  int ld;
  const uint16_t* gain;
  int nh, nd, qd;  // S_NOPE
  float eps;
  const float* src2;  // S_DOWN: src = expert activations [np][F], src2 = shared activations [M][SF]
  int np;
  // rows and outputs
  const uint16_t *W0, *W1, *W2, *Wg, *Wu;
  const uint16_t* safe;  // a valid weight address for lanes without a row
  int n0, n1;
  float *out0, *out1, *out2;
  int ldo0, ldo1, ldo2;
  int rph, seg;    // G_OFF
  int E, SF, F, H;  // G_RS / G_EXP / G_DOWN
  float *rlog, *sact, *eact;
  const Route* rt;
  unsigned long long* hmax;  // LM head of a greedy step: per-row argmax keys of the workgroup (LDS)

  __device__ __forceinline__ RowRef row(int t, int which) const {
    RowRef r{nullptr, K, 0, M, 0, nullptr};
    switch (kind) {
      case G_STACK:
        if (t < n0) r.w = W0 + (size_t)t * K;
        else if (t < n0 + n1) r.w = W1 + (size_t)(t - n0) * K;
        else r.w = W2 + (size_t)(t - n0 - n1) * K;
        break;
      case G_RESID:
        r.w = W0 + (size_t)t * K;
        break;
      case G_OFF:
        r.w = W0 + (size_t)t * seg;
        r.len = seg;
        r.xoff = (t / rph) * seg;
        break;
      case G_RS:
        if (t < E) r.w = which ? nullptr : W0 + (size_t)t * K;
        else r.w = (which ? Wu : Wg) + (size_t)(t - E) * K;
        break;
      case G_EXP: {
        if (t >= n0) {  // router fusion: the shared expert's gate/up pair (every token row)
          r.w = (which ? W1 : W0) + (size_t)(t - n0) * K;
          break;
        }
        const int u = t / F, j = t - u * F;
        r.w = (which ? Wu : Wg) + ((size_t)rt->uexp[u] * F + j) * K;
        const int s0 = rt->ustart[u];
        r.ntok = rt->ustart[u + 1] - s0;
        r.tok = rt->ptok + s0;
        break;
      }
      default:  // G_DOWN: row `which` of the unique experts, then the shared expert's row
        if (which < rt->nu) {
          r.w = Wg + ((size_t)rt->uexp[which] * H + t) * F;
          r.len = F;
          const int s0 = rt->ustart[which];
          r.ntok = rt->ustart[which + 1] - s0;
          r.tbase = s0;
        } else {
          r.w = Wu + (size_t)t * SF;
          r.len = SF;
          r.tbase = np;
        }
    }
    return r;
  }

  // a0/a1: the task's accumulators (LDS), res: its residual inputs (LDS, token stride rs)
  __device__ __forceinline__ void epilogue(int t, const float* a0, const float* a1, const float* res, int rs) const {
    switch (kind) {
      case G_STACK: {
        // one store loop per output block: a pointer and stride selected per lane would be kept
        // in a scratch array
        if (t < n0) {
          if (out0)
            for (int k = 0; k < M; ++k) stc(out0 + (size_t)k * ldo0 + t, a0[k]);
        } else if (t < n0 + n1) {
          for (int k = 0; k < M; ++k) stc(out1 + (size_t)k * ldo1 + (t - n0), a0[k]);
        } else {
          for (int k = 0; k < M; ++k) stc(out2 + (size_t)k * ldo2 + (t - n0 - n1), a0[k]);
        }
        if (hmax)
          for (int k = 0; k < M; ++k)
            __hip_atomic_fetch_max(hmax + k, argmax_key(a0[k], t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      case G_RESID:
      case G_DOWN:
        for (int k = 0; k < M; ++k) stc(out0 + (size_t)k * ldo0 + t, res[k * rs] + a0[k]);
        break;
      case G_OFF:
        for (int k = 0; k < M; ++k) stc(out0 + (size_t)k * ldo0 + t, a0[k]);
        break;
      case G_RS:
        if (t < E) {
          for (int k = 0; k < M; ++k) stc(rlog + (size_t)k * E + t, a0[k]);
        } else {
          for (int k = 0; k < M; ++k) stc(sact + (size_t)k * SF + (t - E), silu(a0[k]) * a1[k]);
        }
        break;
      default: {  // G_EXP
        if (t >= n0) {
          for (int k = 0; k < M; ++k) stc(sact + (size_t)k * SF + (t - n0), silu(a0[k]) * a1[k]);
          break;
        }
        const int u = t / F, j = t - u * F;
        const int s0 = rt->ustart[u], n = rt->ustart[u + 1] - s0;
        for (int k = 0; k < n; ++k) stc(eact + (size_t)(s0 + k) * F + j, silu(a0[k]) * a1[k]);
      }
    }
  }

  // Issue the staging of input columns [k0, k0+ks) into dst (LDS) as rows of ks floats at a row
  // stride of DS floats, and of the slab's norm gain (bf16) into gl. Direct memory-to-LDS copies;
  // the caller waits.
  __device__ __forceinline__ void stage_issue(const Ws& ws, float* dst, uint16_t* gl, int k0, int ks, int DS) const {
    if (stage == S_DOWN) {  // expert activation rows, then shared activation rows
      const int ue = max(0, min(F - k0, ks)) >> 2, us = max(0, min(SF - k0, ks)) >> 2;
      dma_rows<kCoherent>(ws.r, dst, np, ue, DS, [&](int r, int c) { return ws.off(src + (size_t)r * F + k0 + 4 * c); });
      dma_rows<kCoherent>(ws.r, dst + np * DS, M, us, DS,
               [&](int r, int c) { return ws.off(src2 + (size_t)r * SF + k0 + 4 * c); });
      return;
    }
    if (stage == S_NOPE) {  // the nope parts of the window's heads, from rows [nh][qd]
      const int h0 = k0 / nd, nhw = ks / nd;
      dma_rows_at<kCoherent>(
          ws.r, dst, M * nhw, nd >> 2,
          [&](int r) {
            const int m = r / nhw;
            return m * DS + (r - m * nhw) * nd;
          },
          [&](int r, int c) {
            const int m = r / nhw;
            return ws.off(src + (size_t)m * nh * qd + (h0 + r - m * nhw) * qd + 4 * c);
          });
      return;
    }
    dma_rows<kCoherent>(ws.r, dst, M, ks >> 2, DS, [&](int r, int c) { return ws.off(src + (size_t)r * ld + k0 + 4 * c); });
    if (stage == S_NORM) {  // the gain of the slab, 8 bf16 per unit
      const Rsrc gr = make_rsrc(gain + k0, (uint32_t)ks * 2);
      dma_rows<0>(gr, reinterpret_cast<float*>(gl), 1, ks >> 3, 0, [&](int, int c) { return (uint32_t)c * 16; });
    }
  }

  // RMSNorm is applied as inv[m] * (W (g . x[m])): staging scales the columns by the gain, the
  // epilogue by the row's factor inv[m] = 1/sqrt(mean(x[m]^2) + eps). The sums of squares come from
  // the raw staged columns, one partial per wave in red[m][wave] (summed over the slabs).
  __device__ __forceinline__ float rms_inv(const float* red, int m) const {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[m * kWaves + w];
    return 1.0f / sqrtf(t / (float)K + eps);
  }
  template <int MM>
  __device__ __forceinline__ void add_sumsq(float (&ss)[MM], float* red, bool first) const {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      if (m < M) {
        const float s = wave_sum(ss[m], 64);
        if (lane_id() == 0) red[m * kWaves + wave_id()] = first ? s : red[m * kWaves + wave_id()] + s;
      }
    }
  }
  // the token whose input row slot k of task t dotted (G_EXP: its expert's pairs in order), and the
  // number of slots
  __device__ __forceinline__ int token_of(int t, int k) const {
    if (kind != G_EXP || t >= n0) return k;
    const int s0 = rt->ustart[t / F];
    return rt->ptok[s0 + k];
  }
  __device__ __forceinline__ int slots_of(int t) const {
    if (kind != G_EXP || t >= n0) return M;
    const int u = t / F;
    return rt->ustart[u + 1] - rt->ustart[u];
  }

  // After the staged data has landed (waited and synchronised): S_NORM columns are scaled by the
  // gain and the rows' sums of squares accumulated (first: the first slab of the phase).
  template <int MM>
  __device__ __forceinline__ void stage_finish(float* dst, const uint16_t* gl, int ks, int DS, bool first,
                                               float* red) const {
    if (stage != S_NORM) return;
    float ss[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) ss[m] = 0.f;
    for (int o = tid_x(); o < (ks >> 3); o += kThreads) {
      float gf[8];
      unpack8(*reinterpret_cast<const uint4*>(gl + 8 * o), gf);
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        if (m < M) {
          f32x4* d = reinterpret_cast<f32x4*>(dst + m * DS + 8 * o);
          f32x4 a = d[0], b = d[1];
          ss[m] += dot4(a, a) + dot4(b, b);
          a.x *= gf[0]; a.y *= gf[1]; a.z *= gf[2]; a.w *= gf[3];
          b.x *= gf[4]; b.y *= gf[5]; b.z *= gf[6]; b.w *= gf[7];
          d[0] = a;
          d[1] = b;
        }
      }
    }
    add_sumsq<MM>(ss, red, first);
  }
};

constexpr int kNC = 8;  // 16-byte chunks of one weight-row block a lane holds in registers

struct RowBuf {
  uint4 v[kNC];
};

// Issue the loads of this lane's chunks of one block of a weight row: chunks c = c0 + sub + u*LPR
// (u < kNC, c < nch) of w. Every load is issued (out-of-range chunks read `safe`, a valid
// address, and are ignored): branches around individual loads make the compiler wait for each
// load before issuing the next.
__device__ __forceinline__ void load_block(const uint16_t* w, int c0, int nch, int sub, int LPR, const uint16_t* safe,
                                           RowBuf& b) {
  const uint16_t* base = w + (size_t)(c0 + sub) * 8;
#pragma unroll
  for (int u = 0; u < kNC; ++u) {
    const bool ok = c0 + sub + u * LPR < nch;
    b.v[u] = ldw(ok ? base + (size_t)u * LPR * 8 : safe);
  }
}

// d[q] = this lane's partial dot product of the block with the staged input row of q
template <int MM>
__device__ __forceinline__ void dot_block(const RowBuf& b, const float* xin, int ldx, int xoff, const RowRef& r, int c0,
                                          int nch, int sub, int LPR, float (&d)[MM]) {
  int tk[MM];
#pragma unroll
  for (int q = 0; q < MM; ++q) {
    tk[q] = r.tok ? r.tok[q < r.ntok ? q : 0] : r.tbase + q;
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
        if (q < r.ntok) {
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

// Static distribution of a phase's tasks, computed once per phase (before its barrier). Each lane
// group streams elements (slab, task it, row which, block blk) in that order, the element count of
// a slab padded to even so that the two register buffers alternate the same way in every slab.
constexpr int kGemvWaves = kWaves;
static_assert(kGemvWaves == 8 && kNC == 8, "make_plan's width choice shifts by log2(8)");

// vp: lane-group tasks per task (2: the SwiGLU gate and up rows of router/shared and routed-expert
// phases go to different lane groups, so few tasks still keep every wave busy); cp: weight rows a
// lane-group task streams one after the other (the down projection's experts and shared expert)
struct Plan {
  int t0, nloc, wbase, Wst, KS, nslab, lg, LPR, G, sub, grp, iters, nblk, per, nel, nelp, ntot, vp, cp, nv;
  bool one_slab;
  float* acc;  // [nloc][2][MM] task accumulators, at the end of the LDS buffer
  float* res;  // [M][nloc] residual inputs
};

__device__ __forceinline__ int log2ceil(int x) { return x <= 1 ? 0 : 32 - __clz(x - 1); }

template <int MM>
__device__ __forceinline__ Plan make_plan(const Gemv& g, float* smem) {
  Plan q;
  const unsigned nt = (unsigned)g.ntasks, gb = blockIdx.x, gn = gridDim.x;  // nt * gn < 2^32
  q.t0 = (int)(nt * gb / gn);
  const int t1 = (int)(nt * (gb + 1) / gn);
  q.nloc = t1 - q.t0;
  const int in_cap = (kLdsFloats - q.nloc * 3 * MM) & ~7;
  q.acc = smem + in_cap;
  q.res = q.acc + q.nloc * 2 * MM;
  q.wbase = 0;
  q.Wst = g.Wst;
  const bool offs = g.kind == G_OFF;
  if (offs && q.nloc > 0) {  // offset phases stage only the window of columns their tasks read
    q.wbase = (q.t0 / g.rph) * g.seg;
    q.Wst = ((t1 - 1) / g.rph) * g.seg + g.seg - q.wbase;
  }
  q.KS = q.Wst;
  if (!offs) {
    const int rows = g.stage == S_DOWN ? g.np + g.M : g.M;
    // staged rows, then (S_NORM) the slab's gain in bf16: rows * KS + KS / 2 floats
    int cap = ((2 * in_cap) / (2 * rows + (g.stage == S_NORM ? 1 : 0))) & ~7;
    if (cap < 8) cap = 8;
    if (q.KS > cap) q.KS = cap;
  }
  q.nslab = q.KS > 0 ? (q.Wst + q.KS - 1) / q.KS : 0;
  const int nch = (offs ? g.seg : q.KS) >> 3;
  q.vp = (g.kind == G_RS || g.kind == G_EXP) && g.pairs == 2 ? 2 : 1;
  q.cp = q.vp == 2 ? 1 : g.pairs;
  q.nv = q.nloc * q.vp;
  // lanes per row (a power of two): enough that kNC chunks per lane cover the row, few enough that
  // every wave has a task when the workgroup has few
  const int lo = min(6, log2ceil(cdiv(nch, kNC))), hi = max(lo, min(6, log2ceil(nch)));
  const int bal = max(0, 6 - log2ceil(max(1, cdiv(q.nv, kGemvWaves))));
  q.lg = min(max(bal, lo), hi);
  // rows that fill their blocks poorly at this width (a 640-chunk row on 64 lanes: 8 chunks per lane,
  // then 2) keep fewer bytes in flight; narrower lane groups with fewer block rounds per lane
  // group (iterations x blocks per row) stream them with full blocks
  // (every divisor is a power of two: shifts; kGemvWaves = kNC = 8)
  if (nch * 4 < 3 * ((nch + (kNC << q.lg) - 1) >> (3 + q.lg)) * (kNC << q.lg)) {
    auto rounds = [&](int lg) {
      return ((q.nv + (8 << (6 - lg)) - 1) >> (9 - lg)) * ((nch + (8 << lg) - 1) >> (3 + lg));
    };
    int best = q.lg, cost = rounds(q.lg);
    for (int lg = q.lg - 1; lg >= max(0, q.lg - 3); --lg) {
      const int c = rounds(lg);
      if (c < cost) {
        cost = c;
        best = lg;
      }
    }
    q.lg = best;
  }
  q.LPR = 1 << q.lg;
  q.G = 64 >> q.lg;
  const int lane = lane_id();
  q.sub = lane & (q.LPR - 1);
  q.grp = lane >> q.lg;
  q.iters = cdiv(q.nv, kGemvWaves * q.G);
  q.nblk = (nch + (kNC << q.lg) - 1) >> (3 + q.lg);
  q.per = q.cp * q.nblk;
  q.nel = q.iters * q.per;
  q.nelp = q.nel + (q.nel & 1);
  q.ntot = q.nslab * q.nelp;
  q.one_slab = q.KS >= q.Wst;
  return q;
}

// Position in a lane group's element stream (wave-uniform): slab, element of the slab, and the
// element's task iteration, row and block.
struct Cursor {
  int slab, ei, it, which, blk;
};
__device__ __forceinline__ void advance(Cursor& c, const Plan& q, int pairs) {
  if (++c.ei == q.nelp) {
    c.ei = c.it = c.which = c.blk = 0;
    ++c.slab;
  } else if (++c.blk == q.nblk) {
    c.blk = 0;
    if (++c.which == pairs) {
      c.which = 0;
      ++c.it;
    }
  }
}

__device__ __forceinline__ int task_of(const Plan& q, int it) { return (it * kGemvWaves + wave_id()) * q.G + q.grp; }

// Issue the loads of the element at c into b (lanes without a row read a valid dummy address).
__device__ __forceinline__ void load_element(const Gemv& g, const Plan& q, const Cursor& c, RowBuf& b) {
  const int k0 = c.slab * q.KS, ks = min(q.KS, q.Wst - k0);
  const int v = task_of(q, c.it), i = v >> (q.vp - 1), which = q.vp == 2 ? v & 1 : c.which;
  const uint16_t* w = g.safe;
  int nc = 0;
  if (c.slab < q.nslab && c.ei < q.nel && v < q.nv) {
    const RowRef r = g.row(q.t0 + i, which);
    if (r.w) {
      w = r.w + k0;
      nc = max(0, min(r.len - k0, ks)) >> 3;
    }
  }
  load_block(w, c.blk * kNC * q.LPR, nc, q.sub, q.LPR, g.safe, b);
}

// Request the first two elements of this lane group's stream (before the phase's barrier; on the
// polling wave the poll then waits for them, which the barrier's own latency mostly covers).
__device__ __forceinline__ void gemv_preload(const Gemv& g, const Plan& q, RowBuf& b0, RowBuf& b1) {
  Cursor c{0, 0, 0, 0, 0};
  if (q.ntot > 0) load_element(g, q, c, b0);
  advance(c, q, q.cp);
  if (q.ntot > 1) load_element(g, q, c, b1);
}

template <int MM>
__device__ __forceinline__ void reduce_task(const Gemv& g, const Plan& q, int v, bool first, float (&a0)[MM],
                                            float (&a1)[MM]) {
  const bool two = g.kind == G_RS || g.kind == G_EXP;
  if (q.vp == 2) {  // one row of the task: gate (slot 0) or up (slot 1)
    const int i = v >> 1, w = v & 1;
#pragma unroll
    for (int k = 0; k < MM; ++k) a0[k] = wave_sum(w ? a1[k] : a0[k], q.LPR);
    if (v < q.nv && q.sub == 0) {
      float* ac = q.acc + (size_t)i * 2 * MM + w * MM;
#pragma unroll
      for (int k = 0; k < MM; ++k) ac[k] = first ? a0[k] : ac[k] + a0[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < MM; ++k) a0[k] = wave_sum(a0[k], q.LPR);
    if (two) {
#pragma unroll
      for (int k = 0; k < MM; ++k) a1[k] = wave_sum(a1[k], q.LPR);
    }
    if (v < q.nloc && q.sub == 0) {
      float* ac = q.acc + (size_t)v * 2 * MM;
#pragma unroll
      for (int k = 0; k < MM; ++k) {
        ac[k] = first ? a0[k] : ac[k] + a0[k];
        if (two) ac[MM + k] = first ? a1[k] : ac[MM + k] + a1[k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < MM; ++k) a0[k] = a1[k] = 0.f;
}

// Consume stream element eg (at cursor cc, of the slab [k0, k0+ks)) from b, then reuse b for
// element eg + 2 (at cursor pc, possibly of the next slab).
template <int MM>
__device__ __forceinline__ void step_element(const Gemv& g, const Plan& q, int eg, Cursor& cc, Cursor& pc, int k0,
                                             int ks, const float* xin, RowBuf& b, float (&a0)[MM],
                                             float (&a1)[MM]) {
  const int v = task_of(q, cc.it), i = v >> (q.vp - 1), which = q.vp == 2 ? v & 1 : cc.which;
  const bool real = cc.ei < q.nel;
  if (real && v < q.nv) {
    const RowRef r = g.row(q.t0 + i, which);
    if (r.w) {
      const int nc = max(0, min(r.len - k0, ks)) >> 3;
      float d[MM];
      dot_block<MM>(b, xin, ks, r.xoff - q.wbase, r, cc.blk * kNC * q.LPR, nc, q.sub, q.LPR, d);
      if (g.kind == G_DOWN && which < g.rt->nu) {  // each pair into its token, with its router weight
#pragma unroll
        for (int k = 0; k < MM; ++k) {
          if (k < r.ntok) {
            const int s = r.tbase + k, m = g.rt->ptok[s];
            const float v = g.rt->pw[s] * d[k];
#pragma unroll
            for (int mm = 0; mm < MM; ++mm) a0[mm] += (mm == m) ? v : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < MM; ++k) {
          a0[k] += which && g.kind != G_DOWN ? 0.f : d[k];
          a1[k] += which && g.kind != G_DOWN ? d[k] : 0.f;
        }
      }
    }
  }
  if (eg + 2 < q.ntot) load_element(g, q, pc, b);
  const bool task_end = real && cc.which == q.cp - 1 && cc.blk == q.nblk - 1;
  const bool first = cc.slab == 0;
  advance(cc, q, q.cp);
  advance(pc, q, q.cp);
  if (task_end) reduce_task<MM>(g, q, v, first, a0, a1);
}

// The hidden state entering layer l (l == L: the final norm's input). With router fusion the
// attention block's output projection writes the next layer's input into the other buffer (its
// router rows read the whole input of the layer while other workgroups write their outputs).
__device__ __forceinline__ float* xcur(const Params& p, int l) { return p.rfuse && (l & 1) ? p.x2 : p.x; }

// Router fusion: the folded router rows (E rows of width RW = H + K) are split over the workgroups
// of the output projection. With at least twice as many workgroups as rows, row e is cut into
// P = min(8, grid / E) column parts, part q on workgroup e P + q (partial logits summed by the
// router in order of q); otherwise each workgroup takes whole rows [e0, e0 + nr) (P = 1).
struct RPart {
  int e0, nr, q, c0, c1;  // rows, part, columns [c0, c1) (multiples of 4)
};
__device__ __forceinline__ int router_parts(int E) { return imax(1, imin(8, (int)gridDim.x / E)); }
__device__ __forceinline__ RPart router_part(int E, int RW) {
  RPart r{0, 0, 0, 0, RW};
  const int P = router_parts(E), b = blockIdx.x;
  if (P > 1) {
    if (b < E * P) {
      const int U = RW >> 2;
      r.e0 = b / P;
      r.q = b - r.e0 * P;
      r.nr = 1;
      r.c0 = 4 * (U * r.q / P);
      r.c1 = 4 * (U * (r.q + 1) / P);
    }
  } else {
    r.e0 = (int)((unsigned)E * b / gridDim.x);
    r.nr = (int)((unsigned)E * (b + 1) / gridDim.x) - r.e0;
  }
  return r;
}

// Router fusion, the output projection's side work. Before the phase's barrier (the folded rows are
// weights, and the layer's input was complete several barriers ago): copy this workgroup's part of
// the folded router rows and the matching columns of the layer's M input rows into LDS, at xo
// (after the staged input): xo [M][span], then wr [nr][span]. The phase's staging wait covers these
// copies too.
__device__ __forceinline__ void router_side_issue(const Params& p, const LayerDev* ly, int l, const Ws& ws, float* xo,
                                                  int M, int K) {
  const int E = p.E, H = p.H, RW = H + K;
  const RPart rp = router_part(E, RW);
  if (rp.nr == 0) return;
  const int span = rp.c1 - rp.c0, hx = imax(0, imin(rp.c1, H) - rp.c0);
  float* wr = xo + M * span;
  const float* xl = xcur(p, l);
  dma_rows<kCoherent>(ws.r, xo, M, hx >> 2, span,
                      [&](int r, int c) { return ws.off(xl + (size_t)r * H + rp.c0 + 4 * c); });
  const Rsrc rr = make_rsrc(rflp(ly->rwx) + (size_t)rp.e0 * RW, (uint32_t)(rp.nr * RW * 4));
  dma_rows<0>(rr, wr, rp.nr, span >> 2, span, [&](int r, int c) { return (uint32_t)((r * RW + rp.c0 + 4 * c) * 4); });
}

// After the phase's barrier, for the matrix-core executor (which converts its staged input in place
// to bf16 parts): copy the part's columns of the phase's input o (rows of stride ld at src) into
// xo beside the layer input's, so that xo[m] holds the part's columns of [layer input | o].
__device__ __forceinline__ void router_side_issue_o(const Params& p, const Ws& ws, float* xo, int M, int K,
                                                    const float* src, int ld) {
  const int H = p.H;
  const RPart rp = router_part(p.E, H + K);
  if (rp.nr == 0) return;
  const int span = rp.c1 - rp.c0, hx = imax(0, imin(rp.c1, H) - rp.c0), o0 = imax(rp.c0, H) - H;
  dma_rows<kCoherent>(ws.r, xo + hx, M, (span - hx) >> 2, span,
                      [&](int r, int c) { return ws.off(src + (size_t)r * ld + o0 + 4 * c); });
}

// Once the copies and the phase's input have landed: the partial logits of the part, rlog[q][m][e]
// = columns [c0, c1) of wr[e] . [layer input | o] (the router logit before the norm's factor), one
// wave per (row, token). The o columns come from xs (fp32 rows at stride DS), or from xo when
// o_in_xo (router_side_issue_o).
struct RSide {
  float* rlog;
  int E, H, M;
};
__device__ __forceinline__ void router_side_logits(const RSide& rs, const float* xs, int DS, int K, const float* xo,
                                                   bool o_in_xo) {
  const int RW = rs.H + K, lane = lane_id();
  const RPart rp = router_part(rs.E, RW);
  const int span = rp.c1 - rp.c0, hx = o_in_xo ? span : imax(0, imin(rp.c1, rs.H) - rp.c0);
  const float* wr = xo + rs.M * span;
  for (int j = wave_id(); j < rp.nr * rs.M; j += kWaves) {
    const int r = j / rs.M, m = j - r * rs.M;
    const float* w = wr + (size_t)r * span;
    float a = 0.f;
    for (int c = 4 * lane; c < span; c += 256) {
      const float* xv = c < hx ? xo + (size_t)m * span + c : xs + (size_t)m * DS + (rp.c0 + c - rs.H);
      a += dot4(*reinterpret_cast<const f32x4*>(w + c), *reinterpret_cast<const f32x4*>(xv));
    }
    a = wave_sum(a, 64);
    if (lane == 0) stc(rs.rlog + ((size_t)rp.q * rs.M + m) * rs.E + rp.e0 + r, a);
  }
}

// After the phase: the sums of squares of this workgroup's outputs (x + W_o o, the MoE input) per
// token, ssq[workgroup][m] (acc: task accumulators [nloc][2][MM], res: residuals [M][nloc]).
template <int MM>
__device__ __forceinline__ void router_side_ssq(float* ssq, int M, int nloc, const float* acc, const float* res) {
  if (wave_id() != 0) return;
  const int lane = lane_id();
  for (int m = 0; m < M; ++m) {
    float ss = 0.f;
    for (int i = lane; i < nloc; i += 64) {
      const float v = res[m * nloc + i] + acc[(size_t)i * 2 * MM + m];
      ss += v * v;
    }
    ss = wave_sum(ss, 64);
    if (lane == 0) stc(ssq + (size_t)blockIdx.x * M + m, ss);
  }
}

// Returns true when the LDS input buffer ends the phase holding the whole normalised input.
// The first two elements of the stream were requested by gemv_preload.
template <int MM>
__device__ __forceinline__ bool gemv_phase(const Gemv& g, const Plan& q, const Ws& ws, float* smem, float* red,
                                           RowBuf& b0, RowBuf& b1, bool keep_in, LdsU64* trace) {
  float* xin = smem;
  const int tid = tid_x();
  const bool compute = true;
  const bool keep = keep_in && q.one_slab;  // input already staged by the previous phase
  const bool resid = g.kind == G_RESID || g.kind == G_DOWN;
  Cursor cc{0, 0, 0, 0, 0}, pc{0, 0, 0, 0, 0};
  advance(pc, q, q.cp);
  advance(pc, q, q.cp);
  if (trace && tid == 0) trace[4] = wall_clock64();
  for (int sl = 0; sl < q.nslab; ++sl) {
    const int k0 = sl * q.KS, ks = min(q.KS, q.Wst - k0);
    __syncthreads();
    uint16_t* gl = reinterpret_cast<uint16_t*>(xin + (g.stage == S_DOWN ? g.np + g.M : g.M) * ks);
    if (!keep) {
      g.stage_issue(ws, xin, gl, q.wbase + k0, ks, ks);
      if (resid && sl == 0) {  // this workgroup's residual inputs, [token][task]
        const float* rs = g.kind == G_RESID ? g.src2 : g.out0;
        dma_rows4<kCoherent>(ws.r, q.res, g.M, q.nloc, q.nloc,
                  [&](int m, int c) { return ws.off(rs + (size_t)m * g.ldo0 + q.t0 + c); });
      }
      wait_vm();
      __syncthreads();
      g.stage_finish<MM>(xin, gl, ks, ks, sl == 0, red);
    }
    __syncthreads();
    if (trace && sl == 0 && tid == 0) trace[2] = wall_clock64();
    if (compute) {
      float a0[MM], a1[MM];
#pragma unroll
      for (int k = 0; k < MM; ++k) a0[k] = a1[k] = 0.f;
      const int eg0 = sl * q.nelp;
      for (int e = 0; e < q.nelp; e += 2) {
        step_element<MM>(g, q, eg0 + e, cc, pc, k0, ks, xin, b0, a0, a1);
        step_element<MM>(g, q, eg0 + e + 1, cc, pc, k0, ks, xin, b1, a0, a1);
      }
    }
  }
  if (trace && tid == 0) trace[3] = wall_clock64();
  // epilogue: one thread per task (a task's rows may have been reduced by different lane groups)
  __syncthreads();
  for (int i = tid; i < q.nloc; i += kThreads) {
    float* ac = q.acc + (size_t)i * 2 * MM;
    if (g.stage == S_NORM) {  // the RMS factor of each input row
      const int n = g.slots_of(q.t0 + i);
      for (int k = 0; k < n; ++k) {
        const float s = g.rms_inv(red, g.token_of(q.t0 + i, k));
        ac[k] *= s;
        ac[MM + k] *= s;
      }
    }
    g.epilogue(q.t0 + i, ac, ac + MM, q.res + i, q.nloc);
  }
  if (trace && tid == 0) trace[5] = wall_clock64();
  return q.one_slab && g.stage == S_NORM;
}


// ----------------------------------------------------------------------------------------------
// routing (every workgroup, one wave per token): softmax over the token's router logits, top-k
// by logit with ties to the lower expert index, weights renormalised over the chosen experts when
// the model asks; then the unique experts in ascending order, each with its (token, weight)
// pairs in token order
// ----------------------------------------------------------------------------------------------
// fused: router fusion. rlog then holds P partial logits per (token, expert), [P][M][E], without the
// norm's factor 1/rms, and ssq the output projection's per-workgroup sums of squares of the MoE
// input [grid][M]; both are summed here in a fixed order. Otherwise rlog holds finished logits.
__device__ __forceinline__ void compute_route(const Params& p, const Ws& ws, int layer, Route* rt, int* sel,
                                              float* wsel, int* cnt, bool fused) {
  const int M = p.M, E = p.E, K = p.topk, lane = lane_id(), tid = tid_x();
  constexpr int R = kMaxExperts / 64;
  for (int m = wave_id(); m < M; m += kWaves) {
    float r[R];
    if (!fused) {
#pragma unroll
      for (int k = 0; k < R; ++k) r[k] = ws.ld1(p.rlog + (size_t)m * E + min(lane + 64 * k, E - 1));
    } else {
      const int P = router_parts(E), G = gridDim.x;
      float v[8][R], s[kMaxGrid / 64];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int k = 0; k < R; ++k)
          v[q][k] = ws.ld1(p.rlog + ((size_t)min(q, P - 1) * M + m) * E + min(lane + 64 * k, E - 1));
#pragma unroll
      for (int k = 0; k < kMaxGrid / 64; ++k) s[k] = ws.ld1(p.ssq + (size_t)min(lane + 64 * k, G - 1) * M + m);
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxGrid / 64; ++k) ss += lane + 64 * k < G ? s[k] : 0.f;
      ss = wave_sum(ss, 64);
      const float inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        float t = v[0][k];
#pragma unroll
        for (int q = 1; q < 8; ++q) t += q < P ? v[q][k] : 0.f;
        r[k] = t * inv;
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) r[k] = lane + 64 * k < E ? r[k] : -INFINITY;
    float mx = r[0];
#pragma unroll
    for (int k = 1; k < R; ++k) mx = fmaxf(mx, r[k]);
    mx = wave_max(mx, 64);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) sum += (lane + 64 * k < E) ? __expf(r[k] - mx) : 0.f;
    sum = wave_sum(sum, 64);
    unsigned taken = 0;
    float tot = 0.f;
    for (int j = 0; j < K; ++j) {
      // the lane's best untaken expert, then the wave's: keys order by logit, then lower index
      unsigned long long best = 0ull;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int e = lane + 64 * k;
        if (e < E && !((taken >> k) & 1u)) {
          const unsigned long long key = argmax_key(r[k], e);
          best = key > best ? key : best;
        }
      }
      best = wave_max_key(best);
      const int be = (int)(0xFFFFFFFFu - (uint32_t)best);
      const float bv = key_value(best);
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      const float pe = __expf(bv - mx) / sum;
      tot += pe;
      if (lane == 0) {
        sel[m * K + j] = be;
        wsel[m * K + j] = pe;
      }
    }
    if (lane == 0) {
      if (p.norm_topk)
        for (int j = 0; j < K; ++j) wsel[m * K + j] /= tot;
      if (p.route != nullptr && blockIdx.x == 0)
        for (int j = 0; j < K; ++j) gp(p.route)[((size_t)layer * M + m) * K + j] = sel[m * K + j];
    }
  }
  __syncthreads();
  // counting sort of the pairs by expert: counts, then one wave scans them (R experts per lane)
  const int nq = M * K;
  for (int e = tid; e < E; e += kThreads) {
    int c = 0;
    for (int q = 0; q < nq; ++q) c += sel[q] == e;
    cnt[e] = c;
  }
  __syncthreads();
  if (wave_id() == 0) {
    int c[R], s = 0, z = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int e = R * lane + k;
      c[k] = e < E ? cnt[e] : 0;
      s += c[k];
      z += c[k] > 0;
    }
    int si = s, zi = z;  // inclusive scans over lanes
    for (int o = 1; o < 64; o <<= 1) {
      const int sv = __shfl_up(si, o, 64), zv = __shfl_up(zi, o, 64);
      if (lane >= o) {
        si += sv;
        zi += zv;
      }
    }
    int start = si - s, u = zi - z;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int e = R * lane + k;
      if (c[k] > 0) {
        rt->uexp[u] = e;
        rt->ustart[u] = start;
        cnt[e] = start;
        ++u;
      } else if (e < E) {
        cnt[e] = -1;
      }
      start += c[k];
    }
    if (lane == 63) {
      rt->ustart[zi] = si;
      rt->nu = zi;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int k = cnt[e];
    if (k >= 0) {
      for (int q = 0; q < nq; ++q) {
        if (sel[q] == e) {
          rt->ptok[k] = q / K;
          rt->pw[k] = wsel[q];
          ++k;
        }
      }
    }
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------------------------
// Matrix-core GEMV executor (steps with several input rows)
//
// From a few input rows on, the vector executor above spends more issue slots on multiply-adds
// and LDS reads than the weight stream allows; here the products run on the matrix cores.
//
// Column segments. An instance for at most MM input rows uses S = mfma_segments(MM) segments
// (4 up to 4 rows, 2 up to 8, 1 above): a unit is 32 S columns, and the 16 A rows of a 16x16x32
// bf16 multiply are R = 16 / S weight rows x S segments of 32 columns (A row s R + r: weight row r,
// columns 32 s .. +32 of the unit), the 16 B columns are R input rows x the same S segments. Of the
// 16x16 products only the S diagonal blocks where the A row's segment is the B column's are
// used; their sum over segments is the dot over the unit. Lane l loads 16 bytes of weight row
// (l % 16) % R, segment (l % 16) / R, columns 8 (l / 16) .. +8 of the segment: one load
// instruction reads R rows x 64 S contiguous bytes (S = 1: 16 rows x 64 bytes, which streams
// at about 5.1 TB/s here against 6.6 for 1 KB of one row; S = 4: 4 rows x 256 bytes). A
// multiply still consumes 1 KB of weights, so S does not change the multiply count.
//
// The inputs are staged in LDS as fp32 and then rewritten in place, each run of 8 columns as its
// bf16 high parts followed by the bf16 of the remainders (x = hi + lo to about 16 significant
// bits), so two multiplies per unit give the products of the bf16 weights with the fp32 inputs,
// accumulated in fp32.
//
// A tile is one group of R output rows and one of its weight-row kinds (SwiGLU gate or up; for
// the down projection, each routed expert and the shared expert). The tiles' units form one
// sequence, cut into eight contiguous ranges, one per wave; a wave streams its range in elements
// of up to kNC units within one tile through the same two register buffers as the vector executor
// (an element's loads are issued two elements ahead, the first two before the phase's barrier),
// and writes the used blocks of its partial result of each tile (each output group, for the down
// projection) to its own LDS slot. After a slab the slots of each tile are summed in wave order,
// then segment order -- a fixed order, so results do not depend on timing -- into the same
// per-task accumulators the vector executor fills, and the same epilogues write the outputs.
//
// Shapes: every row length and slab width is a multiple of 32 S columns, and per-head rows (G_OFF)
// come in whole groups of 16 inside one head; the host launches this executor only then.
// ----------------------------------------------------------------------------------------------
struct MPlan {
  int t0, nloc, wbase, Wst, KS, DS, nslab, ngrp, nat;
  bool one_slab;
  float* acc;    // [nloc][2][MM] task accumulators
  float* res;    // [M][nloc] residual inputs
  float* piece;  // [nat + kWaves][S][R columns][R rows] partial tiles (the matching-segment blocks), slot = acc tile + wave
};

// A slab's unit counts: per tile (nuk), or for the down projection per routed-expert tile (ne) and
// for the shared-expert tile (ns), pg per group; U over all tiles of the workgroup.
struct MGeo {
  int k0, ks, nuk, ne, ns, pg, U;
};

// (S: column segments per tile; a unit is 32 S columns)
template <int S>
__device__ __forceinline__ MGeo mgeo(const Gemv& g, const MPlan& q, int slab) {
  constexpr int lu = S == 4 ? 7 : S == 2 ? 6 : 5;
  MGeo e;
  e.k0 = slab * q.KS;
  e.ks = imin(q.KS, q.Wst - e.k0);
  if (g.kind == G_DOWN) {
    e.ne = imax(0, imin(g.F - e.k0, e.ks)) >> lu;
    e.ns = g.SF > 0 ? imax(0, imin(g.SF - e.k0, e.ks)) >> lu : 0;
    e.pg = rfl(g.rt->nu) * e.ne + e.ns;
    e.nuk = 0;
    e.U = q.ngrp * e.pg;
  } else {
    int len = e.ks;
    if (g.kind == G_OFF) len = g.seg;
    e.nuk = len >> lu;
    e.ne = e.ns = 0;
    e.pg = g.pairs * e.nuk;
    e.U = q.ngrp * e.pg;
  }
  return e;
}

// (values, not a conditional over fields: a selected field address keeps the struct in memory)
__device__ __forceinline__ int tile_units(const Gemv& g, const MGeo& e, int j) {
  if (g.kind != G_DOWN) return e.nuk;
  int u = e.ns;
  if (j % g.pairs < rfl(g.rt->nu)) u = e.ne;
  return u;
}
// accumulator tile of tile j: the down projection sums all of a group's tiles into one
__device__ __forceinline__ int acc_tile(const Gemv& g, int j) { return g.kind == G_DOWN ? j / g.pairs : j; }

// first unit of wave w's range
__device__ __forceinline__ int wave_start(const MGeo& e, int w) { return (w * e.U) / kWaves; }

template <int MM>
__device__ __forceinline__ MPlan mmake_plan(const Gemv& g, float* smem) {
  constexpr int S = mfma_segments(MM), R = 16 / S;
  MPlan q;
  const unsigned gb = blockIdx.x, gn = gridDim.x;
  const bool offs = g.kind == G_OFF;
  int t1;
  if (offs) {  // whole groups of R rows, so that a group never spans two heads
    const unsigned ng = (unsigned)g.ntasks / R;
    q.t0 = R * (int)(ng * gb / gn);
    t1 = R * (int)(ng * (gb + 1) / gn);
  } else {
    const unsigned nt = (unsigned)g.ntasks;
    q.t0 = (int)(nt * gb / gn);
    t1 = (int)(nt * (gb + 1) / gn);
  }
  q.nloc = t1 - q.t0;
  q.ngrp = (q.nloc + R - 1) / R;
  q.nat = g.kind == G_DOWN ? q.ngrp : q.ngrp * g.pairs;
  const int in_cap = (kLdsFloats - q.nloc * 3 * MM - (q.nat + kWaves) * (256 / S)) & ~7;
  q.acc = smem + in_cap;
  q.res = q.acc + q.nloc * 2 * MM;
  q.piece = q.res + q.nloc * MM;
  q.wbase = 0;
  q.Wst = g.Wst;
  if (offs && q.nloc > 0) {
    q.wbase = (q.t0 / g.rph) * g.seg;
    q.Wst = ((t1 - 1) / g.rph) * g.seg + g.seg - q.wbase;
  }
  const int rows = g.stage == S_DOWN ? g.np + g.M : g.M;
  if (offs) {
    q.KS = q.Wst;
    q.nslab = 1;
  } else {
    // staged rows at a stride of KS + 4 floats, then (S_NORM) the slab's gain in bf16
    int cap = ((2 * (in_cap - 4 * rows)) / (2 * rows + (g.stage == S_NORM ? 1 : 0))) & ~(32 * S - 1);
    if (cap < 32 * S) cap = 32 * S;
    q.nslab = cdiv(q.Wst, cap);
    q.KS = (cdiv(q.Wst, q.nslab) + 32 * S - 1) & ~(32 * S - 1);  // balanced slabs
  }
  if (q.nloc == 0) q.nslab = 0;
  q.DS = q.KS + 4;
  q.one_slab = q.nslab == 1;
  return q;
}

// Position in a wave's element stream (wave-uniform): slab, tile, first unit and unit count of the
// element (n == 0: the padding element that keeps a slab's element count even), units left in the
// wave's range of the slab, and the parity of the elements so far in the slab.
struct MCur {
  int slab, j, us, n, rem, cnt;
};

// (The cursor functions take and return cursors by value: stores to different fields of a
// referenced cursor on different paths would be merged into one store through a selected address,
// and the cursor would then live in scratch memory.)
template <int S>
__device__ __forceinline__ MCur mcur_slab(const Gemv& g, const MPlan& q, int slab) {
  const int w = wave_id();
  MCur c;
  for (; slab < q.nslab; ++slab) {
    const MGeo e = mgeo<S>(g, q, slab);
    const int s = wave_start(e, w), t = wave_start(e, w + 1);
    if (t > s) {
      int j, us;
      if (g.kind == G_DOWN) {
        const int nu = rfl(g.rt->nu), gi = s / e.pg, r = s - gi * e.pg, nue = nu * e.ne;
        const int which = r < nue ? r / e.ne : nu;
        us = r - which * e.ne;
        j = gi * g.pairs + which;
      } else {
        j = s / e.nuk;
        us = s - j * e.nuk;
      }
      c.slab = slab;
      c.j = j;
      c.us = us;
      c.rem = t - s;
      c.cnt = 0;
      c.n = imin(imin(kNC, tile_units(g, e, j) - us), t - s);
      return c;
    }
  }
  c.slab = q.nslab;
  c.j = c.us = c.n = c.rem = c.cnt = 0;
  return c;
}

template <int S>
__device__ __forceinline__ MCur madvance(const Gemv& g, const MPlan& q, const MCur& c0) {
  const int slab = c0.slab, n = c0.n;
  if (slab >= q.nslab) return c0;
  if (n == 0) return mcur_slab<S>(g, q, slab + 1);  // after the padding element
  const int rem = c0.rem - n, cnt = c0.cnt ^ 1;
  if (rem == 0) {
    if (cnt == 0) return mcur_slab<S>(g, q, slab + 1);
    MCur c;  // the padding element keeps the slab's element count even
    c.slab = slab;
    c.j = c0.j;
    c.us = c0.us;
    c.n = 0;
    c.rem = 0;
    c.cnt = 0;
    return c;
  }
  const MGeo e = mgeo<S>(g, q, slab);
  int j = c0.j, us = c0.us + n;
  if (us == tile_units(g, e, j)) {
    us = 0;
    do ++j;
    while (tile_units(g, e, j) == 0);
  }
  MCur c;
  c.slab = slab;
  c.j = j;
  c.us = us;
  c.n = imin(imin(kNC, tile_units(g, e, j) - us), rem);
  c.rem = rem;
  c.cnt = cnt;
  return c;
}

// Issue the loads of element c into b: lane l reads row (l % 16) % R of the tile's group (R = 16 / S
// rows), segment (l % 16) / R, columns 8 (l / 16) .. +8 of the segment, of each unit (rows the
// workgroup does not own, and kinds a row lacks, read a valid dummy address; their results are
// never used).
template <int S>
__device__ __forceinline__ void mload_element(const Gemv& g, const MPlan& q, const MCur& c, RowBuf& b) {
  constexpr int R = 16 / S;
  const int lane = lane_id(), r = lane & (R - 1), sg = (lane & 15) / R, kq = lane >> 4;
  const uint16_t* w = g.safe;
  bool ok = false;
  if (c.slab < q.nslab && c.n > 0) {
    const int gi = c.j / g.pairs, which = c.j - gi * g.pairs, i = gi * R + r;
    if (i < q.nloc) {
      const RowRef rr = g.row(q.t0 + i, which);
      if (rr.w) {
        w = rr.w + c.slab * q.KS + 32 * S * c.us + 32 * sg + 8 * kq;
        ok = true;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kNC; ++u) b.v[u] = ldw(ok && u < c.n ? w + 32 * S * u : g.safe);
}

template <int S>
__device__ __forceinline__ void mgemv_preload(const Gemv& g, const MPlan& q, RowBuf& b0, RowBuf& b1) {
  MCur c = mcur_slab<S>(g, q, 0);
  mload_element<S>(g, q, c, b0);
  c = madvance<S>(g, q, c);
  mload_element<S>(g, q, c, b1);
}

// Consume the element at cc from b (its slab is staged in xs), then reuse b for the element at pc
// (two ahead); a partial tile goes to its slot when the next element belongs to another. B column
// n holds input row n % R at segment n / R of each unit.
template <int S>
__device__ __forceinline__ void mstep(const Gemv& g, const MPlan& q, MCur& cc, MCur& pc, const float* xs, RowBuf& b,
                                      f32x4& dt) {
  constexpr int R = 16 / S;
  const int lane = lane_id(), m = lane & 15, kq = lane >> 4, mt = m & (R - 1), sg = m / R;
  if (cc.n > 0) {
    const int gi = cc.j / g.pairs, which = cc.j - gi * g.pairs;
    int brow = imin(mt, g.M - 1);  // columns past the last input row repeat it; their results are unused
    uint32_t keep = ~0u;
    int col = 32 * S * cc.us + 32 * sg + 8 * kq;
    if (g.kind == G_DOWN) {
      const int nu = rfl(g.rt->nu);
      if (which < nu) {  // this expert's (token, weight) pair of the column's token, if any
        const int s0 = rfl(g.rt->ustart[which]), s1 = rfl(g.rt->ustart[which + 1]);
        bool has = false;
        int ps = 0;
        for (int s = s0; s < s1; ++s) {
          if (g.rt->ptok[s] == mt) {
            ps = s;
            has = true;
          }
        }
        brow = ps;
        keep = has ? ~0u : 0u;
      } else {
        brow += g.np;
      }
    } else if (g.kind == G_OFF) {
      col += ((q.t0 + R * gi) / g.rph) * g.seg - q.wbase;
    }
    const float* xp = xs + brow * q.DS + col;
#pragma unroll
    for (int u = 0; u < kNC; ++u) {
      if (u < cc.n) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(xp + 32 * S * u) & keep;
        const u32x4 l = *reinterpret_cast<const u32x4*>(xp + 32 * S * u + 4) & keep;
        const bf16x8 a = as_bf16x8(u32x4{b.v[u].x, b.v[u].y, b.v[u].z, b.v[u].w});
        dt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(h), dt, 0, 0, 0);
        dt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(l), dt, 0, 0, 0);
      }
    }
  }
  mload_element<S>(g, q, pc, b);
  const MCur old = cc;
  cc = madvance<S>(g, q, cc);
  pc = madvance<S>(g, q, pc);
  if (old.n > 0 && (cc.slab != old.slab || cc.n == 0 || acc_tile(g, cc.j) != acc_tile(g, old.j))) {
    // lane l holds column l % 16, rows 4 (l / 16) .. +4 of the tile; only the blocks where the row's
    // segment is the column's are kept
    if ((4 * kq) / R == sg) {
      f32x4* slot = reinterpret_cast<f32x4*>(q.piece + (size_t)(acc_tile(g, old.j) + wave_id()) * (256 / S) +
                                             (sg * R + mt) * R + ((4 * kq) & (R - 1)));
      *slot = dt;
    }
    dt = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Staged rows to bf16 high/low parts in place, after the gain (S_NORM; the rows' sums of squares
// are accumulated from the raw columns, the RMS factor is applied when the tiles are summed) or
// the router weight of each expert pair row (S_DOWN).
template <int MM>
__device__ __forceinline__ void mconvert(const Gemv& g, float* xs, const uint16_t* gl, int ks, int DS, bool first,
                                         float* red) {
  const int nco = ks >> 3, nr = g.stage == S_DOWN ? g.np + g.M : g.M;
  const bool norm = g.stage == S_NORM;
  float ss[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) ss[m] = 0.f;
  for (int e = tid_x(); e < nr * nco; e += kThreads) {
    const int r = e / nco, o = e - r * nco;
    f32x4* p = reinterpret_cast<f32x4*>(xs + r * DS + 8 * o);
    f32x4 a = p[0], b = p[1];
    if (norm) {
      const float s2 = dot4(a, a) + dot4(b, b);
#pragma unroll
      for (int m = 0; m < MM; ++m) ss[m] += m == r ? s2 : 0.f;
      float gf[8];
      unpack8(*reinterpret_cast<const uint4*>(gl + 8 * o), gf);
      a.x *= gf[0]; a.y *= gf[1]; a.z *= gf[2]; a.w *= gf[3];
      b.x *= gf[4]; b.y *= gf[5]; b.z *= gf[6]; b.w *= gf[7];
    } else if (g.stage == S_DOWN && r < g.np) {
      const float s = g.rt->pw[r];
      a *= s;
      b *= s;
    }
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_bf16(a.x, a.y, h0, l0);
    split_bf16(a.z, a.w, h1, l1);
    split_bf16(b.x, b.y, h2, l2);
    split_bf16(b.z, b.w, h3, l3);
    p[0] = __builtin_bit_cast(f32x4, u32x4{h0, h1, h2, h3});
    p[1] = __builtin_bit_cast(f32x4, u32x4{l0, l1, l2, l3});
  }
  if (norm) g.add_sumsq<MM>(ss, red, first);
}

// Sum each tile's wave slots (in wave order) into the task accumulators; G_EXP keeps, per task,
// the columns of its expert's tokens in pair order.
template <int MM>
__device__ __forceinline__ void mreduce(const Gemv& g, const MPlan& q, const MGeo& e, bool first, bool last,
                                        const float* red) {
  constexpr int S = mfma_segments(MM), R = 16 / S;
  const int na = g.kind == G_DOWN ? 1 : g.pairs;
  const int n = na * MM * q.nloc;
  for (int x = tid_x(); x < n; x += kThreads) {
    const int ak = x / q.nloc, i = x - ak * q.nloc, a = ak / MM, k = ak - a * MM;
    int col = k;
    if (g.kind == G_EXP && q.t0 + i < g.n0) {
      const int u = (q.t0 + i) / g.F, s0 = g.rt->ustart[u];
      if (k >= g.rt->ustart[u + 1] - s0) continue;
      col = g.rt->ptok[s0 + k];
    } else if (k >= g.M) {
      continue;
    }
    const int gi = i / R, r = i & (R - 1);
    const int at = g.kind == G_DOWN ? gi : gi * g.pairs + a;
    int len = e.nuk;
    if (g.kind == G_DOWN) len = e.pg;
    const int u0 = (g.kind == G_DOWN ? gi : at) * len, u1 = u0 + len;
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) {  // the waves whose (non-empty) ranges meet the tile
      const int ws = wave_start(e, w), we = wave_start(e, w + 1);
      if (we > ws && ws < u1 && we > u0) {  // the products of matching segments (A row, B column sg R + .)
#pragma unroll
        for (int sg = 0; sg < S; ++sg) v += q.piece[(size_t)(at + w) * (256 / S) + (sg * R + col) * R + r];
      }
    }
    float* ac = q.acc + (size_t)i * 2 * MM + a * MM + k;
    if (!first) v += *ac;
    if (last && g.stage == S_NORM) v *= g.rms_inv(red, col);
    *ac = v;
  }
}

// Returns true when the LDS input buffer ends the phase holding the whole normalised input (in
// the split bf16 form this executor reads).
template <int MM>
__device__ __forceinline__ bool mgemv_phase(const Gemv& g, const MPlan& q, const Ws& ws, float* smem, float* red,
                                            RowBuf& b0, RowBuf& b1, bool keep_in, LdsU64* trace) {
  float* xs = smem;
  const int tid = tid_x();
  const bool keep = keep_in && q.one_slab;
  const bool resid = g.kind == G_RESID || g.kind == G_DOWN;
  const int rows = g.stage == S_DOWN ? g.np + g.M : g.M;
  constexpr int S = mfma_segments(MM);
  MCur cc = mcur_slab<S>(g, q, 0);
  MCur pc = madvance<S>(g, q, madvance<S>(g, q, cc));
  f32x4 dt = {0.f, 0.f, 0.f, 0.f};
  if (trace && tid == 0) trace[4] = trace[2] = wall_clock64();
  for (int sl = 0; sl < q.nslab; ++sl) {
    const MGeo e = mgeo<S>(g, q, sl);
    __syncthreads();
    uint16_t* gl = reinterpret_cast<uint16_t*>(xs + rows * q.DS);
    if (!keep) {
      g.stage_issue(ws, xs, gl, q.wbase + e.k0, e.ks, q.DS);
      if (resid && sl == 0) {
        const float* rs = g.kind == G_RESID ? g.src2 : g.out0;
        dma_rows4<kCoherent>(ws.r, q.res, g.M, q.nloc, q.nloc,
                             [&](int m, int c) { return ws.off(rs + (size_t)m * g.ldo0 + q.t0 + c); });
      }
      wait_vm();
      __syncthreads();
      mconvert<MM>(g, xs, gl, e.ks, q.DS, sl == 0, red);
    }
    __syncthreads();
    if (trace && sl == 0 && tid == 0) trace[2] = wall_clock64();
    while (cc.slab == sl) {
      mstep<S>(g, q, cc, pc, xs, b0, dt);
      mstep<S>(g, q, cc, pc, xs, b1, dt);
    }
    __syncthreads();
    mreduce<MM>(g, q, e, sl == 0, sl == q.nslab - 1, red);
  }
  if (trace && tid == 0) trace[3] = wall_clock64();
  __syncthreads();
  for (int i = tid; i < q.nloc; i += kThreads) {
    const float* ac = q.acc + (size_t)i * 2 * MM;
    g.epilogue(q.t0 + i, ac, ac + MM, q.res + i, q.nloc);
  }
  if (trace && tid == 0) trace[5] = wall_clock64();
  return q.one_slab && g.stage == S_NORM;
}

// ----------------------------------------------------------------------------------------------
// attention
// ----------------------------------------------------------------------------------------------
// RoPE table of the step, in LDS: table[(t * kMaxRopePairs + j) * 2 + {cos, sin}]
__device__ __forceinline__ void rope_pair(const float* table, int t, int j, float& x0, float& x1) {
  const float c = table[(t * kMaxRopePairs + j) * 2], s = table[(t * kMaxRopePairs + j) * 2 + 1];
  const float a = x0, b = x1;
  x0 = a * c - b * s;
  x1 = b * c + a * s;
}

// GQA split-KV partials (flash decoding). Task (b, g, s): positions [s*C, s*C+C) of sequence b,
// kv head g, every query head of the group and every new token (rows r = t*qg + head in group,
// nr of them, in tiles of 16). The task streams its positions in sub-tiles of kGSub: the cache
// rows of the next sub-tile are in flight in registers while the current one is scored, and
// each row keeps a running maximum and sum of weights (online softmax), so the task writes one
// partial whatever its length. New positions in the chunk are rotated, rounded to bf16, appended
// to the cache and attended from the rounded values.
// Scores and value sums run on the matrix cores (16x16x32 bf16 multiplies): the queries and the
// softmax weights enter as bf16 high and low parts (two multiplies each), the keys and values as
// stored. A value multiply takes 32 positions as its K dimension in the order p = k/8 + 4 (k%8)
// (k the operand index), so that the four lane groups read staged value rows 1 apart; value rows
// are padded to 8 LDS banks apart and key, query and score rows to 4, which keeps every operand
// read free of bank conflicts. The unnormalised value sums stay in registers: tile j of the
// (row tile, 16-column tile) grid belongs to wave j % 8, rescaled as each row's maximum moves.
template <int HD, bool ONE>
__device__ __forceinline__ void gqa_attn_phase(const Params& p, const LayerDev* ly, const Ws& ws, float* smem,
                                               const float* rope, LdsU64* trace) {
  const int d = HD ? HD : p.hd, nq = p.nh, nkv = p.nkv, T = ONE ? 1 : p.T, cap = p.cap, d2 = d / 2, d4 = d / 4, d8 = d / 8;
  const int npos = p.kv_len + T, C = p.chunk, nsplit = p.nsplit, kvl = p.kv_len;
  const int qg = nq / nkv, nr = T * qg, nrt = (nr + 15) >> 4, nrp = 16 * nrt;
  const int nct = d >> 4, nvt = nrt * nct;  // value tiles: row tiles x column tiles
  const int ntask = (ONE ? 1 : p.B) * nkv * nsplit;
  const int tid = tid_x(), lane = lane_id(), wave = wave_id(), ml = lane & 15, mq = lane >> 4;
  const int dk = d + 8;   // bf16 per staged key row and per query row (hi, lo)
  const int dv = d + 16;  // bf16 per staged value row
  const int ss = kGSub + 4;  // floats per score row
  uint16_t* Kb = reinterpret_cast<uint16_t*>(smem);  // [kGSub][dk] bf16 keys
  uint16_t* Vb = Kb + kGSub * dk;                    // [kGSub][dv] bf16 values
  uint16_t* Qh = Vb + kGSub * dv;                    // [nrp][dk] query high parts
  uint16_t* Ql = Qh + nrp * dk;                      // [nrp][dk] query low parts
  float* Qs = reinterpret_cast<float*>(Ql + nrp * dk);  // [nr][d] rotated queries; at the end the value sums [nrp][d]
  float* S = Qs + nrp * d;                           // [nrp][ss] scores, then weights
  float* Mx = S + nrp * ss;                          // [nrp] running maximum
  float* Ls = Mx + nrp;                              // [nrp] running sum of weights
  float* Sc = Ls + nrp;                              // [nrp] rescale of the value sums this sub-tile
  const size_t lstride = (size_t)p.Bmax * nkv * cap * d;
  uint16_t* Kc = rflp(p.kv) + (size_t)rfl(ly->ord) * lstride;
  uint16_t* Vc = rflp(p.kv) + (size_t)p.L * lstride + (size_t)rfl(ly->ord) * lstride;
  const float scale = 1.0f / sqrtf((float)d);
  const int stride = d + kPartPad, U = kGSub * d8;  // U: 16-byte units of K (and of V) per sub-tile
  constexpr int kU = kGSub * 16 / kThreads;         // units per thread (head_dim <= 128)
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, g = (task / nsplit) % nkv, b = task / (nsplit * nkv);
    const int p0 = s * C, p1 = min(npos, p0 + C), pc = min(p1, kvl);  // [p0, pc): cached positions
    const size_t row0 = ((size_t)b * nkv + g) * cap;                     // cache row of position 0
    uint4 kra[kU], vra[kU];  // the rows of the next sub-tile, in flight while one is scored
    auto issue = [&](int q0, uint4(&kr)[kU], uint4(&vr)[kU]) __attribute__((always_inline)) {
      // the cached rows of the sub-tile at q0 (others read row 0)
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = u * kThreads + tid, pl = i / d8, c = i - pl * d8, pos = q0 + pl;
        const size_t off = (row0 + ((i < U && pos < pc) ? pos : 0)) * d + 8 * (i < U ? c : 0);
        kr[u] = ldw(Kc + off);
        vr[u] = ldw(Vc + off);
      }
    };
    __syncthreads();
    issue(p0, kra, vra);
    copy_units<4>(
        ws, nr * d4,
        [&](int i) {
          const int r = i / d4, t = r / qg, hq = g * qg + (r - t * qg);
          return p.a1 + (size_t)(b * T + t) * nq * d + hq * d + 4 * (i - r * d4);
        },
        [&](int i) { return Qs + 4 * i; });
    for (int e = tid; e < nrp; e += kThreads) {
      Mx[e] = -INFINITY;
      Ls[e] = 0.f;
    }
    __syncthreads();
    for (int e = tid; e < nr * d2; e += kThreads) {  // rotate the queries
      const int r = e / d2, j = e - r * d2, t = r / qg;
      float q0 = Qs[r * d + j], q1 = Qs[r * d + j + d2];
      rope_pair(rope, t, j, q0, q1);
      Qs[r * d + j] = q0;
      Qs[r * d + j + d2] = q1;
    }
    __syncthreads();
    for (int e = tid; e < nrp * d2; e += kThreads) {  // queries as bf16 high and low parts (rows past nr: 0)
      const int r = e / d2, j = 2 * (e - r * d2);
      uint32_t hi = 0u, lo = 0u;
      if (r < nr) split_bf16(Qs[r * d + j], Qs[r * d + j + 1], hi, lo);
      *reinterpret_cast<uint32_t*>(Qh + r * dk + j) = hi;
      *reinterpret_cast<uint32_t*>(Ql + r * dk + j) = lo;
    }
    f32x4 u[kGqaTiles];  // value sums of this wave's tiles (rows 4 mq + i, column ml)
#pragma unroll
    for (int k = 0; k < kGqaTiles; ++k) u[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool first = task == (int)blockIdx.x && trace && tid == 0;  // stamps of the first task
    if (first) trace[2] = wall_clock64();
    auto subtile = [&](int q0, uint4(&kr)[kU], uint4(&vr)[kU]) __attribute__((always_inline)) {
      const int ns = min(kGSub, p1 - q0);
      __syncthreads();  // the previous sub-tile is consumed
#pragma unroll
      for (int u = 0; u < kU; ++u) {  // cached rows into LDS
        const int i = u * kThreads + tid, pl = i / d8, c = i - pl * d8;
        if (i < U && q0 + pl < pc) {
          *reinterpret_cast<uint4*>(Kb + pl * dk + 8 * c) = kr[u];
          *reinterpret_cast<uint4*>(Vb + pl * dv + 8 * c) = vr[u];
        }
      }
      if (q0 + kGSub < pc) issue(q0 + kGSub, kr, vr);
      // new positions of the sub-tile: rotate the key, round to bf16, append, stage
      const int n0 = max(q0, kvl), nn = max(0, q0 + ns - n0);
      for (int e = tid; e < nn * d2; e += kThreads) {
        const int r = e / d2, j = e - r * d2, pl = n0 - q0 + r, t = n0 - kvl + r, m = b * T + t;
        const float* kp = p.a2 + (size_t)m * nkv * d + g * d;
        const float* vp = p.a3 + (size_t)m * nkv * d + g * d;
        float k0 = ws.ld1(kp + j), k1 = ws.ld1(kp + j + d2);
        const float v0 = ws.ld1(vp + j), v1 = ws.ld1(vp + j + d2);
        rope_pair(rope, t, j, k0, k1);
        const uint16_t kb0 = f2bf(k0), kb1 = f2bf(k1), vb0 = f2bf(v0), vb1 = f2bf(v1);
        const size_t ci = (row0 + n0 + r) * d;
        gp(Kc)[ci + j] = kb0;
        gp(Kc)[ci + j + d2] = kb1;
        gp(Vc)[ci + j] = vb0;
        gp(Vc)[ci + j + d2] = vb1;
        Kb[pl * dk + j] = kb0;
        Kb[pl * dk + j + d2] = kb1;
        Vb[pl * dv + j] = vb0;
        Vb[pl * dv + j + d2] = vb1;
      }
      __syncthreads();
      // scores: tile (row tile rt, position tile pt) per wave; D rows 4 mq + i, column ml
      for (int jt = wave; jt < nrt * (kGSub / 16); jt += kWaves) {
        const int rt = jt / (kGSub / 16), pt = jt - rt * (kGSub / 16);
        const uint16_t* ah = Qh + (16 * rt + ml) * dk + 8 * mq;
        const uint16_t* al = Ql + (16 * rt + ml) * dk + 8 * mq;
        const uint16_t* bk = Kb + (16 * pt + ml) * dk + 8 * mq;
        f32x4 dd = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < d; kk += 32) {
          const bf16x8 bv = ld_bf16x8(bk + kk);
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(ah + kk), bv, dd, 0, 0, 0);
          dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(al + kk), bv, dd, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) S[(16 * rt + 4 * mq + i) * ss + 16 * pt + ml] = dd[i] * scale;
      }
      __syncthreads();
      if (first && q0 == p0) trace[4] = wall_clock64();
      // online softmax: one wave per row, lane = position; rows past nr and rows that see no
      // position yet get weight 0 and keep their sums (rescale 1)
      for (int r = wave; r < nrp; r += kWaves) {
        const int t = r / qg;
        const float sv = (r < nr && lane < ns && q0 + lane <= kvl + t) ? S[r * ss + lane] : -INFINITY;
        const float mold = Mx[r], mnew = fmaxf(mold, wave_max(sv, 64));
        float w = 0.f, alpha = 1.f;
        if (mnew != -INFINITY) {
          alpha = mold == -INFINITY ? 0.f : __expf(mold - mnew);
          w = sv == -INFINITY ? 0.f : __expf(sv - mnew);
        }
        const float ls = wave_sum(w, 64);
        S[r * ss + lane] = w;
        if (lane == 0) {
          if (mnew != -INFINITY) {
            Mx[r] = mnew;
            Ls[r] = alpha * Ls[r] + ls;
          }
          Sc[r] = alpha;
        }
      }
      __syncthreads();
      if (first && q0 == p0) trace[5] = wall_clock64();
      // value sums: A = weights [16 rows][32 positions] (high, low), B = value rows [32][16 columns]
#pragma unroll
      for (int k = 0; k < kGqaTiles; ++k) {
        const int jt = wave + kWaves * k;
        if (jt < nvt) {
          const int rt = jt / nct, ct = jt - rt * nct, col = 16 * ct + ml;
#pragma unroll
          for (int i = 0; i < 4; ++i) u[k][i] *= Sc[16 * rt + 4 * mq + i];
          const float* wr = S + (16 * rt + ml) * ss + mq;
#pragma unroll
          for (int ks = 0; ks < kGSub; ks += 32) {
            float wv[8];
            uint32_t vv[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              const int pa = ks + mq + 4 * i, pb = pa + 4;
              wv[i] = wr[ks + 4 * i];
              wv[i + 1] = wr[ks + 4 * i + 4];
              const uint32_t va = pa < ns ? Vb[pa * dv + col] : 0u;
              const uint32_t vb = pb < ns ? Vb[pb * dv + col] : 0u;
              vv[i >> 1] = va | (vb << 16);
            }
            uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
            split_bf16(wv[0], wv[1], h0, l0);
            split_bf16(wv[2], wv[3], h1, l1);
            split_bf16(wv[4], wv[5], h2, l2);
            split_bf16(wv[6], wv[7], h3, l3);
            const bf16x8 bv = as_bf16x8(u32x4{vv[0], vv[1], vv[2], vv[3]});
            u[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{h0, h1, h2, h3}), bv, u[k], 0, 0, 0);
            u[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{l0, l1, l2, l3}), bv, u[k], 0, 0, 0);
          }
        }
      }
    };
    for (int q0 = p0; q0 < p1; q0 += kGSub) subtile(q0, kra, vra);
    if (first) trace[3] = wall_clock64();
    // the value sums to LDS (over the queries, no longer read), then the task's partial
    float* Acc = Qs;
#pragma unroll
    for (int k = 0; k < kGqaTiles; ++k) {
      const int jt = wave + kWaves * k;
      if (jt < nvt) {
        const int rt = jt / nct, ct = jt - rt * nct;
#pragma unroll
        for (int i = 0; i < 4; ++i) Acc[(16 * rt + 4 * mq + i) * d + 16 * ct + ml] = u[k][i];
      }
    }
    __syncthreads();
    for (int r = wave; r < nr; r += kWaves) {  // the task's partial: max, sum, values
      const int t = r / qg, hq = g * qg + (r - t * qg), m = b * T + t;
      float* dst = p.part + ((size_t)(m * nq + hq) * nsplit + s) * stride;
      for (int j = lane; j < d; j += 64) stc(dst + kPartPad + j, Acc[r * d + j]);
      if (lane == 0) {
        stc(dst, Mx[r]);
        stc(dst + 1, Ls[r]);
      }
    }
  }
}

// an int as a type: the lane-group width of a generic lambda, fixed at compile time
template <int N>
struct IntC {
  static constexpr int value = N;
};

// Merge split-KV partials: out[m][h*dim + j] = sum_s e^{mx_s - M} u_s[j] / sum_s e^{mx_s - M} l_s
// over the splits s (M the largest mx_s). Task = (m, h, 32 values); a workgroup takes a contiguous
// range of tasks, so its tasks share few (m, h) units. As many of them as LDS holds are one batch:
// the statistics of the batch's units and every split's values of its tasks are copied into LDS
// together (one memory round trip per batch, not per task). A group of P lanes then owns four
// values of a task: it takes the unit's maximum over splits r, r + P, ... (lane r), then the split
// weights, weighted values and weighted sums over the same splits, and reduces each over the group
// (P = 64 for a batch of one task, else 8).
__device__ __forceinline__ void merge_phase(const Params& p, const Ws& ws, int heads, int dim, float* out,
                                            float* smem) {
  const int nsplit = rfl(p.nsplit), stride = dim + kPartPad, nj = (dim + 31) >> 5, ntask = rfl(p.M) * heads * nj;
  const float* part = rflp(p.part);
  const int tid = tid_x();
  const int t0 = (int)((unsigned)ntask * blockIdx.x / gridDim.x), t1 = (int)((unsigned)ntask * (blockIdx.x + 1) / gridDim.x);
  // tasks per batch: a batch of tb tasks spans at most tb + 1 units of 4 statistics per split; a
  // task holds 32 values per split
  const int tb = max(1, (kLdsFloats - 4 * nsplit) / (36 * nsplit));
  for (int b0 = t0; b0 < t1; b0 += tb) {
    const int nt = min(tb, t1 - b0), u0 = b0 / nj, nu = (b0 + nt - 1) / nj - u0 + 1;
    float* hdr = smem;                  // [nu][nsplit][4] max, sum
    float* val = hdr + 4 * nu * nsplit;  // [nt][nsplit][32] values
    __syncthreads();  // the previous batch is consumed
    dma_rows<kCoherent>(ws.r, hdr, nu, nsplit, 4 * nsplit,
                        [&](int r, int c) { return ws.off(part + ((size_t)(u0 + r) * nsplit + c) * stride); });
    dma_rows<kCoherent>(ws.r, val, nt, 8 * nsplit, 32 * nsplit, [&](int r, int c) {
      const int t = b0 + r, u = t / nj, j0 = (t - u * nj) * 32, nv = min(32, dim - j0) >> 2, q = c & 7;
      return ws.off(part + ((size_t)u * nsplit + (c >> 3)) * stride + kPartPad + j0 + 4 * min(q, nv - 1));
    });
    wait_vm();
    __syncthreads();
    // items (task, quad of values), P lanes per item: 64 when the batch is one task, else 8
    const int G = nt * 8;
    auto items = [&](auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      const int r = tid & (P - 1);
      for (int g0 = 0; g0 < G; g0 += kThreads / P) {
        const int g = g0 + tid / P, tl = min(g, G - 1) >> 3, q = g & 7;
        const int t = b0 + tl, u = t / nj, j0 = (t - u * nj) * 32, nv = min(32, dim - j0) >> 2;
        const float* hu = hdr + 4 * (u - u0) * nsplit;
        float mx = -INFINITY;
#pragma unroll 4
        for (int s = r; s < nsplit; s += P) mx = fmaxf(mx, hu[4 * s]);
        mx = wave_max(mx, P);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        const float* vt = val + 32 * tl * nsplit + 4 * q;
#pragma unroll 4
        for (int s = r; s < nsplit; s += P) {
          const float2 st = *reinterpret_cast<const float2*>(hu + 4 * s);
          const float w = st.x == -INFINITY ? 0.f : __expf(st.x - mx);
          lsum += w * st.y;
          acc += w * *reinterpret_cast<const f32x4*>(vt + 32 * s);
        }
        lsum = wave_sum(lsum, P);
        acc.x = wave_sum(acc.x, P);
        acc.y = wave_sum(acc.y, P);
        acc.z = wave_sum(acc.z, P);
        acc.w = wave_sum(acc.w, P);
        if (g < G && q < nv && r == 0) ws.st4(out + (size_t)u * dim + j0 + 4 * q, acc * (1.0f / lsum));
      }
    };
    if (nt == 1)
      items(IntC<64>{});
    else
      items(IntC<8>{});
  }
}

// MLA split-KV partials over the latent cache. Task (b, s) covers positions [s*C, s*C + C) of
// sequence b for every head and every new token. Scores use the absorbed query (W_uk^T q_nope)
// against the latent part and the rotated query against the shared rope key, scaled by
// 1/sqrt(nope + rope); positions are staged kSub at a time (bf16, as stored) with a running max and
// sum per head; scores (query split into bf16 high and low parts) and value sums (weights split
// likewise) run on the matrix cores. New entries (normalised latent, rotated rope key, rounded to
// bf16) are appended to the cache by the task whose range holds their position.
// The cache rows the workgroup's first task reads first (the rows already in the cache, direct copies
// into LDS): issued before the phase's barrier, since they do not depend on the step's earlier phases.
__device__ __forceinline__ void mla_prefetch_rows(const Params& p, const LayerDev* ly, float* smem) {
  const int kv_len = rfl(p.kv_len), Bmax = rfl(p.Bmax), B = rfl(p.B), T = rfl(p.T), cap = rfl(p.cap);
  const int lat = rfl(p.kvl) + rfl(p.rd), cst = lat + 8;
  const int npos = kv_len + T, C = rfl(p.chunk), nsplit = rfl(p.nsplit), task = blockIdx.x;
  if (task >= B * nsplit) return;
  const int s = task % nsplit, b = task / nsplit;
  const int p0 = s * C, p1 = imin(npos, p0 + C), pe = imin(p1, kv_len + 1);
  if (pe <= p0) return;
  const int n = p1 - p0 <= kSub ? p1 - p0 : imin(kSub, pe - p0);
  const int nold = imax(0, imin(kv_len - p0, n));
  const uint16_t* Lb = rflp(p.kv) + ((size_t)rfl(ly->ord) * Bmax + b) * cap * lat;
  const Rsrc lr = make_rsrc(Lb, (uint32_t)cap * lat * 2);
  // every wave but the polling one: its polls would complete only after its copies
  const int w = wave_id(), lane = lane_id(), U = lat >> 3, bpr = (U + 63) >> 6, nb = nold * bpr;
  if (w == kPollWave) return;
  for (int bk = w; bk < nb; bk += kWaves - 1) {
    const int r = bk / bpr, c0 = (bk - r * bpr) << 6, c = c0 + lane;
    if (c < U)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (LdsPtr)(smem + r * (cst / 2) + 4 * c0), 16,
                                               (uint32_t)((p0 + r) * lat) * 2 + c * 16, 0, 0, 2);
  }
}

// RD: the rope dimension when it is known at compile time (64 in the MLA family's instances, whose
// models all have it), else 0 (read from the parameters: the hybrid family's instances, which also
// run MLA models of other rope dimensions). Constant row strides and loop bounds take about 3% off
// the K3-scale share's batch-1 step. ONE: the 1-row instance (one sequence, one new token).
template <int RD, bool ONE>
__device__ __forceinline__ void mla_attn_phase(const Params& p, const LayerDev* ly, const Ws& ws, float* smem,
                                               const float* rope, LdsU64* trace) {
  static_assert(kSub == 32, "score lanes map one position each in a half wave");
  // step values in scalar registers (read from the parameter block in LDS)
  const int kv_len = rfl(p.kv_len), Bmax = rfl(p.Bmax), B = ONE ? 1 : rfl(p.B);
  const float eps = rflf(p.eps);
  const float* a2 = rflp(p.a2);
  const float* a3 = rflp(p.a3);
  const float* a4 = rflp(p.a4);
  float* part = rflp(p.part);
  uint16_t* kvc = rflp(p.kv);
  constexpr int kvl = 512;  // the host admits kv_lora 512 only (a constant stride: 1% of the step)
  const int nh = rfl(p.nh), rd = RD ? RD : rfl(p.rd), nd = rfl(p.nd), T = ONE ? 1 : rfl(p.T), cap = rfl(p.cap);
  const int lat = kvl + rd, qd = nd + rd, h2 = rd / 2, half = lat / 2;
  const int cst = lat + 8;  // bf16 per staged cache row: 16-byte aligned rows, banks staggered by 4
  const int npos = kv_len + T, C = rfl(p.chunk), nsplit = rfl(p.nsplit), ntask = B * nsplit;
  const int tid = tid_x(), lane = lane_id(), wave = wave_id();
  uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);  // [kSub][cst] cache rows (bf16)
  // The heads are the rows of 16-row matrix-core tiles: a share with fewer heads (an even number up
  // to 16) pads them to 16. Padding rows are never filled; they only reach the tiles' padding rows,
  // whose results are not used.
  constexpr int nhp = 16;
  float* Qt = smem + kSub * cst / 2;                  // [nhp][lat] query of one token (fp32), then
  uint16_t* Qh = reinterpret_cast<uint16_t*>(Qt);     //   its bf16 high parts [nhp][lat]
  uint16_t* Ql = Qh + nhp * lat;                      //   and low parts [nhp][lat]; finally values [nhp][kvl]
  float* Nw = Qt + nhp * lat;                         // [T][lat] new latent rows (values of their bf16)
  float* Sp = Nw + T * lat;                           // [4][nhp][kSub] partial scores of the K groups
  float* S = Sp + 4 * nhp * kSub;                     // [nhp][kSub] weights
  float* st = S + nhp * kSub;                         // [nhp][4] running max, running sum, rescale
  float* nrm = st + nhp * 4;                          // [8] RMS scale of the new rows
  uint16_t* gk = reinterpret_cast<uint16_t*>(nrm + 8);  // [kvl] latent norm gain (bf16)
  uint16_t* Lc = kvc + (size_t)rfl(ly->ord) * Bmax * cap * lat;
  const float scale = 1.0f / sqrtf((float)qd);
  const int stride = kvl + kPartPad;
  const int nks = lat / 32;                    // 32-wide K steps of the scores
  const int kgs = (nks + 3) / 4;               // K steps per group (4 groups x 2 position tiles = 8 waves)
  const int ml = lane & 15, mq = lane >> 4;    // MFMA lane: row/column l % 16, K octet l / 16
  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int s = task % nsplit, b = task / nsplit;
    const int p0 = s * C, p1 = min(npos, p0 + C);
    uint16_t* Lb = Lc + (size_t)b * cap * lat;
    const Rsrc lr = make_rsrc(Lb, (uint32_t)cap * lat * 2);
    const int n0 = max(p0, kv_len), nnew = max(0, p1 - n0), tA = n0 - kv_len;
    __syncthreads();
    if (nnew > 0) {  // raw new rows (kv_a output) and the latent norm gain, then normalise and rotate
      dma_rows<kCoherent>(ws.r, Nw + tA * lat, nnew, lat >> 2, lat,
               [&](int r, int c) { return ws.off(a2 + (size_t)(b * T + tA + r) * lat + 4 * c); });
      const Rsrc gr = make_rsrc(rflp(ly->kv_norm), (uint32_t)kvl * 2);
      dma_rows<0>(gr, reinterpret_cast<float*>(gk), 1, kvl >> 3, 0, [&](int, int c) { return (uint32_t)c * 16; });
      wait_vm();
      __syncthreads();
      for (int r = wave; r < nnew; r += kWaves) {
        float ss = 0.f;
        for (int j = lane; j < kvl; j += 64) {
          const float v = Nw[(tA + r) * lat + j];
          ss += v * v;
        }
        ss = wave_sum(ss, 64);
        if (lane == 0) nrm[r] = 1.0f / sqrtf(ss / (float)kvl + eps);
      }
      __syncthreads();
      const int per = kvl + h2;
      for (int e = tid; e < nnew * per; e += kThreads) {
        const int r = e / per, j = e - r * per, t = tA + r;
        float* row = Nw + t * lat;
        uint16_t* dst = Lb + (size_t)(kv_len + t) * lat;
        if (j < kvl) {
          const uint16_t v = f2bf(row[j] * nrm[r] * bf2f(gk[j]));
          row[j] = bf2f(v);
          gp(dst)[j] = v;
        } else {
          const int jj = j - kvl;
          float x0 = row[kvl + jj], x1 = row[kvl + jj + h2];
          rope_pair(rope, t, jj, x0, x1);
          const uint16_t v0 = f2bf(x0), v1 = f2bf(x1);
          row[kvl + jj] = bf2f(v0);
          row[kvl + jj + h2] = bf2f(v1);
          gp(dst)[kvl + jj] = v0;
          gp(dst)[kvl + jj + h2] = v1;
        }
      }
    }
    // Stage cache rows [c0, c0+n): rows already in the cache by direct copy, new rows from Nw
    // (after the copies have landed: see fill_new).
    auto issue_c = [&](int c0, int n) {
      const int nold = max(0, min(kv_len - c0, n));
      dma_rows<2>(lr, reinterpret_cast<float*>(Cs), nold, lat >> 3, cst / 2,
               [&](int r, int c) { return (uint32_t)((c0 + r) * lat) * 2 + c * 16; });
    };
    auto fill_new = [&](int c0, int n) {
      const int r0 = max(0, kv_len - c0);
      for (int e = tid; e < (n - r0) * (lat >> 2); e += kThreads) {
        if (r0 >= n) break;
        const int r = r0 + e / (lat >> 2), c = e - (r - r0) * (lat >> 2);
        const f32x4 v = *reinterpret_cast<const f32x4*>(Nw + (c0 + r - kv_len) * lat + 4 * c);
        uint2 w;
        w.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
        w.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
        *reinterpret_cast<uint2*>(Cs + r * cst + 4 * c) = w;
      }
    };
    // The rows of the next sub-tile are in flight in registers while the current one is scored: a
    // direct copy into LDS would make every LDS read of the scoring wait for it (LDS reads after a
    // copy into LDS wait for the copy). The host admits kv_lora 512 and rope_dim <= 2 kMaxRopePairs,
    // so a row has at most (512 + 2 kMaxRopePairs) / 8 units of 16 bytes.
    constexpr int kMU = (kSub * ((512 + 2 * kMaxRopePairs) / 8) + kThreads - 1) / kThreads;
    const int lu = lat >> 3;
    uint4 cr[kMU];
    auto issue_r = [&](int c0, int n) __attribute__((always_inline)) {
      const int nold = max(0, min(kv_len - c0, n));
#pragma unroll
      for (int u = 0; u < kMU; ++u) {
        const int i = u * kThreads + tid, r = i / lu, c = i - r * lu;
        const bool ok = r < nold;  // (other lanes read row 0)
        cr[u] = ldw(Lb + (size_t)(ok ? c0 + r : 0) * lat + 8 * (ok ? c : 0));
      }
    };
    auto store_r = [&](int c0, int n) __attribute__((always_inline)) {
      const int nold = max(0, min(kv_len - c0, n));
#pragma unroll
      for (int u = 0; u < kMU; ++u) {
        const int i = u * kThreads + tid, r = i / lu, c = i - r * lu;
        if (r < nold) *reinterpret_cast<uint4*>(Cs + r * cst + 8 * c) = cr[u];
      }
    };
    const bool whole = p1 - p0 <= kSub;  // the range is staged once, by the first token that reads it
    bool staged = false;
    for (int t = 0; t < T; ++t) {
      const int m = b * T + t, qpos = kv_len + t, pe = min(p1, qpos + 1);
      f32x4 u[4];  // values: column tiles 4*wave + ct, rows 4*mq + i (heads), column ml
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) u[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (tid < nh) {
        st[tid * 4] = -INFINITY;
        st[tid * 4 + 1] = 0.f;
        st[tid * 4 + 2] = 1.f;
      }
      if (pe > p0) {
        // the token's query (absorbed latent part | raw rope part) and the first cache rows
        const int nfirst = (!whole || !staged) ? (whole ? p1 - p0 : min(kSub, pe - p0)) : 0;
        dma_rows<kCoherent>(ws.r, Qt, nh, kvl >> 2, lat,
                            [&](int h, int c) { return ws.off(a4 + ((size_t)m * nh + h) * kvl + 4 * c); });
        dma_rows<kCoherent>(ws.r, Qt + kvl, nh, rd >> 2, lat,
                            [&](int h, int c) { return ws.off(a3 + ((size_t)m * nh + h) * qd + nd + 4 * c); });
        if (task != (int)blockIdx.x || t != 0) issue_c(p0, nfirst);  // else requested before the barrier
        wait_vm();
        __syncthreads();
        fill_new(p0, nfirst);
        staged = true;
        if (trace && tid == 0 && task == (int)blockIdx.x && t == 0) trace[2] = wall_clock64();
        for (int e = tid; e < nh * h2; e += kThreads) {
          const int h = e / h2, jj = e - h * h2;
          float* qr = Qt + h * lat + kvl;
          float x0 = qr[jj], x1 = qr[jj + h2];
          rope_pair(rope, t, jj, x0, x1);
          qr[jj] = x0;
          qr[jj + h2] = x1;
        }
        __syncthreads();
        // query as bf16 high and low parts (q = hi + lo to 16 bits), in place
        {
          const int nq4 = nh * lat / 4;
          f32x4 qv[5];
#pragma unroll
          for (int k = 0; k < 5; ++k) {
            const int i = k * kThreads + tid;
            if (k * kThreads < nq4) qv[k] = *reinterpret_cast<const f32x4*>(Qt + 4 * min(i, nq4 - 1));
          }
          __syncthreads();
#pragma unroll
          for (int k = 0; k < 5; ++k) {
            const int i = k * kThreads + tid;
            if (k * kThreads < nq4 && i < nq4) {
              uint32_t h01, h23, l01, l23;
              split_bf16(qv[k].x, qv[k].y, h01, l01);
              split_bf16(qv[k].z, qv[k].w, h23, l23);
              *reinterpret_cast<uint2*>(Qh + 4 * i) = make_uint2(h01, h23);
              *reinterpret_cast<uint2*>(Ql + 4 * i) = make_uint2(l01, l23);
            }
          }
        }
        for (int c0 = p0; c0 < pe; c0 += kSub) {
          const int n = min(kSub, pe - c0);
          if (c0 != p0) {
            __syncthreads();  // the previous sub-tile is consumed
            store_r(c0, n);
            fill_new(c0, n);
          }
          __syncthreads();
          if (c0 + kSub < pe) issue_r(c0 + kSub, min(kSub, pe - c0 - kSub));
          const bool mark = trace && tid == 0 && task == (int)blockIdx.x && t == 0 && c0 == p0;
          // scores on the matrix cores: wave -> position tile (wave & 1) x K group (wave >> 1)
          {
            const int pt = wave & 1, kg = wave >> 1;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* brow = Cs + (16 * pt + ml) * cst + 8 * mq;
            const uint16_t* ahi = Qh + ml * lat + 8 * mq;
            const uint16_t* alo = Ql + ml * lat + 8 * mq;
            for (int kk = kg * kgs; kk < min(nks, kg * kgs + kgs); ++kk) {
              const bf16x8 bv = ld_bf16x8(brow + 32 * kk);
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(ahi + 32 * kk), bv, d, 0, 0, 0);
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(alo + 32 * kk), bv, d, 0, 0, 0);
            }
            // D: column ml (position 16 pt + ml), rows 4 mq + i (heads 4 mq + i of this 16-head block)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sp[(kg * nhp + 4 * mq + i) * kSub + 16 * pt + ml] = d[i];
          }
          __syncthreads();
          if (mark) trace[4] = wall_clock64();
          // running max and sum: half a wave per head
          for (int hp = wave; hp < (nh >> 1); hp += kWaves) {
            const int h = 2 * hp + (lane >> 5), pl = lane & 31;
            float sv = -INFINITY;
            if (pl < n) {
              float a = 0.f;
              for (int k = 0; k < 4; ++k) a += Sp[(k * nhp + h) * kSub + pl];
              sv = a * scale;
            }
            const float cm = wave_max(sv, 32);
            const float mo = st[h * 4], lo = st[h * 4 + 1];
            const float mn = fmaxf(mo, cm);
            const float sc = mn == -INFINITY ? 1.f : __expf(mo - mn);
            const float w = sv == -INFINITY ? 0.f : __expf(sv - mn);
            const float ls = wave_sum(w, 32);
            S[h * kSub + pl] = w;
            if (pl == 0) {
              st[h * 4] = mn;
              st[h * 4 + 1] = lo * sc + ls;
              st[h * 4 + 2] = sc;
            }
          }
          __syncthreads();
          if (mark) trace[5] = wall_clock64();
          // values on the matrix cores: A = weights [16 heads][32 positions] (bf16 high and low
          // parts), B = cache rows [32 positions][16 columns]; wave -> column tiles 4 wave + ct
          {
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(S + ml * kSub + 8 * mq);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(S + ml * kSub + 8 * mq + 4);
            uint32_t h0, h1, h2_, h3, l0, l1, l2, l3;
            split_bf16(w0.x, w0.y, h0, l0);
            split_bf16(w0.z, w0.w, h1, l1);
            split_bf16(w1.x, w1.y, h2_, l2);
            split_bf16(w1.z, w1.w, h3, l3);
            const bf16x8 whi = as_bf16x8(u32x4{h0, h1, h2_, h3}), wlo = as_bf16x8(u32x4{l0, l1, l2, l3});
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sc = st[(4 * mq + i) * 4 + 2];
#pragma unroll
              for (int ct = 0; ct < 4; ++ct) u[ct][i] *= sc;
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
              const int col = 16 * (4 * wave + ct) + ml;
              uint32_t bw[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int r0 = 8 * mq + 2 * j, r1 = r0 + 1;
                const uint32_t v0 = r0 < n ? Cs[r0 * cst + col] : 0u;
                const uint32_t v1 = r1 < n ? Cs[r1 * cst + col] : 0u;
                bw[j] = v0 | (v1 << 16);
              }
              const bf16x8 bv = as_bf16x8(u32x4{bw[0], bw[1], bw[2], bw[3]});
              u[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi, bv, u[ct], 0, 0, 0);
              u[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo, bv, u[ct], 0, 0, 0);
            }
          }
        }
      }
      __syncthreads();
      if (trace && tid == 0 && task == (int)blockIdx.x && t == 0) trace[3] = wall_clock64();
      // values to LDS [nh][kvl] (the query's space), then to the partials in 16-byte rows
      float* Ut = Qt;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Ut[(4 * mq + i) * kvl + 16 * (4 * wave + ct) + ml] = u[ct][i];
      __syncthreads();
      for (int e = tid; e < nh * (kvl >> 2); e += kThreads) {
        const int h = e / (kvl >> 2), c = e - h * (kvl >> 2);
        ws.st4(part + ((size_t)(m * nh + h) * nsplit + s) * stride + kPartPad + 4 * c,
               *reinterpret_cast<const f32x4*>(Ut + h * kvl + 4 * c));
      }
      if (tid < nh)
        ws.st4(part + ((size_t)(m * nh + tid) * nsplit + s) * stride, f32x4{st[tid * 4], st[tid * 4 + 1], 0.f, 0.f});
    }
  }
}

// gated delta rule: task (b, h, cb) owns columns [8cb, 8cb+8) of S_bh, one wave per task
__device__ __forceinline__ void kda_phase(const Params& p, const LayerDev* ly, const Ws& ws) {
  const int nh = p.nh, dk = p.dk, dv = p.dv, T = p.T;
  const int ncb = dv / 8;
  const int ntask = p.B * nh * ncb;
  const int gw = blockIdx.x * kWaves + wave_id(), tw = gridDim.x * kWaves;
  const int lane = lane_id();
  const int rpl = dk / 64;  // rows per lane (dk is 64 or 128)
  float* St = rflp(p.kda_state) + (size_t)rfl(ly->ord) * p.Bmax * nh * dk * dv;
  for (int task = gw; task < ntask; task += tw) {
    const int cb = task % ncb, h = (task / ncb) % nh, b = task / (ncb * nh);
    float* Sbh = St + ((size_t)b * nh + h) * dk * dv;
    float S[2][8];
    float al[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + (r < rpl ? r : 0) * 64;
      const f32x4 a = *(const GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8);
      const f32x4 c = *(const GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8 + 4);
      S[r][0] = a.x; S[r][1] = a.y; S[r][2] = a.z; S[r][3] = a.w;
      S[r][4] = c.x; S[r][5] = c.y; S[r][6] = c.z; S[r][7] = c.w;
      al[r] = gp(rflp(ly->alpha))[h * dk + i];
    }
    const float beta = gp(rflp(ly->beta))[h];
    for (int t = 0; t < T; ++t) {
      const int m = b * T + t;
      const float* kv = p.a2 + (size_t)m * nh * dk + h * dk;
      const float* qv = p.a1 + (size_t)m * nh * dk + h * dk;
      const float* vv = p.a3 + (size_t)m * nh * dv + h * dv + cb * 8;
      float kk[2], qq[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = lane + (r < rpl ? r : 0) * 64;
        kk[r] = ws.ld1(kv + i);
        qq[r] = ws.ld1(qv + i);
      }
      const f32x4 va = ws.ld4(vv), vb = ws.ld4(vv + 4);
      const float vj[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
      float nrm = 0.f;
#pragma unroll
      for (int r = 0; r < 2; ++r) nrm += r < rpl ? kk[r] * kk[r] : 0.f;
      nrm = wave_sum(nrm, 64);
      const float inv = 1.0f / sqrtf(nrm);
#pragma unroll
      for (int r = 0; r < 2; ++r) kk[r] *= inv;
      float kS[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (r < rpl) {
            S[r][j] *= al[r];
            a += kk[r] * S[r][j];
          }
        }
        kS[j] = wave_sum(a, 64);
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (r < rpl) {
            S[r][j] = S[r][j] - beta * kk[r] * kS[j] + beta * kk[r] * vj[j];
            a += S[r][j] * qq[r];
          }
        }
        o[j] = wave_sum(a, 64);
      }
      if (lane == 0) {
        float* od = p.att + (size_t)m * nh * dv + h * dv + cb * 8;
        ws.st4(od, f32x4{o[0], o[1], o[2], o[3]});
        ws.st4(od + 4, f32x4{o[4], o[5], o[6], o[7]});
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r < rpl) {
        const int i = lane + r * 64;
        *(GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8) = f32x4{S[r][0], S[r][1], S[r][2], S[r][3]};
        *(GLOBAL f32x4*)(Sbh + (size_t)i * dv + cb * 8 + 4) = f32x4{S[r][4], S[r][5], S[r][6], S[r][7]};
      }
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
  float red[kWaves * MK_MAX_M];
  float rope[MK_MAX_NEW_TOKENS * kMaxRopePairs * 2];
  float rw[kMaxQueue];
  int rsel[kMaxQueue];
  int cnt[kMaxExperts];
  Route route;
  LayerDev lyd[2];  // layer table rows of the current and the next layer
  unsigned long long hmax[MK_MAX_M];  // greedy steps: this workgroup's argmax keys of the LM head
  int amx[MK_MAX_M];
  int abort;
  uint64_t stamps[2][kTraceStamps];  // trace stamps of the current and the previous record
};

enum PhaseType : int { PT_GEMV = 0, PT_ATTN_GQA, PT_ATTN_MLA, PT_MERGE, PT_KDA, PT_EXPERT, PT_MUV };

__device__ __forceinline__ int attn_phases(int kind, int mfuse) {
  return kind == kGqa ? 4 : kind == kMla ? 7 - mfuse : 3;
}

// ----------------------------------------------------------------------------------------------
// Split-KV merge and W_uv in one phase (mfuse; the host uses it for 1- and 2-row steps of MLA
// layers), so W_uv waits on no grid barrier of its own. Merge arithmetic as merge_phase: weights
// exp(max_s - max), values summed and divided by the weighted sums.
// The head's 512 latent values are split into JB blocks (4 at 1 row, 2 at 2 rows, 1 at 3-8 rows on
// the matrix-core instances) and its 128 W_uv output rows into RB blocks rb (4 of 32 rows; 2 of 64
// in the 8-row instance), at most 256 tasks at 16 heads. Task (m, h, jb, rb) runs on workgroup
// rb*M*nh*JB + (m*nh + h)*JB + jb (the four row blocks that read the same values sit on one XCD): it
// merges its latent block (1/JB of the head's partials) and writes the 32 partial sums of its
// W_uv block over it. The last of a (m, h, rb)'s JB tasks to finish (an integer counter per
// (m, h, rb); old == JB - 1 marks it) adds the JB partials in block order, so the result does not
// depend on which task finished last, and sets the counter back to zero: every phase, whatever
// its JB, starts from zero (the workspace starts zeroed; the static scratch's flags are cleared
// before each launch), and the store completes before that workgroup's next barrier arrival.
// ----------------------------------------------------------------------------------------------
constexpr int kMuvRB = 4;     // output row blocks per head (up to 4 rows)
constexpr int kMuvNB = 8;     // splits per thread per batch of loads
// the counters, one per (row, head, row block): the last 128 of the barrier's flag words, which no
// grid polls
constexpr int kMuvCtr = kMaxBlocks - 128;
static_assert(kMaxGrid <= kMuvCtr, "the merge counters sit beyond the barrier's flags");
template <int MM>
__device__ __forceinline__ void muv_phase(const Params& p, const LayerDev* ly, const Ws& ws, float* smem) {
  constexpr int kvl = 512, vd = 128;                 // the host admits kv_lora 512, v_dim 128
  constexpr int JB = MM == 1 ? 4 : MM == 2 ? 2 : 1;  // latent blocks per head
  constexpr int RB = MM == 8 ? 2 : kMuvRB;           // output row blocks per head
  constexpr int rows = vd / RB, tpr = kThreads / rows;  // threads per output row
  constexpr int cols = kvl / JB, nq = cols / 4, ng = kThreads / nq, nu = cols / (8 * tpr);
  static_assert(nu >= 1 && nu * 8 * tpr == cols, "tpr threads per row, 8*nu of the block's columns each");
  const int nh = rfl(p.nh), nsplit = rfl(p.nsplit), stride = kvl + kPartPad;
  const int M = MM <= 2 ? MM : rfl(p.M);  // the matrix-core instances take 3..MM rows
  const int b = blockIdx.x;
  if (b >= M * nh * RB * JB) return;
  const int g = b % (M * nh * JB), rb = b / (M * nh * JB), m = g / (nh * JB), h = (g / JB) % nh, jb = g % JB;
  const int tid = tid_x(), lane = lane_id(), w = wave_id();
  const float* part = rflp(p.part) + (size_t)(m * nh + h) * nsplit * stride;
  float* hdr = smem;                // [nsplit][4] max, sum
  f32x4* grp = reinterpret_cast<f32x4*>(hdr + 4 * kMaxGrid);  // [ng][nq] split-group sums
  float* vb = hdr + 4 * kMaxGrid + 4 * kThreads;              // [cols] merged values
  float* ls = vb + kvl;                                       // the weighted sum; the counter's verdict
  // this thread's W_uv row (rb*rows + tid/tpr) and its 8*nu columns of the block, nu chunks
  const uint16_t* wr =
      rflp(ly->w_uv) + ((size_t)h * vd + rb * rows + tid / tpr) * kvl + jb * cols + 8 * nu * (tid % tpr);
  uint4 wv[nu];
#pragma unroll
  for (int u = 0; u < nu; ++u) wv[u] = ldw(wr + 8 * u);
  dma_rows<kCoherent>(ws.r, hdr, 1, nsplit, 0, [&](int, int c) { return ws.off(part + (size_t)c * stride); });
  // values: thread (quad cq of the block, split group sg of ng) sums splits sg + ng*k
  const int cq = tid % nq, sg = tid / nq, per = (nsplit + ng - 1 - sg) / ng, nb = (per + kMuvNB - 1) / kMuvNB;
  auto load = [&](f32x4 (&v)[kMuvNB], int k) {
#pragma unroll
    for (int u = 0; u < kMuvNB; ++u) {
      const int s = min(sg + ng * (k * kMuvNB + u), nsplit - 1);
      v[u] = ws.ld4(part + (size_t)s * stride + kPartPad + jb * cols + 4 * cq);
    }
  };
  f32x4 va[kMuvNB], vbb[kMuvNB];
  load(va, 0);
  wait_vm();
  __syncthreads();
  float mx = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, hdr[4 * s]);
  mx = wave_max(mx, 64);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](const f32x4 (&v)[kMuvNB], int k) {
#pragma unroll
    for (int u = 0; u < kMuvNB; ++u) {
      const int j = k * kMuvNB + u, s = sg + ng * j;
      if (j < per) {
        const float ms = hdr[4 * s];
        acc += (ms == -INFINITY ? 0.f : __expf(ms - mx)) * v[u];
      }
    }
  };
  for (int k = 0; k < nb; k += 2) {
    if (k + 1 < nb) load(vbb, k + 1);
    add(va, k);
    if (k + 2 < nb) load(va, k + 2);
    if (k + 1 < nb) add(vbb, k + 1);
  }
  grp[sg * nq + cq] = acc;
  if (w == 0) {  // the weighted sum of the splits' sums
    float l = 0.f;
    for (int s = lane; s < nsplit; s += 64) {
      const float ms = hdr[4 * s];
      l += (ms == -INFINITY ? 0.f : __expf(ms - mx)) * hdr[4 * s + 1];
    }
    l = wave_sum(l, 64);
    if (lane == 0) ls[0] = l;
  }
  __syncthreads();
  if (tid < nq) {
    f32x4 v = grp[tid];
#pragma unroll
    for (int g = 1; g < ng; ++g) v += grp[g * nq + tid];
    *reinterpret_cast<f32x4*>(vb + 4 * tid) = v * (1.0f / ls[0]);
  }
  __syncthreads();
  // this workgroup's W_uv rows over its block: tpr threads per row, 8*nu columns each
  float a = 0.f;
#pragma unroll
  for (int u = 0; u < nu; ++u) {
    float f[8];
    unpack8(wv[u], f);
    const float* x = vb + 8 * nu * (tid % tpr) + 8 * u;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(x), x1 = *reinterpret_cast<const f32x4*>(x + 4);
    a += f[0] * x0.x + f[1] * x0.y + f[2] * x0.z + f[3] * x0.w + f[4] * x1.x + f[5] * x1.y + f[6] * x1.z + f[7] * x1.w;
  }
  a = wave_sum(a, tpr);
  if constexpr (JB == 1) {  // whole heads: the sum is complete
    if (tid % tpr == 0) stc(rflp(p.o2) + ((size_t)m * nh + h) * vd + rb * rows + tid / tpr, a);
    return;
  }
  // partials [m][h][rb][jb][rows] in the merge's output buffer (unused when the merge is fused)
  float* op = rflp(p.att) + (size_t)((m * nh + h) * RB + rb) * JB * rows;
  if ((tid & 15) == 0) stc(op + jb * rows + (tid >> 4), a);
  wait_vm();  // this workgroup's partials complete before its count
  __syncthreads();
  uint32_t* ctr = p.flags + kMuvCtr + (m * nh + h) * RB + rb;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add((GLOBAL uint32_t*)ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    reinterpret_cast<uint32_t*>(ls)[1] = old;
  }
  __syncthreads();
  if (reinterpret_cast<const uint32_t*>(ls)[1] == JB - 1 && tid < rows) {
    if (tid == 0) stc_u32(ctr, 0u);  // every arrival is in: the next phase starts from zero
    float q[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) q[j] = ws.ld1(op + j * rows + tid);
    float sum = q[0];
#pragma unroll
    for (int j = 1; j < JB; ++j) sum += q[j];
    stc(rflp(p.o2) + ((size_t)m * nh + h) * vd + rb * rows + tid, sum);
  }
}


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

// the attention block's output projection of layer l: residual from the layer's input, output
// into the MoE block's input
__device__ __forceinline__ void resid_out(Gemv& g, const Params& p, const LayerDev* ly, int l) {
  g.kind = G_RESID;
  g.W0 = g.safe = ly->wo;
  g.src2 = xcur(p, l);
  g.out0 = xcur(p, l + 1);
  g.ldo0 = p.H;
  g.ntasks = p.H;
}

// Phase i of layer l (l == L: the final norm and LM head; ly: the layer's table row, in LDS). Fills
// g for GEMV phases; the down projection reads this workgroup's routing of the layer (rt).
// Fam: the model's attention family (MK_ATTN_GQA: every layer GQA; MK_ATTN_MLA: every layer MLA;
// MK_ATTN_HYBRID: MLA and delta-rule layers).
template <int Fam>
__device__ __forceinline__ int describe(const Params& p, int l, int i, Gemv& g, const Route* rt, const LayerDev* ly) {
  g.M = p.M;
  g.eps = p.eps;
  g.pairs = 1;
  g.n1 = 0;
  if (l == p.L) {
    norm_input(g, xcur(p, l), p.H, p.H, p.final_norm);
    g.kind = G_STACK;
    g.W0 = g.safe = p.lm_head;
    g.n0 = p.V;
    g.out0 = p.logits;
    g.ldo0 = p.V;
    g.ntasks = p.V;
    return PT_GEMV;
  }
  const int kind = ly->kind;
  const int na = attn_phases(kind, p.mfuse);
  float* xl = xcur(p, l);
  if (i >= na) {
    float* xm = xcur(p, l + 1);  // the MoE block's input (and output: its residual is added in place)
    const bool rf = p.rfuse;
    if (i == na && !rf) {
      norm_input(g, xm, p.H, p.H, ly->moe_norm);
      g.kind = G_RS;
      g.E = p.E;
      g.SF = p.SF;
      g.W0 = ly->router;
      g.safe = p.E ? ly->router : ly->sh_gate;  // dense: no router rows
      g.Wg = ly->sh_gate;
      g.Wu = ly->sh_up;
      g.rlog = p.rlog;
      g.sact = p.sact;
      g.ntasks = p.E + p.SF;
      g.pairs = p.SF > 0 ? 2 : 1;
      return PT_GEMV;
    }
    if (i == na + (rf ? 0 : 1) && p.E > 0) {  // a dense model has no routed-expert phase
      norm_input(g, xm, p.H, p.H, ly->moe_norm);
      g.kind = G_EXP;
      g.F = p.F;
      g.Wg = g.safe = ly->exp_gate;
      g.Wu = ly->exp_up;
      g.eact = p.eact;
      g.pairs = 2;
      g.ntasks = 0;  // known after routing
      if (rf) {  // router fusion: the shared expert's gate/up pairs follow the routed ones
        g.W0 = ly->sh_gate;
        g.W1 = ly->sh_up;
        g.SF = p.SF;
        g.sact = p.sact;
      }
      return PT_EXPERT;
    }
    // routed down projections (pool rows [E][H][F]) and the shared down projection
    g.kind = G_DOWN;
    g.stage = S_DOWN;
    g.src = p.eact;
    g.src2 = p.sact;
    g.rt = rt;
    g.np = rt->ustart[rt->nu];
    g.F = p.F;
    g.SF = p.SF;
    g.H = p.H;
    g.K = g.Wst = p.F > p.SF ? p.F : p.SF;
    g.Wg = ly->exp_down;
    g.safe = p.E ? ly->exp_down : ly->sh_down;  // dense: the (empty) expert pool has no rows
    g.Wu = ly->sh_down;
    g.out0 = xm;
    g.ldo0 = p.H;
    g.ntasks = p.H;
    g.pairs = rt->nu + (p.SF > 0 ? 1 : 0);
    return PT_GEMV;
  }
  if constexpr (Fam == MK_ATTN_GQA) {
    const int dq = p.nh * p.hd, dkv = p.nkv * p.hd;
    if (i == 0) {
      norm_input(g, xl, p.H, p.H, ly->attn_norm);
      g.kind = G_STACK;
      g.W0 = g.safe = ly->wq; g.W1 = ly->wk; g.W2 = ly->wv;
      g.n0 = dq; g.n1 = dkv;
      g.out0 = p.a1; g.out1 = p.a2; g.out2 = p.a3;
      g.ldo0 = dq; g.ldo1 = dkv; g.ldo2 = dkv;
      g.ntasks = dq + 2 * dkv;
      return PT_GEMV;
    }
    if (i == 1) return PT_ATTN_GQA;
    if (i == 2) return PT_MERGE;
    plain_input(g, p.att, dq, dq);
    resid_out(g, p, ly, l);
    return PT_GEMV;
  } else {
  if (kind == kMla) {
    const int lat = p.kvl + p.rd, qd = p.nd + p.rd;
    if (p.mfuse && i == 4) return PT_MUV;
    switch (p.mfuse && i >= 5 ? i + 1 : i) {
      case 0:
        norm_input(g, xl, p.H, p.H, ly->attn_norm);
        g.kind = G_STACK;
        g.W0 = g.safe = ly->w_dq; g.W1 = ly->w_dkv;
        g.n0 = p.ql; g.n1 = lat;
        g.out0 = p.a1; g.out1 = p.a2;
        g.ldo0 = p.ql; g.ldo1 = lat;
        g.ntasks = p.ql + lat;
        return PT_GEMV;
      case 1:
        norm_input(g, p.a1, p.ql, p.ql, ly->q_norm);
        g.kind = G_STACK;
        g.W0 = g.safe = ly->w_uq;
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
        g.W0 = g.safe = ly->w_ukT;
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
        g.W0 = g.safe = ly->w_uv;
        g.rph = p.vd;
        g.seg = p.kvl;
        g.out0 = p.o2;
        g.ldo0 = p.nh * p.vd;
        g.ntasks = p.nh * p.vd;
        return PT_GEMV;
      default:
        plain_input(g, p.o2, p.nh * p.vd, p.nh * p.vd);
        resid_out(g, p, ly, l);
        return PT_GEMV;
    }
  }
  // gated delta rule
  if constexpr (Fam != MK_ATTN_HYBRID) return PT_GEMV;  // (no such layer)
  const int dq = p.nh * p.dk, dvv = p.nh * p.dv;
  if (i == 0) {
    norm_input(g, xl, p.H, p.H, ly->attn_norm);
    g.kind = G_STACK;
    g.W0 = g.safe = ly->kwq; g.W1 = ly->kwk; g.W2 = ly->kwv;
    g.n0 = dq; g.n1 = dq;
    g.out0 = p.a1; g.out1 = p.a2; g.out2 = p.a3;
    g.ldo0 = dq; g.ldo1 = dq; g.ldo2 = dvv;
    g.ntasks = 2 * dq + dvv;
    return PT_GEMV;
  }
  if (i == 1) return PT_KDA;
  plain_input(g, p.att, dvv, dvv);
  resid_out(g, p, ly, l);
  return PT_GEMV;
  }
}

__device__ __forceinline__ void scalarize(Gemv& g) {
  g.kind = rfl(g.kind); g.stage = rfl(g.stage); g.ntasks = rfl(g.ntasks); g.K = rfl(g.K); g.Wst = rfl(g.Wst);
  g.pairs = rfl(g.pairs); g.M = rfl(g.M); g.src = rflp(g.src); g.ld = rfl(g.ld); g.gain = rflp(g.gain);
  g.nh = rfl(g.nh); g.nd = rfl(g.nd); g.qd = rfl(g.qd); g.eps = rflf(g.eps);
  g.src2 = rflp(g.src2); g.np = rfl(g.np);
  g.W0 = rflp(g.W0); g.W1 = rflp(g.W1); g.W2 = rflp(g.W2); g.Wg = rflp(g.Wg); g.Wu = rflp(g.Wu);
  g.safe = rflp(g.safe); g.n0 = rfl(g.n0); g.n1 = rfl(g.n1);
  g.out0 = rflp(g.out0); g.out1 = rflp(g.out1); g.out2 = rflp(g.out2);
  g.ldo0 = rfl(g.ldo0); g.ldo1 = rfl(g.ldo1); g.ldo2 = rfl(g.ldo2); g.rph = rfl(g.rph); g.seg = rfl(g.seg);
  g.E = rfl(g.E); g.SF = rfl(g.SF); g.F = rfl(g.F); g.H = rfl(g.H);
  g.rlog = rflp(g.rlog); g.sact = rflp(g.sact); g.eact = rflp(g.eact); g.hmax = rflp(g.hmax);
}

// Copy layer l's table row into LDS slot l % 2 (a direct copy; it has landed by the time the
// layer starts, after many waits and barriers in between).
__device__ __forceinline__ void fetch_layer(const Params& p, LayerDev* lyd, int l) {
  const Rsrc tr = make_rsrc(rflp(p.layers), (uint32_t)(rfl(p.L) * sizeof(LayerDev)));
  dma_rows<0>(tr, reinterpret_cast<float*>(lyd + (l & 1)), 1, (int)(sizeof(LayerDev) / 16), 0,
              [&](int, int c) { return (uint32_t)(l * sizeof(LayerDev) + c * 16); });
}

#define MK_FINISH()                                   \
  do {                                                \
    if (!barrier_finish(&sm.abort)) return;           \
  } while (0)

// ----------------------------------------------------------------------------------------------
// temperature / nucleus (top-p) sampling of one row of logits by one workgroup, after the LM head
// (the MoE model's server offers greedy or temperature/top-p generation: "tpu-megakernels README",
// section "OpenAI-compatible servers"). With e = exp((logit - max) / temperature) and Z its sum,
// the kept set is every token with e >= tau, tau the largest value whose kept sum reaches
// top_p * Z (found by bisection on the bits of tau: the kept sum only changes at the values of e,
// so the bisection ends on one of them and keeps every token tied with it); the token is the
// first, in index order, at which the running kept sum exceeds u * (kept sum), u the caller's
// uniform number. Thread t holds kSR consecutive logits of each tile of kThreads * kSR (the whole
// row when the vocabulary fits one tile); every sum is taken in a fixed order, so the result does
// not change from run to run.
// ----------------------------------------------------------------------------------------------
constexpr int kSR = 80;  // logits per thread and tile

// sum / maximum over the workgroup (every thread receives it); red holds kWaves floats
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v, 64);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < kWaves; ++w) t += red[w];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v, 64);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < kWaves; ++w) t = fmaxf(t, red[w]);
  return t;
}

__device__ __noinline__ void sample_row(const Params& p, int m, float* lds) {
  const int V = p.V, tid = tid_x(), lane = lane_id();
  const int tile = kThreads * kSR, ntile = (V + tile - 1) / tile;
  const float* row = p.logits + (size_t)m * V;
  const Rsrc lr = make_rsrc(row, (uint32_t)V * 4u);  // loads past the row read zero
  float* red = lds;       // [16] reductions and flags
  float* pre = lds + 16;  // [kThreads + 1] per-thread kept sums, then their prefixes
  float x[kSR];
  auto load = [&](int t) __attribute__((always_inline)) {
    const int base = t * tile + tid * kSR;
#pragma unroll
    for (int k = 0; k < kSR; k += 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lr, (uint32_t)(base + k) * 4u, 0, kCoherent);
      x[k] = __uint_as_float(v.x);
      x[k + 1] = __uint_as_float(v.y);
      x[k + 2] = __uint_as_float(v.z);
      x[k + 3] = __uint_as_float(v.w);
    }
  };
  const float invt = 1.0f / p.temperature;
  float mx = -INFINITY;
  for (int t = 0; t < ntile; ++t) {
    load(t);
#pragma unroll
    for (int k = 0; k < kSR; ++k)
      if (t * tile + tid * kSR + k < V) mx = fmaxf(mx, x[k]);
  }
  mx = block_max(mx, red);
  // e in place (the last tile stays resident; with one tile, the whole row)
  auto weights = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kSR; ++k) x[k] = t * tile + tid * kSR + k < V ? __expf((x[k] - mx) * invt) : 0.f;
  };
  auto tile_e = [&](int t) __attribute__((always_inline)) {
    if (ntile > 1) {
      load(t);
      weights(t);
    }
  };
  if (ntile == 1) weights(0);
  auto kept_sum = [&](float tau) __attribute__((always_inline)) {  // sum of e >= tau over the row
    float s = 0.f;
    for (int t = 0; t < ntile; ++t) {
      tile_e(t);
#pragma unroll
      for (int k = 0; k < kSR; ++k) s += x[k] >= tau ? x[k] : 0.f;
    }
    return block_sum(s, red);
  };
  const float Z = kept_sum(0.f);
  const float goal = p.top_p * Z;
  uint32_t lo = 0u, hi = __float_as_uint(1.0f) + 1u;  // kept_sum(lo) >= goal > kept_sum(hi)
  float mass = Z;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float s = kept_sum(__uint_as_float(mid));
    if (s >= goal) {
      lo = mid;
      mass = s;
    } else {
      hi = mid;
    }
  }
  const float tau = __uint_as_float(lo);
  const float target = gp(p.uniform)[m] * mass;
  // the running kept sum in index order: per-thread kept sums, then one non-decreasing sequence of
  // prefixes pre[0..kThreads] (group sums chained by one lane, each clamped to the next group's
  // start), so the half-open ranges [pre[t], pre[t+1]) tile [0, total) and exactly one thread holds
  // the target; it scans its own logits
  int tok = -1, last = -1;
  float base = 0.f;
  for (int t = 0; t < ntile && tok < 0; ++t) {
    tile_e(t);
    float sk = 0.f;
#pragma unroll
    for (int k = 0; k < kSR; ++k) sk += x[k] >= tau ? x[k] : 0.f;
    __syncthreads();
    pre[tid] = sk;
    __syncthreads();
    if (wave_id() == 0) {  // lane j: threads 8j .. 8j+7
      float g = 0.f;
      for (int i = 0; i < 8; ++i) g += pre[8 * lane + i];
      // group starts: one sequential chain, run identically by every lane on scalar reads of the
      // group sums, so every lane sees the same values (no exchange through memory)
      float g0 = 0.f, g1 = 0.f, chain = 0.f;
      for (int j = 0; j < 64; ++j) {
        if (lane == j) g0 = chain;
        chain += lane_f(g, j);
        if (lane == j) g1 = chain;
      }
      float run = g0;
      for (int i = 0; i < 8; ++i) {
        const float v = pre[8 * lane + i];
        pre[8 * lane + i] = fminf(run, g1);
        run += v;
      }
      if (lane == 63) pre[kThreads] = g1;
    }
    __syncthreads();
    const float start = base + pre[tid], next = base + pre[tid + 1];
    int mine = -1, lastk = -1;
    if (start <= target && target < next) {
      float c = start;
#pragma unroll
      for (int k = 0; k < kSR; ++k) {
        if (x[k] >= tau && x[k] > 0.f) {
          c += x[k];
          lastk = t * tile + tid * kSR + k;
          if (mine < 0 && c > target) mine = lastk;
        }
      }
      if (mine < 0) mine = lastk;  // rounding: the range's last kept token
    } else {
#pragma unroll
      for (int k = 0; k < kSR; ++k)
        if (x[k] >= tau && x[k] > 0.f) lastk = t * tile + tid * kSR + k;
    }
    base += pre[kThreads];
    __syncthreads();
    if (tid == 0) red[9] = -1.f;
    __syncthreads();
    if (mine >= 0) red[9] = (float)mine;  // at most one thread
    __syncthreads();
    tok = (int)red[9];
    last = max(last, (int)block_max((float)lastk, red));
  }
  if (tid == 0) gp(p.sampled)[m] = tok >= 0 ? tok : last;  // rounding past the end: the last kept
}

template <bool MF>
struct PlanOf {
  typedef Plan type;
};
template <>
struct PlanOf<true> {
  typedef MPlan type;
};

// MM: input rows the kernel is built for (at least M); MF: GEMV phases on the matrix cores
// AF: the model's attention family (MK_ATTN_GQA, MK_ATTN_MLA, MK_ATTN_HYBRID); each instance holds
// only its family's attention code, which keeps the others' registers out of its allocation
template <int MM, bool MF, int AF>
__global__ void __launch_bounds__(kThreads, 1) mk_decode_kernel(Params pk) {
  __shared__ Smem sm;
  // the parameters live in LDS: read where needed instead of pinning ~100 scalar registers
  __shared__ Params sp;
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&pk);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&sp);
    for (int i = tid_x(); i < (int)(sizeof(Params) / 4); i += kThreads) dst[i] = src[i];
    __syncthreads();
  }
  const Params& p = sp;
  const char* wsb = rflp(p.wsb);
  const Ws ws{make_rsrc(wsb, (uint32_t)rfl((int)p.ws_bytes)), wsb};
  uint32_t gen = 0;
  const int M = MM <= 2 ? MM : p.M, H = p.H;
  const int rpairs = ((p.kvl > 0) ? p.rd : p.hd) / 2;

  // ---- embedding rows and the RoPE table of this step's positions ----
  {
    const int n = M * H;
    for (int e = blockIdx.x * kThreads + tid_x(); e < n; e += gridDim.x * kThreads) {
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
    for (int e = tid_x(); e < p.T * rpairs; e += kThreads) {
      const int t = e / rpairs, j = e - t * rpairs;
      const double inv_freq = pow((double)p.rope_theta, -2.0 * j / (2 * rpairs));
      const double a = (double)(p.kv_len + t) * inv_freq;
      sm.rope[(t * kMaxRopePairs + j) * 2] = (float)cos(a);
      sm.rope[(t * kMaxRopePairs + j) * 2 + 1] = (float)sin(a);
    }
    fetch_layer(p, sm.lyd, 0);
    if (tid_x() < 2 * kTraceStamps) (&sm.stamps[0][0])[tid_x()] = 0;
    if (tid_x() == 0) {  // no routed experts until a routing phase fills the queues (dense: never)
      sm.route.nu = 0;
      sm.route.ustart[0] = 0;
    }
    // greedy steps: clear the device-wide argmax keys (many barriers precede the LM head's updates)
    if (p.greedy && blockIdx.x == 0 && tid_x() < M)
      __hip_atomic_store((GLOBAL unsigned long long*)(p.amax + tid_x()), 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    wait_vm();
    __syncthreads();
  }

  bool resident = false;  // the LDS input buffer holds this layer's normalised MoE input
  for (int l = 0; l <= p.L; ++l) {
    const LayerDev* ly = &sm.lyd[l & 1];
    const int nph = (l == p.L) ? 1 : attn_phases(ly->kind, p.mfuse) + (p.E && !p.rfuse ? 3 : 2);
    for (int i = 0; i < nph; ++i) {
      Gemv g{};
      typename PlanOf<MF>::type q{};
      RowBuf b0, b1;  // per phase: dead outside GEMV phases
      // Arrive at the barrier before this phase, then prepare the phase while the others arrive:
      // its descriptor, its plan and (for GEMV phases) the loads of its first weight rows (on the
      // polling wave too: its polls then queue behind them, which costs less than holding the
      // workgroup while it requests them after the poll). The routed-expert phase waits first
      // (routing needs every router logit). The weight rows are requested at one place so the
      // buffers are never copied.
      barrier_arrive(p, gen, (LdsU64*)sm.stamps);
      LdsU64* trec = kTrace && p.trace ? (LdsU64*)sm.stamps + ((gen - 1) & 1) * kTraceStamps : nullptr;
      const int type = rfl(describe<AF>(p, l, i, g, &sm.route, ly));
      if (l == p.L) {  // LM head: logits optional on greedy steps, per-workgroup argmax keys
        if (tid_x() < MK_MAX_M) sm.hmax[tid_x()] = 0ull;
        g.hmax = p.greedy ? sm.hmax : nullptr;
      }
      scalarize(g);
      if constexpr (MM <= 2) g.M = MM;  // the 1- and 2-row instances run exactly that many token rows
      if (trec && tid_x() == 0) trec[10] = wall_clock64();
      const bool early = type == PT_GEMV;  // prepared while waiting
      if (!early) {
        if constexpr (AF != MK_ATTN_GQA)
          if (type == PT_ATTN_MLA) mla_prefetch_rows(p, ly, sm.buf);
        if (wave_id() == kPollWave) barrier_poll(p, gen, &sm.abort, (LdsU64*)sm.stamps);
        MK_FINISH();
        if (trec && tid_x() == 0) trec[7] = wall_clock64();
        if (type == PT_EXPERT) {
          compute_route(p, ws, l, &sm.route, sm.rsel, sm.rw, sm.cnt, p.rfuse != 0);
          if (trec && tid_x() == 0) trec[6] = wall_clock64();
          g.rt = &sm.route;
          g.n0 = rfl(sm.route.nu * p.F);  // routed pairs; router fusion: the shared pairs after them
          g.ntasks = rfl(sm.route.nu * p.F + (p.rfuse ? p.SF : 0));
        }
      }
      if (type == PT_GEMV || type == PT_EXPERT) {
        if constexpr (MF) {
          q = mmake_plan<MM>(g, sm.buf);
          if (trec && tid_x() == 0) trec[11] = wall_clock64();
          mgemv_preload<mfma_segments(MM)>(g, q, b0, b1);
          if (g.kind == G_RESID && p.rfuse) router_side_issue(p, ly, l, ws, sm.buf + g.M * q.DS, g.M, g.Wst);
        } else {
          q = make_plan<MM>(g, sm.buf);
          if (trec && tid_x() == 0) trec[11] = wall_clock64();
          gemv_preload(g, q, b0, b1);
          if constexpr (MM <= 2)
            if (g.kind == G_RESID && p.rfuse) router_side_issue(p, ly, l, ws, sm.buf + MM * q.KS, MM, g.Wst);
        }
      }
      if (early) {
        if (trec && tid_x() == 0) trec[9] = wall_clock64();
        if (wave_id() == kPollWave) barrier_poll(p, gen, &sm.abort, (LdsU64*)sm.stamps);
        MK_FINISH();
        if (trec && tid_x() == 0) trec[7] = wall_clock64();
      }
      switch (type) {
        case PT_GEMV:
        case PT_EXPERT: {
          const bool keep = type == PT_EXPERT && resident;
          const bool side = g.kind == G_RESID && p.rfuse;
          if constexpr (MF) {
            if (side) router_side_issue_o(p, ws, sm.buf + g.M * q.DS, g.M, g.Wst, g.src, g.ld);
            resident = mgemv_phase<MM>(g, q, ws, sm.buf, sm.red, b0, b1, keep, trec) && g.kind == G_RS;
            if (side) router_side_logits(RSide{rflp(p.rlog), p.E, p.H, g.M}, sm.buf, q.DS, g.Wst, sm.buf + g.M * q.DS, true);
          } else {
            resident = gemv_phase<MM>(g, q, ws, sm.buf, sm.red, b0, b1, keep, trec) && g.kind == G_RS;
            if constexpr (MM <= 2)
              if (side) router_side_logits(RSide{rflp(p.rlog), p.E, p.H, MM}, sm.buf, q.KS, g.Wst, sm.buf + MM * q.KS, false);
          }
          if (side) router_side_ssq<MM>(rflp(p.ssq), g.M, q.nloc, q.acc, q.res);
          break;
        }
        // The next layer's table row is requested during the layer's attention phase, which waits
        // for its own copies into LDS anyway: a copy into LDS still in flight when a GEMV phase
        // starts would make every LDS read of its streaming loop wait for all loads (the compiler
        // cannot tell the two LDS areas apart).
        case PT_ATTN_GQA:
          if constexpr (AF == MK_ATTN_GQA) {
            if (l + 1 < p.L) fetch_layer(p, sm.lyd, l + 1);
            if (p.hd == 128) gqa_attn_phase<128, MM == 1 && !MF>(p, ly, ws, sm.buf, sm.rope, trec);
            else gqa_attn_phase<0, MM == 1 && !MF>(p, ly, ws, sm.buf, sm.rope, trec);
            resident = false;
          }
          break;
        case PT_ATTN_MLA:
          if constexpr (AF != MK_ATTN_GQA) {
            if (l + 1 < p.L) fetch_layer(p, sm.lyd, l + 1);
            mla_attn_phase<AF == MK_ATTN_MLA ? 64 : 0, MM == 1 && !MF>(p, ly, ws, sm.buf, sm.rope, trec);
            resident = false;
          }
          break;
        case PT_MUV:
          if constexpr (AF != MK_ATTN_GQA && ((MM <= 2 && !MF) || ((MM == 4 || MM == 8) && MF))) {
            muv_phase<MM>(p, ly, ws, sm.buf);
            resident = false;
          }
          break;
        case PT_MERGE:
          merge_phase(p, ws, p.nh, p.kvl > 0 ? p.kvl : p.hd, p.att, sm.buf);
          resident = false;
          break;
        case PT_KDA:
          if constexpr (AF == MK_ATTN_HYBRID) {
            if (l + 1 < p.L) fetch_layer(p, sm.lyd, l + 1);
            kda_phase(p, ly, ws);
            resident = false;
          }
          break;
        default:
          break;
      }
      if (l == p.L && p.greedy) {  // the workgroup's keys into the device-wide ones
        __syncthreads();
        if (tid_x() < rfl(p.M) && sm.hmax[tid_x()] != 0ull)
          __hip_atomic_fetch_max((GLOBAL unsigned long long*)(p.amax + tid_x()), sm.hmax[tid_x()], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_vm();
      if (trec && tid_x() == 0) trec[8] = wall_clock64();
    }
  }
  if (p.greedy || p.sample) {  // one more barrier: every row's logits (or argmax keys) are complete
    barrier_arrive(p, gen, (LdsU64*)sm.stamps);
    if (wave_id() == kPollWave) barrier_poll(p, gen, &sm.abort, (LdsU64*)sm.stamps);
    MK_FINISH();
  }
  // (the step's row count read again from the parameter block: kept live from the start of the
  // step to here, it would be spilled to scratch memory)
  const int Mend = rfl(p.M);
  if (p.sample) {
    for (int m = blockIdx.x; m < Mend; m += gridDim.x) sample_row(p, m, sm.buf);
  }
  if (p.greedy) {  // workgroup 0 turns the keys into tokens and accepts drafts
    if (blockIdx.x == 0) {
      const int tid = tid_x();
      if (tid < Mend) {
        const unsigned long long key =
            __hip_atomic_load((GLOBAL unsigned long long*)(p.amax + tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int tok = (int)(0xFFFFFFFFu - (uint32_t)key);
        sm.amx[tid] = tok;
        gp(p.argmax)[tid] = tok;
      }
      __syncthreads();
      if (p.accepted != nullptr && tid < p.B) {  // drafts accepted while they equal the previous argmax
        const int T = p.T;
        int n = 0;
        while (n + 1 < T && gp(p.tokens)[tid * T + n + 1] == sm.amx[tid * T + n]) ++n;
        gp(p.accepted)[tid] = n;
      }
    }
  }
  if (kTrace && p.trace) {  // the last record, and one more holding the time the workgroup finished the step
    __syncthreads();
    const int lane = tid_x();
    if (lane < kTraceStamps)
      gp(p.trace)[((size_t)(gen - 1) * gridDim.x + blockIdx.x) * kTraceStamps + lane] =
          ((LdsU64*)sm.stamps)[((gen - 1) & 1) * kTraceStamps + lane];
    const uint64_t now = wall_clock64();
    if (lane < kTraceStamps) gp(p.trace)[((size_t)gen * gridDim.x + blockIdx.x) * kTraceStamps + lane] = now;
  }
}

// words [0, n) of p to zero (the static workspace's barrier flags and status before a step: a fill
// kernel, not a memset, so that a caller may capture the step in a graph)
__global__ void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + tid_x(); i < n; i += gridDim.x * blockDim.x) gp(p)[i] = 0u;
}

// W_uk [h][nope][kv_lora] -> W_ukT [h][kv_lora][nope]
__global__ void transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl) {
  const size_t n = (size_t)nh * nd * kvl;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + tid_x(); e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t h = e / ((size_t)nd * kvl), r = e - h * nd * kvl, i = r / kvl, j = r - i * kvl;
    gp(dst)[(h * kvl + j) * nd + i] = gp(src)[e];
  }
}

// The router of one MoE layer folded onto its attention output projection. The router logit of the
// MoE input x' = x + W_o o before the norm's factor is sum over t of W_r[e][t] g[t] x'[t]
// = sum_t (W_r[e][t] g[t]) x[t] + sum_j (sum_t W_r[e][t] g[t] W_o[t][j]) o[j]. Row e of out holds
// the two coefficient vectors, [H] then [K]: the products of two bf16 values (exact in fp32), and the
// sums over t accumulated in fp64 and rounded once to fp32. One thread per output element.
__global__ void fold_router(const uint16_t* wr, const uint16_t* gain, const uint16_t* wo, float* out, int E, int H,
                            int K) {
  const int W = H + K;
  const size_t n = (size_t)E * W;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + tid_x(); e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t i = e / W, c = e - i * W;
    const uint16_t* w = wr + i * H;
    if (c < (size_t)H) {
      gp(out)[e] = bf2f(gp(w)[c]) * bf2f(gp(gain)[c]);
    } else {
      const size_t j = c - H;
      double acc = 0.0;
      for (int t = 0; t < H; ++t)
        acc += (double)(bf2f(gp(w)[t]) * bf2f(gp(gain)[t])) * (double)bf2f(gp(wo)[(size_t)t * K + j]);
      gp(out)[e] = (float)acc;
    }
  }
}

}  // namespace

// The workspace of mk_decode_step_static: one copy of this array on every GPU the library runs on.
// In host code `scratch` only names the symbol; its device address (a different one on every GPU)
// comes from hipGetSymbolAddress with that GPU current, and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace mk {

// The device address of `scratch` on `device`, looked up once per device (with that device
// current) and kept for the life of the process.
hipError_t static_scratch(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipSetDevice(device);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = hipSetDevice(cur);
    if (e == hipSuccess) e = back;
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[device] = ptr;
  }
  *out = addr[device];
  return hipSuccess;
}

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(clear_words, dim3(1), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

bool device_trace_built() { return kTrace; }

size_t kernel_lds_bytes() { return sizeof(Smem) + sizeof(Params); }
int max_grid() { return kMaxGrid; }

// the instance for the model's attention family
template <int MM, bool MF>
hipError_t launch_family(const Params& p, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.family == MK_ATTN_GQA)
    hipLaunchKernelGGL((mk_decode_kernel<MM, MF, MK_ATTN_GQA>), grid, block, 0, stream, p);
  else if (p.family == MK_ATTN_MLA)
    hipLaunchKernelGGL((mk_decode_kernel<MM, MF, MK_ATTN_MLA>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((mk_decode_kernel<MM, MF, MK_ATTN_HYBRID>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const Params& p, int nblocks, bool matrix_cores, hipStream_t stream) {
  const int mm = p.M <= 1 ? 1 : p.M <= 2 ? 2 : p.M <= 4 ? 4 : p.M <= 8 ? 8 : 16;
  const dim3 grid(nblocks), block(kThreads);
#ifdef MK_ONLY_MM1
  if (mm != 1) return hipErrorNotSupported;
  (void)matrix_cores;
  return launch_family<1, false>(p, grid, block, stream);
#else
  if (matrix_cores && mm >= 2) {
    switch (mm) {
      case 2: return launch_family<2, true>(p, grid, block, stream);
      case 4: return launch_family<4, true>(p, grid, block, stream);
      case 8: return launch_family<8, true>(p, grid, block, stream);
      default: return launch_family<16, true>(p, grid, block, stream);
    }
  }
  switch (mm) {
    case 1: return launch_family<1, false>(p, grid, block, stream);
    case 2: return launch_family<2, false>(p, grid, block, stream);
    case 4: return launch_family<4, false>(p, grid, block, stream);
    case 8: return launch_family<8, false>(p, grid, block, stream);
    default: return launch_family<16, false>(p, grid, block, stream);
  }
#endif
}

hipError_t launch_transpose_uk(const uint16_t* src, uint16_t* dst, int nh, int nd, int kvl, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_uk, dim3(256), dim3(256), 0, stream, src, dst, nh, nd, kvl);
  return hipGetLastError();
}

hipError_t launch_fold_router(const uint16_t* router, const uint16_t* gain, const uint16_t* wo, float* out, int E, int H,
                              int K, hipStream_t stream) {
  hipLaunchKernelGGL(fold_router, dim3(1024), dim3(256), 0, stream, router, gain, wo, out, E, H, K);
  return hipGetLastError();
}

hipError_t occupancy(int* blocks_per_cu) {
#ifdef MK_ONLY_MM1
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mk_decode_kernel<1, false, MK_ATTN_HYBRID>, kThreads, 0);
#else
  int n[6] = {0, 0, 0, 0, 0, 0};
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[0], mk_decode_kernel<16, false, MK_ATTN_GQA>, kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[1], mk_decode_kernel<16, true, MK_ATTN_GQA>, kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[2], mk_decode_kernel<16, false, MK_ATTN_MLA>, kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[3], mk_decode_kernel<16, true, MK_ATTN_MLA>, kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[4], mk_decode_kernel<16, false, MK_ATTN_HYBRID>, kThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[5], mk_decode_kernel<16, true, MK_ATTN_HYBRID>, kThreads, 0);
  int m = n[0];
  for (int k = 1; k < 6; ++k) m = n[k] < m ? n[k] : m;
  *blocks_per_cu = m;
  return e;
#endif
}

}  // namespace mk
