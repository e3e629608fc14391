// mk_stream.hip -- read-bandwidth probe (include/mk_stream.h): one pass over a buffer with one of the
// megakernel's load kinds. Not part of the decode path; the benchmark states the megakernel's
// bandwidth against it and calibrates the hardware traffic counters with it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk_stream.h"

#define GLOBAL __attribute__((address_space(1)))

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* LdsPtr;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                          // 16-byte loads per thread and tile
constexpr uint64_t kTile = kThreads * kUnroll * 16;  // 16 KiB per workgroup and tile
constexpr int kCoherent = 16;                       // device-scope cache policy of the buffer loads

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Tile t is read by workgroup t % gridDim.x; thread i reads 16 bytes at i*16 + u*4096 of the tile.
template <int KIND>
__global__ void __launch_bounds__(kThreads) stream_read(const unsigned char* buf, uint64_t ntiles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kTile / 4];
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const unsigned char* base = buf + t * kTile;
    if constexpr (KIND == MK_STREAM_WEIGHTS || KIND == MK_STREAM_CACHED) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const GLOBAL u32x4* q = (const GLOBAL u32x4*)(base + (uint64_t)u * kThreads * 16 + tid * 16);
        v[u] = KIND == MK_STREAM_WEIGHTS ? __builtin_nontemporal_load(q) : *q;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    } else {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0, (int)kTile, 0x00020000);
      if constexpr (KIND == MK_STREAM_COHERENT) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * kThreads * 16 + tid * 16), 0, kCoherent);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
      } else {  // memory-to-LDS copies: a wave instruction moves 64 lanes x 16 bytes to consecutive LDS
        const int w = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t off = (uint32_t)(u * kThreads * 16 + w * 1024);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(lds + off / 4), 16, off + lane * 16, 0, 0, kCoherent);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        acc ^= lds[tid];
        __syncthreads();
      }
    }
  }
  if (tid == 0) sink[blockIdx.x & 4095] = acc;
  else if (acc == 0x9E3779B9u) sink[(blockIdx.x + tid) & 4095] = acc;  // keeps every lane's loads live
}

}  // namespace

extern "C" int mk_stream_read(const void* d_buf, uint64_t bytes, int kind, uint32_t* d_sink, void* hip_stream) {
  if (!d_buf || !d_sink || (reinterpret_cast<uintptr_t>(d_buf) & 255) || bytes == 0 || bytes % kTile ||
      bytes > (1ull << 40) || kind < 0 || kind > 3)
    return -1;
  const uint64_t ntiles = bytes / kTile;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -5;
  // eight workgroups per CU stay resident (LDS 16 KiB each); each walks its tiles in grid strides
  const uint64_t want = (uint64_t)cus * 8;
  const dim3 grid((unsigned)(ntiles < want ? ntiles : want)), block(kThreads);
  const unsigned char* b = static_cast<const unsigned char*>(d_buf);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (kind == MK_STREAM_WEIGHTS)
    hipLaunchKernelGGL(stream_read<MK_STREAM_WEIGHTS>, grid, block, 0, s, b, ntiles, d_sink);
  else if (kind == MK_STREAM_COHERENT)
    hipLaunchKernelGGL(stream_read<MK_STREAM_COHERENT>, grid, block, 0, s, b, ntiles, d_sink);
  else if (kind == MK_STREAM_CACHED)
    hipLaunchKernelGGL(stream_read<MK_STREAM_CACHED>, grid, block, 0, s, b, ntiles, d_sink);
  else
    hipLaunchKernelGGL(stream_read<MK_STREAM_TO_LDS>, grid, block, 0, s, b, ntiles, d_sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
