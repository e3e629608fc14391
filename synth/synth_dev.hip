// synth_dev.hip -- device implementation of the seeded input generator defined in synth.h.
// It fills device buffers directly so that hundreds of GB of synthetic weights never cross
// PCIe. Every step is integer arithmetic plus one fp32 multiply, so the results equal the
// host implementation bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ int32_t ih(uint64_t key, uint64_t i) {
  uint64_t r = mix64(key + (i + 1) * kGolden);
  int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) + (int32_t)((r >> 32) & 0xFFFF) +
              (int32_t)((r >> 48) & 0xFFFF);
  return s - 131070;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_normal_bf16(uint64_t key, float scale, uint64_t off, uint64_t n, uint16_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = to_bf16(__fmul_rn((float)ih(key, off + j), scale));
}

__global__ void fill_normal_f32(uint64_t key, float scale, uint64_t off, uint64_t n, float* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = __fmul_rn((float)ih(key, off + j), scale);
}

int launch_dims(uint64_t n) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) blocks = 1;
  return (int)blocks;
}

}  // namespace

extern "C" {

// Fill n bf16 values of stream `key` (elements off .. off+n-1) into device memory d_out.
// Returns 0 on success, otherwise the hipError_t of the launch.
int synth_dev_normal_bf16(uint64_t key, float scale, uint64_t off, uint64_t n, void* d_out, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_normal_bf16, dim3(launch_dims(n)), dim3(256), 0, (hipStream_t)stream, key, scale, off, n,
                     (uint16_t*)d_out);
  return (int)hipGetLastError();
}

// Same definition with fp32 output (used for the recurrent state of linear-attention layers).
int synth_dev_normal_f32(uint64_t key, float scale, uint64_t off, uint64_t n, void* d_out, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_normal_f32, dim3(launch_dims(n)), dim3(256), 0, (hipStream_t)stream, key, scale, off, n,
                     (float*)d_out);
  return (int)hipGetLastError();
}

}  // extern "C"
