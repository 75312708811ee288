// Device side of the counter-based synthetic generator of synth/gen.py
// (hash_normal): element i of stream `key` is SplitMix64 (Steele, Lea &
// Flood, OOPSLA 2014) at counter i, mapped to the Irwin-Hall sum of twelve
// 5-bit fields, (sum - 186) / 32, then multiplied by `scale` in float32 and
// stored as float32 or bfloat16 (nearest, ties to even).  Holds no LLA
// arithmetic; it only fills multi-GB input buffers on the device.
#include <cstdint>

#include <hip/hip_runtime.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float hash_value(uint64_t key, uint64_t i) {
  const uint64_t z = mix64(key + (i + 1ull) * 0x9E3779B97F4A7C15ull);
  int s = 0;
#pragma unroll
  for (int f = 0; f < 12; ++f) s += (int)((z >> (5 * f)) & 31ull);
  return (float)(s - 186) * 0.03125f;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_bf16(uint16_t *dst, int64_t n, uint64_t key, int64_t first, float scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = to_bf16(hash_value(key, (uint64_t)(first + i)) * scale);
}

__global__ void fill_f32(float *dst, int64_t n, uint64_t key, int64_t first, float scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = hash_value(key, (uint64_t)(first + i)) * scale;
}

}  // namespace

// dtype 0: float32, 1: bfloat16.  Returns a hipError_t value.
extern "C" int synth_fill(void *dst, int64_t n, int32_t dtype, uint64_t key, int64_t first,
                          float scale, hipStream_t stream) {
  if (n <= 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (dtype == 1)
    hipLaunchKernelGGL(fill_bf16, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint16_t *)dst, n, key, first, scale);
  else
    hipLaunchKernelGGL(fill_f32, dim3((unsigned)blocks), dim3(256), 0, stream, (float *)dst, n,
                       key, first, scale);
  return (int)hipGetLastError();
}
