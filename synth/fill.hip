// Device side of the counter-based synthetic generator of synth/gen.py
// (hash_normal): element i of stream `key` is SplitMix64 (Steele, Lea &
// Flood, OOPSLA 2014) at counter i, mapped to the Irwin-Hall sum of twelve
// 5-bit fields, (sum - 186) / 32, then multiplied by `scale` in float32 and
// stored as float32 or bfloat16 (nearest, ties to even).  Holds no LLA
// arithmetic; it only fills multi-GB input buffers on the device.
//
// Also here, for the benchmark's context figures: a plain streaming-read
// kernel (synth_read_stream) and a register-only matrix-core kernel
// (synth_mfma_spin), the practical HBM and bf16 MFMA ceilings the decode
// kernels are compared with, and a kernel that measures how far the matrix
// cores and the vector ALU of one SIMD overlap (synth_mfma_valu_overlap).
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

// Streaming read of n16 16-byte words.  Workgroup g walks the contiguous
// range [g * per, (g + 1) * per); each thread keeps 8 nontemporal 16-byte
// loads in flight and folds what it read with XOR.  A thread writes its fold
// only if it equals a fixed pattern (practically never, but the compiler
// cannot drop the loads), so the kernel's traffic is the read alone.
constexpr int kReadUnroll = 8;
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_stream(const u32x4_v *src, int64_t n16, int64_t per,
                                                    u32x4_v *sink) {
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (kReadUnroll - 1) * 256 < b1; i += 256 * kReadUnroll) {
    u32x4_v v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      a0 ^= v[u].x;
      a1 ^= v[u].y;
      a2 ^= v[u].z;
      a3 ^= v[u].w;
    }
  }
  for (; i < b1; i += 256) {  // the tail of the last workgroup's range
    const u32x4_v v = __builtin_nontemporal_load(src + i);
    a0 ^= v.x;
    a1 ^= v.y;
    a2 ^= v.z;
    a3 ^= v.w;
  }
  if ((a0 ^ a1 ^ a2 ^ a3) == 0x9E3779B9u)
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = u32x4_v{a0, a1, a2, a3};
}

// Streaming write (src null) or copy of n16 16-byte words in chunks of
// 2048 words (one unrolled round of a workgroup): workgroup g takes chunks
// g, g + grid, g + 2 grid, ..., so that the chunks in flight at any time are
// neighbours in memory; eight 16-byte stores per thread in flight (loads of
// a copy nontemporal).  The write and read-plus-write ceilings the
// write-bound kernels are compared with.
__global__ __launch_bounds__(256) void write_stream(const u32x4_v *src, u32x4_v *dst,
                                                     int64_t n16) {
  const u32x4_v pat = {0x3F803F80u, 0x3F803F80u, (uint32_t)blockIdx.x, threadIdx.x};
  const int64_t chunk = 256 * kReadUnroll;
  for (int64_t c0 = (int64_t)blockIdx.x * chunk; c0 < n16; c0 += (int64_t)gridDim.x * chunk) {
    const int64_t i = c0 + threadIdx.x;
    if (c0 + chunk <= n16) {
      u32x4_v v[kReadUnroll];
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u)
        v[u] = src ? __builtin_nontemporal_load(src + i + u * 256) : pat;
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) dst[i + u * 256] = v[u];
    } else {
      for (int64_t k = i; k < n16; k += 256) dst[k] = src ? src[k] : pat;
    }
  }
}

// Matrix-core ceiling: every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 accumulations on operands held in registers (no
// memory traffic), then writes its sum only if it equals a fixed pattern.
typedef short bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void mfma_spin(int iters, float *sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  bf16x8_v a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (short)(0x3F80 + ((lane + e) & 7));  // bf16 values near 1
    b[e] = (short)(0x3C00 + ((lane * 3 + e) & 7));
  }
  f32x16_v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) t += c0[k] + c1[k] + c2[k] + c3[k];
  if (t == 1234.5f) sink[blockIdx.x * 256 + threadIdx.x] = t;
#endif
}

// Overlap of the two pipes of a SIMD: 512-thread workgroups, waves w and
// w + 4 share a SIMD.  mode bit 0: waves 0-3 run the register-only MFMA
// rounds of mfma_spin; mode bit 1: waves 4-7 run 32 fp32 FMAs per round
// (eight independent chains, one wave64 v_fma per instruction).
__global__ __launch_bounds__(512) void mfma_valu_overlap(int iters, int mode, float *sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float t = 0.f;
  if ((mode & 1) && wave < 4) {
    bf16x8_v a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (short)(0x3F80 + ((lane + e) & 7));
      b[e] = (short)(0x3C00 + ((lane * 3 + e) & 7));
    }
    f32x16_v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) t += c0[k] + c1[k] + c2[k] + c3[k];
  }
  if ((mode & 2) && wave >= 4) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 1.0f + 1e-7f * (float)(lane + e);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int rep = 0; rep < 4; ++rep)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(x[e], 0.999999f, 1e-7f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t += x[e];
  }
  if (t == 1234.5f) sink[blockIdx.x * 512 + threadIdx.x] = t;
#endif
}

}  // namespace

// Launches the overlap kernel: `blocks` workgroups of eight waves; see
// mfma_valu_overlap for `mode`.  sink holds blocks * 512 floats.
extern "C" int synth_mfma_valu_overlap(int32_t blocks, int32_t iters, int32_t mode, float *sink,
                                       hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || mode < 1 || mode > 3) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_valu_overlap, dim3((unsigned)blocks), dim3(512), 0, stream, iters, mode,
                     sink);
  return (int)hipGetLastError();
}

// Launches the matrix-core ceiling kernel: `blocks` workgroups of four waves,
// each wave 4 * iters MFMAs of 32x32x16 (32768 flop each).
extern "C" int synth_mfma_spin(int32_t blocks, int32_t iters, float *sink, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_spin, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from src with `blocks` workgroups of 256
// threads; sink holds blocks * 256 16-byte words.  Returns a hipError_t value.
extern "C" int synth_read_stream(const void *src, int64_t bytes, int32_t blocks, void *sink,
                                 hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  // whole unrolled rounds per workgroup (2048 words), so that only the last
  // range has a tail
  const int64_t round = 256 * kReadUnroll;
  const int64_t per = ((n16 + blocks - 1) / blocks + round - 1) / round * round;
  hipLaunchKernelGGL(read_stream, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_v *)src, n16, per, (u32x4_v *)sink);
  return (int)hipGetLastError();
}

// Writes `bytes` (a multiple of 16) to dst, copied from src or, with src
// null, a fixed pattern, with `blocks` workgroups of 256 threads.  Returns a
// hipError_t value.
extern "C" int synth_write_stream(const void *src, void *dst, int64_t bytes, int32_t blocks,
                                  hipStream_t stream) {
  if (!dst || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(write_stream, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_v *)src, (u32x4_v *)dst, bytes / 16);
  return (int)hipGetLastError();
}

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
