// Device-side helpers for the gfx950 kernels: bfloat16 conversion, wave64
// reductions, wait-count encoding.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace lla {

constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 <-> float32.  bf16 -> f32 is exact (a 16-bit shift); f32 -> bf16
// is the hardware conversion (v_cvt_pk_bf16_f32): round to nearest, ties to
// even, NaN stays NaN.  Branch-free, two values per instruction when packed.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// bf16(lo) | bf16(hi) << 16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// Element access for the two storage types.
struct bf16_t {
  uint16_t bits;
};
__device__ __forceinline__ float load_elem(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i].bits);
}
__device__ __forceinline__ void store_elem(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(bf16_t *p, int64_t i, float v) {
  p[i].bits = f32_to_bf16_bits(v);
}

// wave64 butterfly reductions (every lane receives the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroup barrier for LDS data: a wave waits for its own LDS operations
// (lgkmcnt) before the barrier, but not for outstanding global loads or
// global-to-LDS transfers, which a __syncthreads() fence would also wait
// for; the signal fences keep the compiler from moving memory accesses
// across the barrier.
constexpr int kWaitLgkmOnly = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and does not wait on the other counters (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int waitcnt_vm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

}  // namespace lla
