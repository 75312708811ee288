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


// Transposing LDS reads (ds_read_b64_tr_b16) issued together, with the wait
// for them in the same asm block.  Within each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4 e (e =
// 0..3).  The builtin form of this read makes the compiler wait for every
// outstanding LDS-direct load (buffer_load ... lds) before it, because it
// cannot tell which LDS bytes those loads write; in a kernel that keeps a
// ring of such loads in flight, that wait would drain the ring at every
// read.  The caller's own vmcnt waits and barriers guarantee that the bytes
// read here have landed.  out[i] = the read at LDS byte address a[i].
typedef short tr_short4_t __attribute__((ext_vector_type(4)));
template <int K>
__device__ __forceinline__ void lds_read_tr16_b64(const uint32_t (&a)[K], tr_short4_t (&out)[K]) {
  static_assert(K >= 1 && K <= 10, "1 to 10 reads per block");
  if constexpr (K == 1)
    asm volatile("ds_read_b64_tr_b16 %0, %1\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0])
                 : "v"(a[0])
                 : "memory");
  else if constexpr (K == 2)
    asm volatile("ds_read_b64_tr_b16 %0, %2\nds_read_b64_tr_b16 %1, %3\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1])
                 : "v"(a[0]), "v"(a[1])
                 : "memory");
  else if constexpr (K == 3)
    asm volatile("ds_read_b64_tr_b16 %0, %3\nds_read_b64_tr_b16 %1, %4\nds_read_b64_tr_b16 %2, %5\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2])
                 : "memory");
  else if constexpr (K == 4)
    asm volatile("ds_read_b64_tr_b16 %0, %4\nds_read_b64_tr_b16 %1, %5\nds_read_b64_tr_b16 %2, %6\nds_read_b64_tr_b16 %3, %7\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                 : "memory");
  else if constexpr (K == 5)
    asm volatile("ds_read_b64_tr_b16 %0, %5\nds_read_b64_tr_b16 %1, %6\nds_read_b64_tr_b16 %2, %7\nds_read_b64_tr_b16 %3, %8\nds_read_b64_tr_b16 %4, %9\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
                 : "memory");
  else if constexpr (K == 6)
    asm volatile("ds_read_b64_tr_b16 %0, %6\nds_read_b64_tr_b16 %1, %7\nds_read_b64_tr_b16 %2, %8\nds_read_b64_tr_b16 %3, %9\nds_read_b64_tr_b16 %4, %10\nds_read_b64_tr_b16 %5, %11\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
                 : "memory");
  else if constexpr (K == 7)
    asm volatile("ds_read_b64_tr_b16 %0, %7\nds_read_b64_tr_b16 %1, %8\nds_read_b64_tr_b16 %2, %9\nds_read_b64_tr_b16 %3, %10\nds_read_b64_tr_b16 %4, %11\nds_read_b64_tr_b16 %5, %12\nds_read_b64_tr_b16 %6, %13\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6])
                 : "memory");
  else if constexpr (K == 8)
    asm volatile("ds_read_b64_tr_b16 %0, %8\nds_read_b64_tr_b16 %1, %9\nds_read_b64_tr_b16 %2, %10\nds_read_b64_tr_b16 %3, %11\nds_read_b64_tr_b16 %4, %12\nds_read_b64_tr_b16 %5, %13\nds_read_b64_tr_b16 %6, %14\nds_read_b64_tr_b16 %7, %15\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                 : "memory");
  else if constexpr (K == 9)
    asm volatile("ds_read_b64_tr_b16 %0, %9\nds_read_b64_tr_b16 %1, %10\nds_read_b64_tr_b16 %2, %11\nds_read_b64_tr_b16 %3, %12\nds_read_b64_tr_b16 %4, %13\nds_read_b64_tr_b16 %5, %14\nds_read_b64_tr_b16 %6, %15\nds_read_b64_tr_b16 %7, %16\nds_read_b64_tr_b16 %8, %17\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7]), "=&v"(out[8])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8])
                 : "memory");
  else if constexpr (K == 10)
    asm volatile("ds_read_b64_tr_b16 %0, %10\nds_read_b64_tr_b16 %1, %11\nds_read_b64_tr_b16 %2, %12\nds_read_b64_tr_b16 %3, %13\nds_read_b64_tr_b16 %4, %14\nds_read_b64_tr_b16 %5, %15\nds_read_b64_tr_b16 %6, %16\nds_read_b64_tr_b16 %7, %17\nds_read_b64_tr_b16 %8, %18\nds_read_b64_tr_b16 %9, %19\ns_waitcnt lgkmcnt(0)"
                 : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7]), "=&v"(out[8]), "=&v"(out[9])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9])
                 : "memory");
}

}  // namespace lla
