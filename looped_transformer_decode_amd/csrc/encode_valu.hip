// Append-time encoder, c = (x - mu) W_down ("Looped Latent Attention:
// Cross-Loop KV Compression for Looped Transformers", Sec. 3 Eq. 2), for
// every new token, stored head and axis, written at the token's slot.
//
// One workgroup computes a 16-row x r block of latents of one (stored head,
// axis).  The stacked length K = T*width is walked in chunks of 128: the
// centred rows (x - mu, float32) and the W_down chunk are staged in LDS,
// each thread accumulates up to eight outputs in float32, and the result is
// rounded once to the store type (nearest, ties to even).
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace detail {

constexpr int kRows = 16;
constexpr int kKc = 128;
constexpr int kThreads = 256;
constexpr int kMaxR = 128;
constexpr int kOut = kRows * kMaxR / kThreads;  // outputs per thread (8)

template <typename E>
__global__ __launch_bounds__(kThreads) void encode_valu(EncodeParams p) {
  const int axis = blockIdx.z, hs = blockIdx.y, row0 = blockIdx.x * kRows;
  const int tid = threadIdx.x;
  const int M = p.B * p.n_new;
  const int r = axis ? p.rv : p.rk;
  const int K = p.K;
  __shared__ float xs[kRows][kKc + 1];
  __shared__ float wc[kKc * kMaxR];

  const E *x = reinterpret_cast<const E *>(p.x[axis]);
  const E *wd = reinterpret_cast<const E *>(p.wd[axis]) + (int64_t)hs * K * r;
  const float *mu = p.mu[axis] + (int64_t)hs * K;

  float acc[kOut];
#pragma unroll
  for (int o = 0; o < kOut; ++o) acc[o] = 0.f;

  for (int kc = 0; kc < K; kc += kKc) {
    const int kn = min(kKc, K - kc);
    for (int i = tid; i < kRows * kKc; i += kThreads) {
      const int rr = i / kKc, kk = i % kKc;
      const int row = row0 + rr;
      float v = 0.f;
      if (row < M && kk < kn)
        v = load_elem(x, ((int64_t)row * p.Hs + hs) * K + kc + kk) - mu[kc + kk];
      xs[rr][kk] = v;
    }
    for (int i = tid; i < kKc * r; i += kThreads) {
      const int kk = i / r;
      wc[i] = (kk < kn) ? load_elem(wd, (int64_t)(kc + kk) * r + (i % r)) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
      const int oi = tid + o * kThreads;
      if (oi < kRows * r) {
        const int rr = oi / r, k = oi % r;
        float a = acc[o];
        for (int kk = 0; kk < kn; ++kk) a = fmaf(xs[rr][kk], wc[kk * r + k], a);
        acc[o] = a;
      }
    }
    __syncthreads();
  }

  E *store = reinterpret_cast<E *>(p.store);
#pragma unroll
  for (int o = 0; o < kOut; ++o) {
    const int oi = tid + o * kThreads;
    if (oi >= kRows * r) continue;
    const int rr = oi / r, k = oi % r;
    const int row = row0 + rr;
    if (row >= M) continue;
    const int b = row / p.n_new, jn = row % p.n_new;
    const int64_t slot = (int64_t)p.start[b] + jn;  // start is caller data
    if (slot < 0 || slot >= p.N) continue;
    const int64_t off = ((((int64_t)b * p.D + p.layer) * p.N + slot) * p.Hs + hs) * p.R +
                        (axis ? p.rk : 0) + k;
    store_elem(store, off, acc[o]);
  }
}

}  // namespace detail

using namespace detail;

hipError_t launch_encode_valu(const EncodeParams &p, int dtype, hipStream_t st) {
  const int M = p.B * p.n_new;
  dim3 grid((M + kRows - 1) / kRows, p.Hs, 2);
  if (dtype == LLA_DT_F32)
    hipLaunchKernelGGL(encode_valu<float>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(encode_valu<bf16_t>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace lla
