// Generic (VALU) decode path and the split-merge kernel shared by all paths.
//
// decode_valu_split follows the paper's formulation literally, one slot per
// thread: reconstruct the loop-t key of the slot (Eq. 3 of "Looped Latent
// Attention: Cross-Loop KV Compression for Looped Transformers", Sec. 3),
// rotate it at the slot's position ("RoPE and reconstruction"), dot it with
// the rotated query, and fold the slot into an online softmax.  Values stay
// in latent space: the weights sum to one, so sum_j p_j (W c_j + mu) equals
// W (sum_j p_j c_j) + mu, and the merge kernel applies W_up,v,t and mu_v,t
// once per (sequence, head).  It serves float32 stores and every shape the
// MFMA path does not cover.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace detail {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <typename E, int RKM>
__global__ __launch_bounds__(kThreads) void decode_valu_split(DecodeParams p) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int d = p.d, half = d / 2, rk = p.rk, rv = p.rv;

  extern __shared__ float smem[];
  float *Wk = smem;                  // [d][rk]
  float *muk = Wk + d * rk;          // [d]
  float *qr = muk + d;               // [d] rotated query * scale * log2(e)
  float *pj = qr + d;                // [kThreads] weights of the current chunk
  float *red = pj + kThreads;        // [2 * kWaves]

  const int pos = min(max(p.pos[b], 0), p.N - 1);
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, pos + 1);
  float *part = p.ws + ((int64_t)(b * p.H + h) * p.S + s) * (rv + 2);
  if (t0 >= t1) {  // split entirely after the query: an empty partial
    for (int r = tid; r < rv + 2; r += kThreads) part[r] = (r == 0) ? -INFINITY : 0.f;
    return;
  }

  const E *wk = reinterpret_cast<const E *>(p.wk) + (int64_t)h * d * rk;
  for (int i = tid; i < d * rk; i += kThreads) Wk[i] = load_elem(wk, i);
  for (int i = tid; i < d; i += kThreads) muk[i] = p.muk[(int64_t)h * d + i];
  const float *qb = p.q + ((int64_t)b * p.H + h) * d;
  const float *rq = p.rope_f32 + (int64_t)pos * d;  // [d/2][2] at the query position
  for (int i = tid; i < half; i += kThreads) {
    const float c = rq[2 * i], sn = rq[2 * i + 1];
    const float a = qb[i], bb = qb[i + half];
    qr[i] = (a * c - bb * sn) * p.scale_log2;
    qr[i + half] = (a * sn + bb * c) * p.scale_log2;
  }
  __syncthreads();

  const E *slab = reinterpret_cast<const E *>(p.store) +
                  ((int64_t)b * p.D + p.layer) * p.N * p.Hs * p.R;
  const int hs = (p.Hs == 1) ? 0 : h;
  const int wave = tid >> 6, lane = tid & 63;

  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;  // acc: V-latent component r = tid
  for (int c0 = t0; c0 < t1; c0 += kThreads) {
    const int j = c0 + tid;
    float sc = -INFINITY;
    if (j < t1) {
      const E *lat = slab + ((int64_t)j * p.Hs + hs) * p.R;
      float ck[RKM];
#pragma unroll
      for (int k = 0; k < RKM; ++k) ck[k] = (k < rk) ? load_elem(lat, k) : 0.f;
      const float *rj = p.rope_f32 + (int64_t)j * d;
      float dot = 0.f;
      for (int i = 0; i < half; ++i) {
        float ka = muk[i], kb = muk[i + half];
        const float *wa = Wk + i * rk, *wb = Wk + (i + half) * rk;
#pragma unroll
        for (int k = 0; k < RKM; ++k) {
          if (k < rk) {
            ka = fmaf(wa[k], ck[k], ka);
            kb = fmaf(wb[k], ck[k], kb);
          }
        }
        const float c = rj[2 * i], sn = rj[2 * i + 1];
        dot = fmaf(qr[i], ka * c - kb * sn, dot);
        dot = fmaf(qr[i + half], ka * sn + kb * c, dot);
      }
      sc = dot;
    }
    // block-wide max of the chunk
    float wm = wave_max(sc);
    if (lane == 0) red[wave] = wm;
    __syncthreads();
    float cm = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) cm = fmaxf(cm, red[w]);
    const float m_new = fmaxf(m_run, cm);
    const float pe = (j < t1) ? exp2f(sc - m_new) : 0.f;
    pj[tid] = pe;
    float ws_ = wave_sum(pe);
    if (lane == 0) red[kWaves + wave] = ws_;
    __syncthreads();
    float lc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) lc += red[kWaves + w];
    const float f = exp2f(m_run - m_new);  // 0 on the first chunk
    l_run = l_run * f + lc;
    m_run = m_new;
    if (tid < rv) {
      const int n = min(kThreads, t1 - c0);
      const E *cv = slab + ((int64_t)c0 * p.Hs + hs) * p.R + rk + tid;
      const int64_t stride = (int64_t)p.Hs * p.R;
      float a = acc * f;
      for (int jj = 0; jj < n; ++jj) a = fmaf(pj[jj], load_elem(cv, jj * stride), a);
      acc = a;
    }
    __syncthreads();
  }
  if (tid == 0) {
    part[0] = m_run;
    part[1] = l_run;
  }
  if (tid < rv) part[2 + tid] = acc;
}

// Merge the context splits of one (sequence, head) by log-sum-exp and apply
// the loop-t value up-projection once: out = W_up,v,t (A / L) + mu_v,t.
template <typename E>
__global__ __launch_bounds__(256) void decode_merge(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int rv = p.rv, d = p.d, S = p.S;
  extern __shared__ float abar[];  // [rv]
  const float *part = p.ws + (int64_t)(b * p.H + h) * S * (rv + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[s * (rv + 2)]);
  float L = 0.f;
  for (int s = 0; s < S; ++s) L += part[s * (rv + 2) + 1] * exp2f(part[s * (rv + 2)] - M);
  for (int r = tid; r < rv; r += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < S; ++s) a += part[s * (rv + 2) + 2 + r] * exp2f(part[s * (rv + 2)] - M);
    abar[r] = a / L;
  }
  __syncthreads();
  const E *wv = reinterpret_cast<const E *>(p.wv) + (int64_t)h * d * rv;
  for (int i = tid; i < d; i += blockDim.x) {
    float o = p.muv[(int64_t)h * d + i];
    const E *w = wv + (int64_t)i * rv;
    for (int r = 0; r < rv; ++r) o = fmaf(load_elem(w, r), abar[r], o);
    p.out[((int64_t)b * p.H + h) * d + i] = o;
  }
}

template <typename E, int RKM>
hipError_t launch_split(const DecodeParams &p, hipStream_t st) {
  const size_t sm = sizeof(float) * ((size_t)p.d * p.rk + 2 * p.d + kThreads + 2 * kWaves);
  dim3 grid(p.S, p.H, p.B);
  hipLaunchKernelGGL((decode_valu_split<E, RKM>), grid, dim3(kThreads), sm, st, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_split_e(const DecodeParams &p, hipStream_t st) {
  if (p.rk <= 16) return launch_split<E, 16>(p, st);
  if (p.rk <= 32) return launch_split<E, 32>(p, st);
  if (p.rk <= 64) return launch_split<E, 64>(p, st);
  return launch_split<E, 128>(p, st);
}

}  // namespace detail

using namespace detail;

hipError_t launch_decode_valu(const DecodeParams &p, int dtype, hipStream_t st) {
  return dtype == LLA_DT_F32 ? launch_split_e<float>(p, st) : launch_split_e<bf16_t>(p, st);
}

hipError_t launch_decode_merge(const DecodeParams &p, int dtype, hipStream_t st) {
  dim3 grid(p.H, p.B);
  const size_t sm = sizeof(float) * p.rv;
  if (dtype == LLA_DT_F32)
    hipLaunchKernelGGL(decode_merge<float>, grid, dim3(128), sm, st, p);
  else
    hipLaunchKernelGGL(decode_merge<bf16_t>, grid, dim3(128), sm, st, p);
  return hipGetLastError();
}

}  // namespace lla
