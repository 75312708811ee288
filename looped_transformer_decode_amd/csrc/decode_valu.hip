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
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <typename E, int RKM>
__global__ __launch_bounds__(kThreads) void decode_valu_split(DecodeParams p) {
  const int s = blockIdx.x, h = blockIdx.y, vb = blockIdx.z;  // vb: query (virtual sequence)
  const int tid = threadIdx.x;
  const int d = p.d, half = d / 2, rk = p.rk, rv = p.rv;

  extern __shared__ float smem[];
  float *Wk = smem;                  // [d][rk]
  float *muk = Wk + d * rk;          // [d]
  float *qr = muk + d;               // [d] rotated query * scale * log2(e)
  float *pj = qr + d;                // [kThreads] weights of the current chunk
  float *red = pj + kThreads;        // [2 * kWaves]

  const QuerySlot qs = query_slot(p, vb);
  const int b = qs.b, pos = qs.qpos;
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, qs.last + 1);
  float *part = p.ws + ((int64_t)(vb * p.H + h) * p.S + s) * (rv + 2);
  if (t0 >= t1) {  // split entirely after the attended slots: an empty partial
    for (int r = tid; r < rv + 2; r += kThreads) part[r] = (r == 0) ? -INFINITY : 0.f;
    return;
  }

  const E *wk = reinterpret_cast<const E *>(p.wk) + (int64_t)h * d * rk;
  for (int i = tid; i < d * rk; i += kThreads) Wk[i] = load_elem(wk, i);
  for (int i = tid; i < d; i += kThreads) muk[i] = p.muk[(int64_t)h * d + i];
  const float *qb = p.q + ((int64_t)vb * p.H + h) * d;
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

constexpr int kLoadBatch = 8;   // loads a thread issues before it waits

// Merge the context splits of every (sequence, head) by log-sum-exp and
// apply the loop-t value up-projection once: out = W_up,v,t (A / L) + mu_v,t.
// A block covers merge_heads_per_block() heads of one sequence, one thread
// per output element.  The block's time is its chain of memory round trips,
// so loads go out in batches of kLoadBatch independent ones (indexes past
// the end clamped to the last element, whose duplicates are then skipped).
template <typename E>
__global__ __launch_bounds__(256) void decode_merge(DecodeParams p) {
  const int tid = threadIdx.x, b = blockIdx.y;
  const int rv = p.rv, d = p.d, S = p.S;
  const int hpb = merge_heads_per_block(d, rv);
  const int h0 = blockIdx.x * hpb;
  extern __shared__ float abar[];  // [hpb][rv]
  for (int t = tid; t < hpb * rv; t += blockDim.x) {
    const int hl = t / rv, r = t % rv;
    if (h0 + hl >= p.H) continue;
    const float *part = p.ws + (int64_t)(b * p.H + h0 + hl) * S * (rv + 2);
    // Online over batches of splits (one batch when S <= kLoadBatch).
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int s0 = 0; s0 < S; s0 += kLoadBatch) {
      float mv[kLoadBatch], lv[kLoadBatch], av[kLoadBatch];
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const float *ps = part + min(s0 + u, S - 1) * (rv + 2);
        mv[u] = ps[0];
        lv[u] = ps[1];
        av[u] = ps[2 + r];
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u)
        if (s0 + u < S) Mb = fmaxf(Mb, mv[u]);
      if (Mb == -INFINITY) continue;  // every split so far empty
      const float g = exp2f(M - Mb);  // 0 while M is -inf
      L *= g;
      A *= g;
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        if (s0 + u < S && mv[u] != -INFINITY) {  // skip empty splits
          const float f = exp2f(mv[u] - Mb);
          L = fmaf(lv[u], f, L);
          A = fmaf(av[u], f, A);
        }
      }
      M = Mb;
    }
    abar[t] = A / L;
  }
  __syncthreads();
  const bool vec = sizeof(E) == 2 && rv % 8 == 0 && ((uintptr_t)p.wv & 15u) == 0;
  for (int o = tid; o < hpb * d; o += blockDim.x) {
    const int hl = o / d, i = o % d, h = h0 + hl;
    if (h >= p.H) continue;
    const float mu = p.muv[(int64_t)h * d + i];
    const float *ab = abar + hl * rv;
    const E *w = reinterpret_cast<const E *>(p.wv) + ((int64_t)h * d + i) * rv;
    float acc = 0.f;
    if (vec) {
      const uint4 *w4 = reinterpret_cast<const uint4 *>(w);
      const int n8 = rv / 8;
      for (int c0 = 0; c0 < n8; c0 += kLoadBatch) {
        uint4 v[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) v[u] = w4[min(c0 + u, n8 - 1)];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          if (c0 + u < n8) {
            const uint32_t uu[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            const float *a8 = ab + 8 * (c0 + u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc = fmaf(bf16_lo(uu[e]), a8[2 * e], acc);
              acc = fmaf(bf16_hi(uu[e]), a8[2 * e + 1], acc);
            }
          }
        }
      }
    } else {
      for (int r = 0; r < rv; ++r) acc = fmaf(load_elem(w, r), ab[r], acc);
    }
    p.out[((int64_t)b * p.H + h) * d + i] = acc + mu;
  }
}

// Merge for LLA-2D stores: the same log-sum-exp merge, batched over
// sequences so that each W_up,v,t head block (d x r_v) is read once per
// kBT sequences instead of once per sequence.  Block = (head, sequence
// tile); one thread per output element of the head.  As in the in-flight
// merge below, a block is a short chain of phases whose time is its number
// of round trips to memory: W_up,v,t of the head is copied to LDS at the
// start with batched 16-byte loads (rows padded to an odd number of dwords,
// so that thread i reading row i hits its own bank), and the partials are
// read in batches of kLoadBatch independent loads.
constexpr int kBT = 8;
static_assert(kBT == 8, "batched_merge_lds() sizes the LDS for tiles of 8 sequences");
constexpr int kOnePer = 8;  // partial elements per thread on the one-split path

// Copies the d x rv block of W_up,v,t at wg (16-byte aligned, rows of a
// whole number of 16-byte chunks) into LDS rows of `pitch` dwords, each
// thread issuing kBatch 16-byte loads before it waits for them.
template <typename E, int kBatch = kLoadBatch>
__device__ __forceinline__ void w_rows_to_lds(const E *wg, int d, int rv, int pitch, uint32_t *wl,
                                              int t, int nt) {
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(wg);
  const int rc = rv * (int)sizeof(E) / 16, n = d * rc;  // 16-byte chunks per row, in all
  for (int c0 = t; c0 < n; c0 += kBatch * nt) {
    u32x4_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = src[min(c0 + u * nt, n - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + u * nt;
      if (c < n) {
        uint32_t *dst = wl + (c / rc) * pitch + 4 * (c % rc);
#pragma unroll
        for (int w = 0; w < 4; ++w) dst[w] = v[u][w];
      }
    }
  }
}

// Element r of an LDS row written by w_rows_to_lds.
template <typename E>
__device__ __forceinline__ float w_lds_elem(const uint32_t *row, int r) {
  if (sizeof(E) == 4) return __uint_as_float(row[r]);
  return (r & 1) ? bf16_hi(row[r >> 1]) : bf16_lo(row[r >> 1]);
}

// G: sequence groups of the up-projection.  With G = 2 (d <= 128) the block
// has 2 d threads and thread (g, i) computes output i of the kBT / 2
// sequences of group g: twice the waves of one thread per output, which the
// chain of LDS reads and FMAs per output needs (measured at d = 128,
// r_v = 128: 15.0 -> 10.1 us per LLA-2D call; four groups 10.5 us).
template <typename E, int G>
__global__ __launch_bounds__(256) void decode_merge_batched(DecodeParams p) {
  const int h = blockIdx.x, b0 = blockIdx.y * kBT, tid = threadIdx.x, nt = blockDim.x;
  const int rv = p.rv, d = p.d, S = p.S;
  const BatchedMergeLds lay = batched_merge_lds(d, rv, S, (int)sizeof(E));
  extern __shared__ float sm[];
  float *abar = sm;                  // [kBT][rv] merged latent averages
  float *fs = abar + kBT * rv;       // [kBT][S] split weights
  float *ls = fs + kBT * S;          // [kBT] merged softmax sums
  uint32_t *wl = reinterpret_cast<uint32_t *>(sm + lay.w_off);  // [d][w_pitch] dwords
  const E *wg = reinterpret_cast<const E *>(p.wv) + (int64_t)h * d * rv;
  const bool w_vec = p.w_lds != 0 && (rv * (int)sizeof(E)) % 16 == 0 &&
                     (reinterpret_cast<uintptr_t>(wg) & 15) == 0;
  if (S == 1 && w_vec && kBT * rv <= kOnePer * nt) {
    // One split (the usual LLA-2D case): the partials this thread needs are
    // loaded together with the W_up,v,t rows, so the block waits for memory
    // once instead of once per phase.  The arithmetic is the general
    // phases' with S = 1 (weight 2^(m - m) = 1, or 0 for an empty split).
    const int na = kBT * rv;
    float mv[kOnePer], lv[kOnePer], av[kOnePer];
#pragma unroll
    for (int u = 0; u < kOnePer; ++u) {
      const int e = min(tid + u * nt, na - 1), b = min(b0 + e / rv, p.B - 1);
      const float *part = p.ws + (int64_t)(b * p.H + h) * (rv + 2);
      mv[u] = part[0];
      lv[u] = part[1];
      av[u] = part[2 + e % rv];
    }
    w_rows_to_lds<E, 2 * kLoadBatch>(wg, d, rv, lay.w_pitch, wl, tid, nt);
#pragma unroll
    for (int u = 0; u < kOnePer; ++u) {
      const int e = tid + u * nt;
      if (e >= na) continue;
      const float f = mv[u] == -INFINITY ? 0.f : exp2f(mv[u] - mv[u]);
      const float a = fmaf(av[u], f, 0.f), L = fmaf(lv[u], f, 0.f);
      abar[e] = b0 + e / rv < p.B ? a / L : 0.f;
    }
  } else {
    if (w_vec) w_rows_to_lds(wg, d, rv, lay.w_pitch, wl, tid, nt);

    // split weights 2^(m_s - M) and merged sum L of every sequence of the tile
    for (int bl = tid; bl < kBT; bl += nt) {
      const int b = b0 + bl;
      if (b >= p.B) {
        for (int s2 = 0; s2 < S; ++s2) fs[bl * S + s2] = 0.f;
        ls[bl] = 1.f;
        continue;
      }
      const float *part = p.ws + (int64_t)(b * p.H + h) * S * (rv + 2);
      float M = -INFINITY;
#pragma unroll 4
      for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, part[s2 * (rv + 2)]);
      float L = 0.f;
#pragma unroll 4
      for (int s2 = 0; s2 < S; ++s2) {
        const float ms = part[s2 * (rv + 2)];
        const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);  // empty split: weight 0
        fs[bl * S + s2] = f;
        L = fmaf(part[s2 * (rv + 2) + 1], f, L);
      }
      ls[bl] = L;
    }
    __syncthreads();
    // averages A / L; sequences past B get zeros
    const int na = kBT * rv;
    for (int e0 = tid; e0 < na; e0 += kLoadBatch * nt) {
      float a[kLoadBatch];
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) a[u] = 0.f;
      for (int s2 = 0; s2 < S; ++s2) {
        float v[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int e = min(e0 + u * nt, na - 1), b = min(b0 + e / rv, p.B - 1);
          v[u] = p.ws[(int64_t)(b * p.H + h) * S * (rv + 2) + s2 * (rv + 2) + 2 + e % rv];
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int e = min(e0 + u * nt, na - 1);
          a[u] = fmaf(v[u], fs[(e / rv) * S + s2], a[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int e = e0 + u * nt;
        if (e < na) abar[e] = b0 + e / rv < p.B ? a[u] / ls[e / rv] : 0.f;
      }
    }
  }
  __syncthreads();
  const bool vec = sizeof(E) == 2 && rv % 8 == 0 && ((uintptr_t)p.wv & 15u) == 0;
  constexpr int NBT = kBT / G;  // sequences per thread
  const int bl0 = G > 1 ? (tid / d) * NBT : 0;
  for (int i = G > 1 ? tid % d : tid; i < d; i += G > 1 ? d : nt) {
    float acc[NBT];
#pragma unroll
    for (int bq = 0; bq < NBT; ++bq) acc[bq] = 0.f;
    const E *w = wg + (int64_t)i * rv;
    if (w_vec || vec) {
      // 8 weights of the row at a time (LDS, else one 16-byte load); the 8
      // matching averages of each sequence as two 16-byte LDS reads (the
      // same address in every lane: a broadcast)
      const uint32_t *wrow = wl + i * lay.w_pitch;
      const uint4 *w4 = reinterpret_cast<const uint4 *>(w);
      for (int r8 = 0; r8 < rv / 8; ++r8) {
        float wf[8];
        if (w_vec) {
#pragma unroll
          for (int e = 0; e < 8; ++e) wf[e] = w_lds_elem<E>(wrow, 8 * r8 + e);
        } else {
          const uint4 v = w4[r8];
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wf[2 * e] = bf16_lo(u[e]);
            wf[2 * e + 1] = bf16_hi(u[e]);
          }
        }
#pragma unroll
        for (int bq = 0; bq < NBT; ++bq) {
          const int bl = bl0 + bq;
          const float4 a0 = *reinterpret_cast<const float4 *>(abar + bl * rv + 8 * r8);
          const float4 a1 = *reinterpret_cast<const float4 *>(abar + bl * rv + 8 * r8 + 4);
          float t = acc[bq];
          t = fmaf(wf[0], a0.x, t);
          t = fmaf(wf[1], a0.y, t);
          t = fmaf(wf[2], a0.z, t);
          t = fmaf(wf[3], a0.w, t);
          t = fmaf(wf[4], a1.x, t);
          t = fmaf(wf[5], a1.y, t);
          t = fmaf(wf[6], a1.z, t);
          t = fmaf(wf[7], a1.w, t);
          acc[bq] = t;
        }
      }
    } else {
      for (int r = 0; r < rv; ++r) {
        const float wf = load_elem(w, r);
#pragma unroll
        for (int bq = 0; bq < NBT; ++bq) acc[bq] = fmaf(wf, abar[(bl0 + bq) * rv + r], acc[bq]);
      }
    }
    const float mu = p.muv[(int64_t)h * d + i];
#pragma unroll
    for (int bq = 0; bq < NBT; ++bq) {
      const int b = b0 + bl0 + bq;
      if (b < p.B) p.out[((int64_t)b * p.H + h) * d + i] = acc[bq] + mu;
    }
  }
}

// Multi-query causal merge with the in-flight tokens.  For query i of
// sequence b (position pos0 + i) and head h the attended set is the store
// slots < pos0 (the split partials (m, l, sum p c_v) of that query) plus the
// in-flight tokens m <= i of the same call, whose loop-t keys and values
// exist only in full precision (their latents need all T loops, Eq. 2):
//   out = [e^(M_s - M) (W_up,v,t A + mu_v,t L_s) + sum_m e^(s_m - M) v_m]
//         / [e^(M_s - M) L_s + sum_m e^(s_m - M)],
//   s_m = scale * RoPE(q_i, pos0 + i) . RoPE(k_m, pos0 + m)   (log2 domain).
// One block per (head, sequence).  Every query's store partials are merged
// at once; each query's maximum, store factor, in-flight weights and
// denominator are formed once.  W_up,v,t is applied to the latent averages
// of all queries on the matrix cores for bf16 stores (W_up,v,t in LDS, d a
// multiple of 16), else by kQGroup queries per pass over its row: with
// R = blockDim / d whole rows of d threads, thread t < R d owns output
// element t % d of query groups t / d, t / d + R, ...
//
// The block's work is a chain of short phases, so its time is set by the
// round trips to memory in that chain.  Every phase issues its global loads
// in batches of kLoadBatch independent ones before using any, the latent
// averages are stored query-minor (the queries of a group are one 32-byte
// LDS read) with the query count padded to a whole group, and no loop over
// queries or value components holds a branch that would split its LDS reads
// into separate waits.  W_up,v,t of the head is copied to LDS when it fits,
// rows padded to an odd number of dwords so that consecutive rows start in
// different banks.
constexpr int kMaxQ = 32;       // in-flight queries per call
constexpr int kQGroup = 8;      // queries per W_up,v,t pass

// Four blocks per CU (at most 128 VGPRs, about 38 KB of LDS at 16 queries,
// d = 128, r_v = 80): the long-recurrence call's 1024 blocks then run as one
// round over the 256 CUs.
template <typename E>
__global__ __launch_bounds__(256, 4) void decode_merge_inflight(DecodeParams p, const float *k_new,
                                                            const float *v_new) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x, nt = blockDim.x;
  const int d = p.d, half = d / 2, rv = p.rv, S = p.S, nq = p.qps, H = p.H;
  const InflightMergeLds lay = inflight_merge_lds(nq, d, rv, S, (int)sizeof(E));
  const int nqp = lay.nq_pad;
  extern __shared__ float sm[];
  float *kr = sm;                 // [nq][d]  rotated in-flight keys, then their values
  float *qr = kr + nq * d;        // [nq][d]  rotated, scaled queries, until the scores
  float *abar = qr;               // [rv][nqp] store latent numerators (query-minor), after
  float *sc = qr + lay.qa_floats; // [nq][nq] in-flight scores (m <= i)
  float *st = sc + nq * nq;       // [nq][4]  store M, L; then fs, fs L, denominator
  float *wsp = st + 4 * nq;       // [nq][S]  split weights
  uint32_t *wl = reinterpret_cast<uint32_t *>(sm + lay.w_off);  // [d][lay.w_pitch] dwords
  const int first = min(max(p.pos[b], 0), p.N);
  const bool act = t < d;

  // Every global load of the first phase goes out before any is waited
  // for: the split maxima and sums of the store partials, the in-flight
  // values, the RoPE operands of the in-flight keys and queries, then
  // W_up,v,t, whose copy into LDS waits for all of them at once (measured
  // with the matrix-core sum below: 30.8 -> 29.2 us per long-recurrence call
  // for this phase, 25.8 us with both).
  const E *wg = reinterpret_cast<const E *>(p.wv) + (int64_t)h * d * rv;
  const int row_bytes = rv * (int)sizeof(E);
  const bool w_vec =
      p.w_lds != 0 && row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(wg) & 15) == 0;
  const float *part_t = p.ws + (int64_t)((b * nq + min(t, nq - 1)) * H + h) * S * (rv + 2);
  constexpr int kSPre = 2;  // splits whose (m, l) a thread holds in registers
  float pm[kSPre], pl[kSPre];
#pragma unroll
  for (int s2 = 0; s2 < kSPre; ++s2) {
    const int sc2 = min(s2, S - 1);
    pm[s2] = part_t[sc2 * (rv + 2)];
    pl[s2] = part_t[sc2 * (rv + 2) + 1];
  }
  // The in-flight values of the first kVAhead tokens (they replace the keys
  // in LDS once the scores are done).
  constexpr int kVAhead = 16;
  float vah[kVAhead];
#pragma unroll
  for (int j = 0; j < kVAhead; ++j)
    vah[j] = v_new[((int64_t)(b * nq + min(j, nq - 1)) * H + h) * d + (act ? t : 0)];
  // rotate-half RoPE of the in-flight keys and the queries at pos0 + m:
  // thread (token slot ms, pair u) forms elements u and u + d/2 of tokens
  // ms, ms + tpp, ... (kRPass of them per batch)
  constexpr int kRPass = 4;
  const int tpp = nt / half;  // tokens per pass
  const int u = t % half, ms = t / half;
  const bool ract = ms < tpp;
  float xk[kRPass], yk[kRPass], xq[kRPass], yq[kRPass], cc[kRPass], ss[kRPass];
  auto rope_load = [&](int m0) {
#pragma unroll
    for (int j = 0; j < kRPass; ++j) {
      const int m = min(m0 + ms + j * tpp, nq - 1);
      const int64_t row = ((int64_t)(b * nq + m) * H + h) * d;
      const float *cs = p.rope_f32 + (int64_t)min(first + m, p.N - 1) * d;  // [d/2][2]
      xk[j] = k_new[row + u];
      yk[j] = k_new[row + u + half];
      xq[j] = p.q[row + u];
      yq[j] = p.q[row + u + half];
      cc[j] = cs[2 * u];
      ss[j] = cs[2 * u + 1];
    }
  };
  auto rope_store = [&](int m0) {
#pragma unroll
    for (int j = 0; j < kRPass; ++j) {
      const int m = m0 + ms + j * tpp;
      if (ract && m < nq) {
        kr[m * d + u] = xk[j] * cc[j] - yk[j] * ss[j];
        kr[m * d + u + half] = yk[j] * cc[j] + xk[j] * ss[j];
        qr[m * d + u] = (xq[j] * cc[j] - yq[j] * ss[j]) * p.scale_log2;
        qr[m * d + u + half] = (yq[j] * cc[j] + xq[j] * ss[j]) * p.scale_log2;
      }
    }
  };
  rope_load(0);
  if (w_vec) w_rows_to_lds(wg, d, rv, lay.w_pitch, wl, t, nt);
  rope_store(0);
  for (int m0 = kRPass * tpp; m0 < nq; m0 += kRPass * tpp) {
    rope_load(m0);
    rope_store(m0);
  }
  // store partials of every query, merged over the splits: the split
  // weights 2^(m_s - M) of every query (the numerators follow the scores)
  for (int i = t; i < nq; i += nt) {
    const float *part = p.ws + (int64_t)((b * nq + i) * H + h) * S * (rv + 2);
    float M = -INFINITY;
    if (i == t && S <= kSPre) {
#pragma unroll
      for (int s2 = 0; s2 < kSPre; ++s2) M = s2 < S ? fmaxf(M, pm[s2]) : M;
    } else {
#pragma unroll 4
      for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, part[s2 * (rv + 2)]);
    }
    float L = 0.f;
    if (i == t && S <= kSPre) {
#pragma unroll
      for (int s2 = 0; s2 < kSPre; ++s2) {
        if (s2 < S) {
          const float w = pm[s2] == -INFINITY ? 0.f : exp2f(pm[s2] - M);
          wsp[i * S + s2] = w;
          L = fmaf(pl[s2], w, L);
        }
      }
    } else {
#pragma unroll 4
      for (int s2 = 0; s2 < S; ++s2) {
        const float msv = part[s2 * (rv + 2)];
        const float w = msv == -INFINITY ? 0.f : exp2f(msv - M);  // empty split: weight 0
        wsp[i * S + s2] = w;
        L = fmaf(part[s2 * (rv + 2) + 1], w, L);
      }
    }
    st[4 * i] = M;
    st[4 * i + 1] = L;
  }
  __syncthreads();
  // scores s[i][m], m <= i: one thread per pair, four partial sums over
  // 16-byte LDS reads (loads batched by the unrolled loop), the chunk order
  // rotated per thread so that threads of a wave read different banks
  const bool vec4 = d % 4 == 0;
  for (int pr = t; pr < nq * nq; pr += nt) {
    const int i = pr / nq, m = pr % nq;
    if (m > i) continue;
    const float *qi = qr + i * d, *km = kr + m * d;
    float v;
    if (vec4) {
      const int nc = d / 4, c0 = pr % nc;
      const float4 *q4 = reinterpret_cast<const float4 *>(qi);
      const float4 *k4 = reinterpret_cast<const float4 *>(km);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
      for (int c = 0; c < nc; ++c) {
        const int cc = c + c0 < nc ? c + c0 : c + c0 - nc;
        const float4 x = q4[cc], y = k4[cc];
        a0 = fmaf(x.x, y.x, a0);
        a1 = fmaf(x.y, y.y, a1);
        a2 = fmaf(x.z, y.z, a2);
        a3 = fmaf(x.w, y.w, a3);
      }
      v = (a0 + a1) + (a2 + a3);
    } else {
      v = 0.f;
      const int e0 = pr % d;
      for (int e = e0; e < d; ++e) v = fmaf(qi[e], km[e], v);
      for (int e = 0; e < e0; ++e) v = fmaf(qi[e], km[e], v);
    }
    sc[i * nq + m] = v;
  }
  __syncthreads();
  // the queries are done with: the store numerators of every query, merged
  // over the splits, take their place
  const int na = nqp * rv;  // padded queries get zero numerators
  for (int e0 = t; e0 < na; e0 += kLoadBatch * nt) {
    float a[kLoadBatch];
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) a[u] = 0.f;
    for (int s2 = 0; s2 < S; ++s2) {
      float v[kLoadBatch];
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int e = min(e0 + u * nt, na - 1), i = min(e / rv, nq - 1), r = e % rv;
        v[u] = p.ws[(int64_t)((b * nq + i) * H + h) * S * (rv + 2) + s2 * (rv + 2) + 2 + r];
      }
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int i = min(min(e0 + u * nt, na - 1) / rv, nq - 1);
        a[u] = fmaf(v[u], wsp[i * S + s2], a[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
      const int e = e0 + u * nt, i = e / rv, r = e % rv;
      if (e < na) abar[r * nqp + i] = i < nq ? a[u] : 0.f;
    }
  }
  // per query, once: the maximum M over the store part and its in-flight
  // scores, the store factor fs = 2^(M_s - M), the in-flight weights
  // 2^(s_m - M) in place of the scores (0 for m > i) and the denominator
  for (int i = t; i < nq; i += nt) {
    const float Ms = st[4 * i], Ls = st[4 * i + 1];
    float M = Ms;
#pragma unroll 8
    for (int m = 0; m < nq; ++m) M = m <= i ? fmaxf(M, sc[i * nq + m]) : M;
    const float fs = (Ms == -INFINITY) ? 0.f : exp2f(Ms - M);
    float den = fs * Ls;
#pragma unroll 8
    for (int m = 0; m < nq; ++m) {
      const float e = m <= i ? exp2f(sc[i * nq + m] - M) : 0.f;
      sc[i * nq + m] = e;
      den += e;
    }
    st[4 * i] = fs;
    st[4 * i + 1] = fs * Ls;
    st[4 * i + 2] = den;
  }
  // the keys are done with: stage the in-flight values instead
  if (act) {
#pragma unroll
    for (int j = 0; j < kVAhead; ++j)
      if (j < nq) kr[j * d + t] = vah[j];
    for (int m0 = kVAhead; m0 < nq; m0 += kLoadBatch) {
      float v[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j)
        v[j] = v_new[((int64_t)(b * nq + min(m0 + j, nq - 1)) * H + h) * d + t];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j)
        if (m0 + j < nq) kr[(m0 + j) * d + t] = v[j];
    }
  }
  __syncthreads();

  if constexpr (sizeof(E) == 2) {
    if (w_vec && d % 16 == 0 && d <= 256 && rv <= 128 && nt == 256) {
      // bf16 W_up,v,t in LDS: (queries x r_v) x (r_v x d) on the matrix
      // cores, v_mfma_f32_16x16x32_bf16 tiles of 16 queries x 16 output
      // elements over 32 value components (components past r_v are zero);
      // wave w takes the element tiles w, w + 4, ...  The latent averages
      // enter as a bf16 pair hi + lo (lo the rounding remainder), so the
      // products see them to about 16 mantissa bits (sums in fp32).  Lane l
      // holds A = averages of query l % 16 at components 8 (l / 16) + 0..7,
      // B = the W_up,v,t row of element l % 16 at the same components, and
      // D = queries 4 (l / 16) + 0..3 of element l % 16.
      constexpr int kMaxKs = 4;  // r_v <= 128
      const int l16 = t & 15, g = (t & 63) >> 4, wave = t >> 6;
      const int nqt = (nq + 15) / 16, nks = (rv + 31) / 32;
      float mus[4];  // mu_v,t of this lane's element in each of its tiles, fetched ahead
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mus[j] = p.muv[(int64_t)h * d + min(16 * (wave + 4 * j) + l16, d - 1)];
      for (int qt = 0; qt < nqt; ++qt) {
        bf16x8_t a[kMaxKs], alo[kMaxKs];
#pragma unroll
        for (int ks = 0; ks < kMaxKs; ++ks) {
          const int q = 16 * qt + l16, r0 = 32 * ks + 8 * g;
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = (r0 < rv && q < nqp) ? abar[(r0 + e) * nqp + q] : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t pk = pack_bf16x2(f[2 * e], f[2 * e + 1]);
            a[ks][2 * e] = (short)(pk & 0xFFFFu);
            a[ks][2 * e + 1] = (short)(pk >> 16);
            const uint32_t pr = pack_bf16x2(f[2 * e] - bf16_lo(pk), f[2 * e + 1] - bf16_hi(pk));
            alo[ks][2 * e] = (short)(pr & 0xFFFFu);
            alo[ks][2 * e + 1] = (short)(pr >> 16);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // element tiles wave + 4 j (d <= 256)
          const int et = wave + 4 * j;
          if (et >= d / 16) break;
          const int el = 16 * et + l16;
          const uint32_t *wr = wl + el * lay.w_pitch;
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < kMaxKs; ++ks) {
            if (ks >= nks) break;
            const int r0 = 32 * ks + 8 * g;
            bf16x8_t bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t pk = r0 < rv ? wr[r0 / 2 + e] : 0u;
              bw[2 * e] = (short)(pk & 0xFFFFu);
              bw[2 * e + 1] = (short)(pk >> 16);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bw, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], bw, acc, 0, 0, 0);
          }
          // sum_m w_m v_m for the tile's 16 queries and 16 elements on the
          // matrix cores (v_mfma_f32_16x16x4_f32: fp32 operands, exact
          // products): A = the weights (query l % 16, token 4 s + l / 16), B =
          // the values (token 4 s + l / 16, element l % 16); tokens past nq
          // enter as zeros.  Two LDS reads per lane and k-step, where a loop
          // per output element read both operands for every token.
          f32x4_t mix = {0.f, 0.f, 0.f, 0.f};
          {
            const int qa = min(16 * qt + l16, nq - 1);
            for (int m0 = 0; m0 < nq; m0 += 4) {
              const int m = m0 + g;
              const float wa = m < nq ? sc[qa * nq + min(m, nq - 1)] : 0.f;
              const float vb = m < nq ? kr[min(m, nq - 1) * d + el] : 0.f;
              mix = __builtin_amdgcn_mfma_f32_16x16x4f32(wa, vb, mix, 0, 0, 0);
            }
          }
          // [fs (W_up,v,t A + mu_v,t L_s) + sum_m w_m v_m] / den, w_m = 0 for m > i
          const float mu = mus[j];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int q = 16 * qt + 4 * g + i;
            if (q < nq) {
              const float num = fmaf(st[4 * q], acc[i], st[4 * q + 1] * mu) + mix[i];
              p.out[((int64_t)(b * nq + q) * H + h) * d + el] = num / st[4 * q + 2];
            }
          }
        }
      }
      return;
    }
  }
  // W_up,v,t row `el` against the latent averages of a group of queries,
  // then the in-flight term of each query of the group
  const int rows = nt / d;  // whole rows of d threads; the rest sit this out
  if (t >= rows * d) return;
  const int el = t % d;
  const uint32_t *wrow = wl + el * lay.w_pitch;
  const E *wgrow = wg + (int64_t)el * rv;
  const float mu = p.muv[(int64_t)h * d + el];
  for (int i0 = (t / d) * kQGroup; i0 < nq; i0 += rows * kQGroup) {
    float wa[kQGroup];
#pragma unroll
    for (int j = 0; j < kQGroup; ++j) wa[j] = 0.f;
#pragma unroll 8
    for (int r = 0; r < rv; ++r) {
      const float w = w_vec ? w_lds_elem<E>(wrow, r) : load_elem(wgrow, r);
      const float *ar = abar + r * nqp + i0;
#pragma unroll
      for (int j = 0; j < kQGroup; ++j) wa[j] = fmaf(w, ar[j], wa[j]);
    }
#pragma unroll
    for (int j = 0; j < kQGroup; ++j) {
      const int i = i0 + j;
      if (i >= nq) break;
      // [fs (W_up,v,t A + mu_v,t L_s) + sum_m w_m v_m] / den, w_m = 0 for m > i
      float num = fmaf(st[4 * i], wa[j], st[4 * i + 1] * mu);
      const float *wi = sc + i * nq;
#pragma unroll 8
      for (int m = 0; m < nq; ++m) num = fmaf(wi[m], kr[m * d + el], num);
      p.out[((int64_t)(b * nq + i) * H + h) * d + el] = num / st[4 * i + 2];
    }
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

hipError_t launch_decode_merge_batched(const DecodeParams &p, int dtype, hipStream_t st) {
  dim3 grid(p.H, (p.B + kBT - 1) / kBT);
  const bool two = p.d <= 128;  // two sequence groups, 2 d threads
  const int threads = two ? 2 * p.d : p.d >= 256 ? 256 : (p.d + 63) / 64 * 64;
  const BatchedMergeLds lay = batched_merge_lds(p.d, p.rv, p.S, dtype == LLA_DT_F32 ? 4 : 2);
  DecodeParams q = p;
  q.w_lds = lay.with_w <= kBatchedMergeWLdsMax ? 1 : 0;  // else W_up,v,t is read from HBM
  const size_t sm = q.w_lds ? lay.with_w : lay.base;
  if (sm > 160 * 1024) return hipErrorInvalidValue;
  const void *fn =
      dtype == LLA_DT_F32
          ? (two ? reinterpret_cast<const void *>(decode_merge_batched<float, 2>)
                 : reinterpret_cast<const void *>(decode_merge_batched<float, 1>))
          : (two ? reinterpret_cast<const void *>(decode_merge_batched<bf16_t, 2>)
                 : reinterpret_cast<const void *>(decode_merge_batched<bf16_t, 1>));
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  if (dtype == LLA_DT_F32) {
    if (two)
      hipLaunchKernelGGL((decode_merge_batched<float, 2>), grid, dim3(threads), sm, st, q);
    else
      hipLaunchKernelGGL((decode_merge_batched<float, 1>), grid, dim3(threads), sm, st, q);
  } else {
    if (two)
      hipLaunchKernelGGL((decode_merge_batched<bf16_t, 2>), grid, dim3(threads), sm, st, q);
    else
      hipLaunchKernelGGL((decode_merge_batched<bf16_t, 1>), grid, dim3(threads), sm, st, q);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge_inflight(const DecodeParams &p, int32_t B_real, const float *k_new,
                                        const float *v_new, int dtype, hipStream_t st) {
  if (p.qps > kMaxQ) return hipErrorInvalidValue;
  if (p.d < 1 || p.d > 256) return hipErrorInvalidValue;
  const int threads = 256;
  const int esize = dtype == LLA_DT_F32 ? 4 : 2;
  const InflightMergeLds lay = inflight_merge_lds(p.qps, p.d, p.rv, p.S, esize);
  DecodeParams q = p;
  q.w_lds = lay.with_w <= kInflightMergeLdsMax ? 1 : 0;  // else W_up,v,t is read from HBM
  const size_t sm = q.w_lds ? lay.with_w : lay.base;
  if (sm > kInflightMergeLdsMax) return hipErrorInvalidValue;
  dim3 grid(p.H, B_real);
  const void *fn = dtype == LLA_DT_F32 ? reinterpret_cast<const void *>(decode_merge_inflight<float>)
                                       : reinterpret_cast<const void *>(decode_merge_inflight<bf16_t>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  if (dtype == LLA_DT_F32)
    hipLaunchKernelGGL(decode_merge_inflight<float>, grid, dim3(threads), sm, st, q, k_new, v_new);
  else
    hipLaunchKernelGGL(decode_merge_inflight<bf16_t>, grid, dim3(threads), sm, st, q, k_new, v_new);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams &p, int dtype, hipStream_t st) {
  const int hpb = merge_heads_per_block(p.d, p.rv);
  dim3 grid((p.H + hpb - 1) / hpb, p.B);
  const size_t sm = sizeof(float) * p.rv * hpb;
  if (dtype == LLA_DT_F32)
    hipLaunchKernelGGL(decode_merge<float>, grid, dim3(256), sm, st, p);
  else
    hipLaunchKernelGGL(decode_merge<bf16_t>, grid, dim3(256), sm, st, p);
  return hipGetLastError();
}

}  // namespace lla
