// Uncompressed K/V cache paths: the comparisons the paper draws against the
// latent store (technical summary, "Serving Capacity": the "fast path" that
// reconstructs and caches full K/V; paper Sec. 3, matched-axis baselines:
// the control that caches only the final loop's K/V and reuses it in every
// loop).  Cache layout [B, D, L, N, H, 2, d], keys stored after RoPE.
//
//   kv_split       flash-decode.  One workgroup per (sequence, group of
//                  heads, context split); a group of LG lanes owns one head,
//                  each lane 16 bytes (8 bf16 / 4 fp32 elements) of the
//                  rotated query, of every K and V row it reads and of the
//                  output accumulator.  K and V rows stream from HBM straight
//                  into registers, eight slots in flight per lane; q.k is
//                  reduced over the lane group with DPP row operations and an
//                  online softmax (lazy rescale) runs per block of 8 slots.
//   kv_merge       log-sum-exp merge of the context splits.
//   kv_fill_mfma   reconstruct-to-cache for bf16: per (sequence, head, 128
//                  slots), x_hat = c W_up,t^T + mu_t as 32x32x16 bf16 MFMA
//                  tiles (slots x r by r x d), RoPE applied in registers to
//                  the (i, i + d/2) column pair each lane holds, the tile
//                  staged in LDS and written as whole 16-byte row pieces.
//   kv_fill_valu   the same for any shape and fp32 (one thread per
//                  rotate-half pair).
//   kv_append      raw K/V rows (rotated) into the cache.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;           // slots in flight per lane
constexpr float kRescaleGap = 8.0f;  // rescale only when the max grows by > 2^8
constexpr int kFillSlots = 128;      // slots one reconstruct-to-cache block covers

// DPP controls (GCN/CDNA data-parallel primitives) within a row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15 - i within 16

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LG lanes.  Every step adds a value to its
// partner's, so all lanes of a group end with the same bits.
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LG >= 2) v += dpp_mov<kDppQuadXor1>(v);
  if constexpr (LG >= 4) v += dpp_mov<kDppQuadXor2>(v);
  if constexpr (LG >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (LG >= 16) v += dpp_mov<kDppRowMirror>(v);
  if constexpr (LG >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LG >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <typename E>
__device__ __forceinline__ void unpack16(const u32x4_t &w, float *f);
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const u32x4_t &w, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4_t &w, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

__device__ __forceinline__ int64_t cache_row(const KvParams &p, int b, int j, int h) {
  return (((((int64_t)b * p.D + p.layer) * p.L + p.cache_loop) * p.N + j) * p.H + h) * 2 * p.d;
}

// ---------------------------------------------------------------------------
// Flash-decode over the cache
// ---------------------------------------------------------------------------
template <typename E, int LG>
__global__ __launch_bounds__(kThreads) void kv_split(KvParams p) {
  constexpr int EPL = 16 / sizeof(E);
  constexpr int HPW = 64 / LG;
  constexpr int HG = HPW * kWaves;
  constexpr int d = LG * EPL;
  constexpr int half = d / 2;
  const int groups = (p.H + HG - 1) / HG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int bid = blockIdx.x;
  const int s = bid % p.S;
  bid /= p.S;
  const int g = bid % groups;
  const int b = bid / groups;
  const int h = g * HG + wave * HPW + lane / LG;
  const int e0 = (lane % LG) * EPL;
  const bool act = h < p.H;
  const int hh = act ? h : p.H - 1;

  const int pos = min(max(p.pos[b], 0), p.N - 1);
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, pos + 1);
  float *part = p.ws + ((int64_t)(b * p.H + hh) * p.S + s) * (d + 2);
  if (t0 >= t1) {  // split past the query position (block-uniform): empty partial
    if (act) {
      if (e0 == 0) {
        part[0] = -INFINITY;
        part[1] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[2 + e0 + e] = 0.f;
    }
    return;
  }

  // this lane's elements of RoPE(q, pos), times scale * log2(e)
  float qf[EPL];
  {
    const float *qb = p.q + ((int64_t)b * p.H + hh) * d;
    const float *cs = p.rope_f32 + (int64_t)pos * d;  // [d/2][2]
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = e0 + e;
      float r;
      if (i < half)
        r = qb[i] * cs[2 * i] - qb[i + half] * cs[2 * i + 1];
      else
        r = qb[i] * cs[2 * (i - half)] + qb[i - half] * cs[2 * (i - half) + 1];
      qf[e] = r * p.scale_log2;
    }
  }

  const int64_t slot_stride = (int64_t)p.H * 2 * d;
  const E *base = reinterpret_cast<const E *>(p.cache) + cache_row(p, b, 0, hh) + e0;

  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  for (int j0 = t0; j0 < t1; j0 += kUnroll) {
    u32x4_t kf[kUnroll], vf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = min(j0 + u, t1 - 1);  // past t1: re-read a valid slot, masked below
      const E *r = base + j * slot_stride;
      kf[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(r));
      vf[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(r + d));
    }
    float sc[kUnroll];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kv[EPL];
      unpack16<E>(kf[u], kv);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kv[e], dot);
      dot = group_sum<LG>(dot);
      sc[u] = j0 + u < t1 ? dot : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    if (mx > m + kRescaleGap) {
      const float f = exp2f(m - mx);  // 0 on the first block (m = -inf)
      l *= f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= f;
      m = mx;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pe = exp2f(sc[u] - m);
      l += pe;
      float vv[EPL];
      unpack16<E>(vf[u], vv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pe, vv[e], acc[e]);
    }
  }
  if (!act) return;
  if (p.S == 1) {
    float *o = p.out + ((int64_t)b * p.H + hh) * d + e0;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
    return;
  }
  if (e0 == 0) {
    part[0] = m;
    part[1] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[2 + e0 + e] = acc[e];
}

// Block (h, b): out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// The split weights 2^(m_s - M) are formed once into LDS (up to kMergeMaxS
// splits; more splits recompute them per element).
constexpr int kMergeThreads = 128;
constexpr int kMergeMaxS = 1024;
__global__ __launch_bounds__(kMergeThreads) void kv_merge(KvParams p) {
  __shared__ float wsh[kMergeMaxS];
  __shared__ float red[2][kMergeThreads / 64];
  const int h = blockIdx.x, b = blockIdx.y, d = p.d, S = p.S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *part = p.ws + (int64_t)(b * p.H + h) * S * (d + 2);
  float M = -INFINITY;
  for (int s = tid; s < S; s += kMergeThreads) M = fmaxf(M, part[(int64_t)s * (d + 2)]);
  M = wave_max(M);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  float L = 0.f;
  for (int s = tid; s < S; s += kMergeThreads) {
    const float ms = part[(int64_t)s * (d + 2)];
    const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
    if (s < kMergeMaxS) wsh[s] = wgt;
    L = fmaf(part[(int64_t)s * (d + 2) + 1], wgt, L);
  }
  L = wave_sum(L);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  L = red[1][0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) L += red[1][w];
  const float inv = 1.0f / L;
  for (int i = tid; i < d; i += kMergeThreads) {
    float a = 0.f;
    const int s_lds = S < kMergeMaxS ? S : kMergeMaxS;
#pragma unroll 8
    for (int s = 0; s < s_lds; ++s) a = fmaf(part[(int64_t)s * (d + 2) + 2 + i], wsh[s], a);
    for (int s = s_lds; s < S; ++s) {
      const float ms = part[(int64_t)s * (d + 2)];
      a = fmaf(part[(int64_t)s * (d + 2) + 2 + i], ms == -INFINITY ? 0.f : exp2f(ms - M), a);
    }
    p.out[((int64_t)b * p.H + h) * d + i] = a * inv;
  }
}

// ---------------------------------------------------------------------------
// Reconstruct-to-cache, MFMA (bf16)
// ---------------------------------------------------------------------------
// Block = 2d threads, grid (slot chunks of 128, H, B).  Waves [0, d/64) form
// K, wave w the dim tiles [32w, 32w + 32) and [32w + d/2, ...), so that each
// lane holds the rotate-half pair (i, i + d/2) of the slots of its rows;
// waves [d/64, d/32) form V, wave w the tiles [64w, 64w + 64).  NK >= the
// number of 16-wide k-steps of either rank.
template <int NK>
__global__ __launch_bounds__(512) void kv_fill_mfma(KvParams p) {
  extern __shared__ __align__(16) uint16_t stage[];  // [32 slots][2d] bf16: K row, V row
  const int d = p.d, half = d / 2, nkw = d / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int slot_lo = p.slot0 + blockIdx.x * kFillSlots;
  const int slot_hi = min(slot_lo + kFillSlots, p.slot0 + p.n);
  const bool is_k = wave < nkw;
  const int pw = is_k ? wave : wave - nkw;
  const int col = lane & 31, kh = lane >> 5;
  const int dim0 = is_k ? 32 * pw + col : 64 * pw + col;
  const int dim1 = is_k ? dim0 + half : dim0 + 32;
  const int r = is_k ? p.rk : p.rv;
  const int nk = r / 16;

  const uint16_t *W = reinterpret_cast<const uint16_t *>(is_k ? p.wk : p.wv) + (int64_t)h * d * r;
  bf16x8_t w0[NK], w1[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
    if (ks < nk) {
      w0[ks] = *reinterpret_cast<const bf16x8_t *>(W + (int64_t)dim0 * r + 16 * ks + 8 * kh);
      w1[ks] = *reinterpret_cast<const bf16x8_t *>(W + (int64_t)dim1 * r + 16 * ks + 8 * kh);
    }
  const float *mu = is_k ? p.muk : p.muv;
  const float mu0 = mu[(int64_t)h * d + dim0], mu1 = mu[(int64_t)h * d + dim1];
  const int64_t slot_elems = (int64_t)p.Hs * p.R;
  const uint16_t *lat = reinterpret_cast<const uint16_t *>(p.store) +
                        ((int64_t)b * p.D + p.layer) * p.N * slot_elems +
                        (p.Hs == 1 ? 0 : (int64_t)h * p.R) + (is_k ? 0 : p.rk) + 8 * kh;
  uint16_t *cache = reinterpret_cast<uint16_t *>(p.cache);
  const int row = 2 * d;           // staged elements per slot
  const int chunks = row / 8;      // 16-byte pieces per slot

  // latent fragments of a tile: slot tile + col, components 16 ks + 8 kh ..
  auto lat_row = [&](int tile) { return lat + min(tile + col, slot_hi - 1) * slot_elems; };
  bf16x8_t lf[NK];
  auto load_lat = [&](int tile) {
    const uint16_t *crow = lat_row(tile);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      if (ks < nk) lf[ks] = *reinterpret_cast<const bf16x8_t *>(crow + 16 * ks);
  };
  // Where the registers allow (ranks up to 128), the next tile's latents are
  // loaded while this one is written out, and this tile's (cos, sin) pairs
  // are loaded before its matrix work rather than after it: 2.50 -> 3.06 TB/s
  // at B = 32.
  constexpr bool kAhead = NK <= 8;
  if (kAhead) load_lat(slot_lo);
  for (int tile = slot_lo; tile < slot_hi; tile += 32) {
    // the (cos, sin) pairs of this lane's 16 slots, one 8-byte load each
    float2 cs[16];
    auto rope_pair = [&](int a) {
      const int j = min(tile + 8 * (a / 4) + 4 * kh + (a % 4), p.N - 1);
      return *reinterpret_cast<const float2 *>(p.rope_f32 + ((int64_t)j * half + dim0) * 2);
    };
    if (kAhead && is_k) {
#pragma unroll
      for (int a = 0; a < 16; ++a) cs[a] = rope_pair(a);
    }
    f32x16_t acc0 = {}, acc1 = {};
    const uint16_t *crow = lat_row(tile);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      if (ks < nk) {
        const bf16x8_t a =
            kAhead ? lf[ks] : *reinterpret_cast<const bf16x8_t *>(crow + 16 * ks);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w0[ks], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w1[ks], acc1, 0, 0, 0);
      }
    if (kAhead && tile + 32 < slot_hi) load_lat(tile + 32);
    __syncthreads();  // the previous tile's write-out has read the stage
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int sl = 8 * (a / 4) + 4 * kh + (a % 4);
      float x0 = acc0[a] + mu0, x1 = acc1[a] + mu1;
      if (is_k) {
        const float2 pr = kAhead ? cs[a] : rope_pair(a);
        const float c = pr.x, sn = pr.y;
        const float r0 = x0 * c - x1 * sn, r1 = x0 * sn + x1 * c;
        x0 = r0;
        x1 = r1;
      }
      const int off = sl * row + (is_k ? 0 : d);
      stage[off + dim0] = f32_to_bf16_bits(x0);
      stage[off + dim1] = f32_to_bf16_bits(x1);
    }
    __syncthreads();
    const int nsl = min(32, slot_hi - tile);
    for (int c = threadIdx.x; c < nsl * chunks; c += blockDim.x) {
      const int sl = c / chunks, ch = c % chunks;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stage + sl * row + 8 * ch);
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4_t *>(cache + cache_row(p, b, tile + sl, h) + 8 * ch));
    }
  }
}

// ---------------------------------------------------------------------------
// Reconstruct-to-cache and raw append, one thread per rotate-half pair
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(kThreads) void kv_fill_valu(KvParams p) {
  const int d = p.d, half = d / 2;
  const int64_t total = (int64_t)p.B * p.n * p.H * half;
  const E *lat = reinterpret_cast<const E *>(p.store);
  const E *wk = reinterpret_cast<const E *>(p.wk);
  const E *wv = reinterpret_cast<const E *>(p.wv);
  E *cache = reinterpret_cast<E *>(p.cache);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(t % half);
    int64_t q = t / half;
    const int h = (int)(q % p.H);
    q /= p.H;
    const int j = p.slot0 + (int)(q % p.n);
    const int b = (int)(q / p.n);
    const int64_t c0 = ((((int64_t)b * p.D + p.layer) * p.N + j) * p.Hs + (p.Hs == 1 ? 0 : h)) * p.R;
    const int64_t ra = (int64_t)h * d + i, rb = ra + half;
    float ka = p.muk[ra], kb = p.muk[rb], va = p.muv[ra], vb = p.muv[rb];
    for (int k = 0; k < p.rk; ++k) {
      const float c = load_elem(lat, c0 + k);
      ka = fmaf(load_elem(wk, ra * p.rk + k), c, ka);
      kb = fmaf(load_elem(wk, rb * p.rk + k), c, kb);
    }
    for (int k = 0; k < p.rv; ++k) {
      const float c = load_elem(lat, c0 + p.rk + k);
      va = fmaf(load_elem(wv, ra * p.rv + k), c, va);
      vb = fmaf(load_elem(wv, rb * p.rv + k), c, vb);
    }
    const float co = p.rope_f32[((int64_t)j * half + i) * 2];
    const float sn = p.rope_f32[((int64_t)j * half + i) * 2 + 1];
    E *row = cache + cache_row(p, b, j, h);
    store_elem(row, i, ka * co - kb * sn);
    store_elem(row, i + half, ka * sn + kb * co);
    store_elem(row, d + i, va);
    store_elem(row, d + i + half, vb);
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void kv_append(KvParams p) {
  const int d = p.d, half = d / 2;
  const int64_t total = (int64_t)p.B * p.n * p.H * half;
  E *cache = reinterpret_cast<E *>(p.cache);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(t % half);
    int64_t q = t / half;
    const int h = (int)(q % p.H);
    q /= p.H;
    const int jj = (int)(q % p.n);
    const int b = (int)(q / p.n);
    const int64_t j64 = (int64_t)p.start[b] + jj;
    if (j64 < 0 || j64 >= p.N) continue;
    const int j = (int)j64;
    const int64_t src = (((int64_t)b * p.n + jj) * p.H + h) * d;
    const float ka = p.k[src + i], kb = p.k[src + i + half];
    const float co = p.rope_f32[((int64_t)j * half + i) * 2];
    const float sn = p.rope_f32[((int64_t)j * half + i) * 2 + 1];
    E *row = cache + cache_row(p, b, j, h);
    store_elem(row, i, ka * co - kb * sn);
    store_elem(row, i + half, ka * sn + kb * co);
    store_elem(row, d + i, p.v[src + i]);
    store_elem(row, d + i + half, p.v[src + i + half]);
  }
}

template <typename E>
hipError_t launch_split(const KvParams &p, dim3 grid, hipStream_t st) {
  constexpr int EPL = 16 / sizeof(E);
  switch (p.d / EPL) {
    case 4: hipLaunchKernelGGL((kv_split<E, 4>), grid, dim3(kThreads), 0, st, p); break;
    case 8: hipLaunchKernelGGL((kv_split<E, 8>), grid, dim3(kThreads), 0, st, p); break;
    case 16: hipLaunchKernelGGL((kv_split<E, 16>), grid, dim3(kThreads), 0, st, p); break;
    case 32: hipLaunchKernelGGL((kv_split<E, 32>), grid, dim3(kThreads), 0, st, p); break;
    case 64: hipLaunchKernelGGL((kv_split<E, 64>), grid, dim3(kThreads), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

dim3 stride_grid(int64_t total) {
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  return dim3((unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536));
}

}  // namespace

bool kv_decode_supported(int32_t d, int dtype) {
  const int epl = dtype == LLA_DT_F32 ? 4 : 8;
  if (d % epl != 0) return false;
  const int lg = d / epl;
  return lg >= 4 && lg <= 64 && (lg & (lg - 1)) == 0;
}

int32_t kv_heads_per_group(int32_t d, int dtype) {
  const int epl = dtype == LLA_DT_F32 ? 4 : 8;
  return 64 / (d / epl) * kWaves;
}

hipError_t launch_kv_decode(const KvParams &p, int dtype, hipStream_t st) {
  const int hg = kv_heads_per_group(p.d, dtype);
  const dim3 grid((unsigned)((int64_t)p.B * ((p.H + hg - 1) / hg) * p.S));
  const hipError_t e = dtype == LLA_DT_F32 ? launch_split<float>(p, grid, st)
                                           : launch_split<bf16_t>(p, grid, st);
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL(kv_merge, dim3(p.H, p.B), dim3(kMergeThreads), 0, st, p);
  return hipGetLastError();
}

bool kv_fill_mfma_supported(int32_t d, int32_t rk, int32_t rv) {
  return (d == 64 || d == 128 || d == 256) && rk % 16 == 0 && rv % 16 == 0 && rk <= 256 &&
         rv <= 256;
}

hipError_t launch_kv_fill(const KvParams &p, int dtype, bool mfma, hipStream_t st) {
  if (!mfma) {
    const dim3 grid = stride_grid((int64_t)p.B * p.n * p.H * (p.d / 2));
    if (dtype == LLA_DT_F32)
      hipLaunchKernelGGL(kv_fill_valu<float>, grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL(kv_fill_valu<bf16_t>, grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
  }
  const dim3 grid((p.n + kFillSlots - 1) / kFillSlots, p.H, p.B);
  const dim3 block(2 * p.d);
  const size_t lds = (size_t)32 * 2 * p.d * sizeof(uint16_t);
  const int nk = (p.rk > p.rv ? p.rk : p.rv) / 16;
  if (nk <= 2)
    hipLaunchKernelGGL(kv_fill_mfma<2>, grid, block, lds, st, p);
  else if (nk <= 4)
    hipLaunchKernelGGL(kv_fill_mfma<4>, grid, block, lds, st, p);
  else if (nk <= 8)
    hipLaunchKernelGGL(kv_fill_mfma<8>, grid, block, lds, st, p);
  else
    hipLaunchKernelGGL(kv_fill_mfma<16>, grid, block, lds, st, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const KvParams &p, int dtype, hipStream_t st) {
  const dim3 grid = stride_grid((int64_t)p.B * p.n * p.H * (p.d / 2));
  if (dtype == LLA_DT_F32)
    hipLaunchKernelGGL(kv_append<float>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(kv_append<bf16_t>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace lla
