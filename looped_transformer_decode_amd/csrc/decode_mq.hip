// Multi-query per-head LLA decode for bf16 stores, d = 128: up to 16 queries
// of one sequence (the tokens of a decode step whose loops run before their
// latents exist) attend the same store slots.  What it computes is that of
// the single-query kernels ("Looped Latent Attention: Cross-Loop KV
// Compression for Looped Transformers", Sec. 3 Eq. 3 and "RoPE and
// reconstruction"), for every query i of sequence b at once:
//     s_ij = scale * RoPE(q_i, pos_i) . RoPE(W_up,k,t c_k,j + mu_k,t, j)
// with an online softmax per query and the latent-space value average
// sum_j p_ij c_v,j per query; the in-flight merge applies W_up,v,t.
//
// Reconstruct first.  With n_q queries sharing every tile, rebuilding the
// keys once and multiplying them by all queries beats the single-query
// bilinear form (whose matrix work grows with the number of queries).  Per
// 32-slot tile and head (one wave per head, four heads per workgroup):
//  * K^T = W_up,k,t [c | 1]^T on v_mfma_f32_32x32x16_bf16, the mean folded
//    in as two extra latent components (mu split exactly into bf16 hi + lo)
//    of value one.  Lane l holds slot l%32 and dims 32T + 8c + 4(l/32) + e,
//    so the rotate-half partner (dim + 64) sits in the same lane; RoPE is
//    applied in registers and four consecutive dims are stored to LDS with
//    one 8-byte write (16-byte chunks XOR-swizzled by slot).
//  * S = Q K^T on v_mfma_f32_16x16x32_bf16 (queries x slots, K = d); lane
//    l owns query rows 4(l/16) + i, which are also the rows it owns in the
//    value accumulator, so softmax state and rescaling stay in registers.
//  * P C_v on v_mfma_f32_16x16x32_bf16 (queries x value columns, K = 32
//    slots), P through LDS, C_v gathered from a staged tile whose row pitch
//    spreads the four slot groups over distinct banks.
// Latent rows are read with direct 16-byte global loads, the next tile's
// issued as soon as the current one's have been consumed.  The rotation of
// each (slot, dim) comes from the RoPE table's bf16 phi tile of the 32 slots,
// copied HBM-to-LDS once per workgroup (a quarter by each wave, two buffers,
// one barrier per tile); every other LDS region is private to a wave.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace mq {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kD = 128;
constexpr int kHalf = kD / 2;
constexpr int kTile = 32;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQ = 16;               // query rows of the MFMA tiles
constexpr float kRescaleGap = 8.0f;  // log2 domain
constexpr int kPhiTileBytes = kTile * kD * 2;  // bf16 phi rows of one 32-slot tile
#define LDS_AS __attribute__((address_space(3)))

template <int RK, int RV>
struct Cfg {
  static constexpr int KS = RK / 16;                       // latent k-steps (+1 for mu)
  static constexpr int VCH = RV / 8;                       // 16-byte chunks of a V row
  static constexpr int VLOADS = (kTile * VCH + 63) / 64;   // V chunks per lane
  static constexpr int VPITCH = RV + 4;                    // staged V row, elements
  static constexpr int VB = RV / 16;                       // value column blocks
  static constexpr int PPITCH = kTile + 8;                 // staged P row, elements
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = kTile * kD * 2;
  static constexpr int P_OFF = V_OFF + (kTile * VPITCH * 2 + 15) / 16 * 16;
  static constexpr int WAVE_BYTES = P_OFF + kQ * PPITCH * 2;
  static constexpr int PHI_OFF = WAVE_BYTES * kWaves;     // two shared phi tiles
  static constexpr int LDS = PHI_OFF + 2 * kPhiTileBytes;
};

// DPP row operations within groups of 16 lanes (see kvcache.hip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}

__device__ __forceinline__ int kswz(int slot, int chunk) { return chunk ^ (slot & 15); }

// Every LDS region here is private to one wave, so lanes of the same wave
// exchange data through it without a workgroup barrier: wait for this
// wave's LDS writes, and keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited
  __builtin_amdgcn_wave_barrier();
}

template <int RK, int RV>
__global__ __launch_bounds__(kThreads) void decode_mq_split(DecodeParams p) {
  using C = Cfg<RK, RV>;
  constexpr int R = RK + RV;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h2 = lane >> 5, l16 = lane & 15, g4 = lane >> 4;
  const int groups = (p.H + kWaves - 1) / kWaves;
  int bid = blockIdx.x;
  const int s = bid % p.S;
  bid /= p.S;
  const int hg = bid % groups;
  const int b = bid / groups;                  // stored sequence
  const int h_raw = hg * kWaves + wave;
  const bool head_ok = h_raw < p.H;
  const int h = head_ok ? h_raw : p.H - 1;
  const int nq = p.qps;
  const int first = min(max(p.pos[b], 0), p.N);  // store slots 0 .. first-1
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, first);

  char *wl = lds + wave * C::WAVE_BYTES;
  uint16_t *Kt = reinterpret_cast<uint16_t *>(wl + C::K_OFF);   // [32][128], swizzled
  uint16_t *Vt = reinterpret_cast<uint16_t *>(wl + C::V_OFF);   // [32][VPITCH]
  uint16_t *Pt = reinterpret_cast<uint16_t *>(wl + C::P_OFF);   // [16][PPITCH]

  auto part_at = [&](int qi) {
    return p.ws + ((int64_t)((b * nq + qi) * p.H + h) * p.S + s) * (RV + 2);
  };
  if (t0 >= t1) {  // nothing of the store in this split (workgroup-uniform)
    if (head_ok)
      for (int e = lane; e < nq * (RV + 2); e += 64) {
        const int qi = e / (RV + 2), r = e % (RV + 2);
        part_at(qi)[r] = r == 0 ? -INFINITY : 0.f;
      }
    return;
  }

  // ---- setup: rotated, scaled queries (A operand of S = Q K^T) ----
  bf16x8_t qa[kD / 32];
  {
    const int qi = l16;
    const bool qok = qi < nq;
    const int qpos = min(first + qi, p.N - 1);
    const float *qrow = p.q + ((int64_t)(b * nq + (qok ? qi : 0)) * p.H + h) * kD;
    const float *cs = p.rope_f32 + (int64_t)qpos * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * ks + 8 * g4 + e;
        float r;
        if (i < kHalf)
          r = qrow[i] * cs[2 * i] - qrow[i + kHalf] * cs[2 * i + 1];
        else
          r = qrow[i] * cs[2 * (i - kHalf)] + qrow[i - kHalf] * cs[2 * (i - kHalf) + 1];
        v[e] = qok ? r * p.scale_log2 : 0.f;
      }
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      qa[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // ---- W_up,k,t rows with mu folded in (A operand of K^T) ----
  bf16x8_t wa[4][C::KS + 1];
  {
    const uint16_t *W = reinterpret_cast<const uint16_t *>(p.wk) + (int64_t)h * kD * RK;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int dim = 32 * T + l32;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        wa[T][ks] = *reinterpret_cast<const bf16x8_t *>(W + (int64_t)dim * RK + 16 * ks + 8 * h2);
      const float mu = p.muk[(int64_t)h * kD + dim];
      const uint16_t hi = f32_to_bf16_bits(mu);
      const uint16_t lo = f32_to_bf16_bits(mu - bf16_bits_to_f32(hi));
      u32x4_t w = {h2 == 0 ? (uint32_t)hi | ((uint32_t)lo << 16) : 0u, 0u, 0u, 0u};
      wa[T][C::KS] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const u32x4_t ones_w = {h2 == 0 ? 0x3F803F80u : 0u, 0u, 0u, 0u};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_w);

  // ---- latent streaming ----
  const int64_t srow = (int64_t)p.Hs * R;  // elements per slot
  const uint16_t *lat = reinterpret_cast<const uint16_t *>(p.store) +
                        ((int64_t)b * p.D + p.layer) * p.N * srow + (int64_t)h * R;
  u32x4_t kb[C::KS], vch[C::VLOADS];
  auto load_k = [&](int tb) {
    const int js = min(tb + l32, t1 - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kb[ks] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t *>(lat + js * srow + 16 * ks + 8 * h2));
  };
  auto load_v = [&](int tb) {
#pragma unroll
    for (int u = 0; u < C::VLOADS; ++u) {
      const int c = lane + 64 * u;
      const int sl = min(c / C::VCH, kTile - 1), q = c % C::VCH;
      const int j = min(tb + sl, t1 - 1);
      if (c < kTile * C::VCH)
        vch[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t *>(lat + j * srow + RK + 8 * q));
    }
  };
  auto load_tile = [&](int tb) {
    load_k(tb);
    load_v(tb);
  };

  // bf16 phi rows of tile tb (the RoPE table's MFMA tiles): the workgroup's
  // four waves each copy a quarter into LDS buffer `buf`, HBM to LDS directly
  const __amdgpu_buffer_rsrc_t rphi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.rope_bf16), (short)0,
      ((p.N + kTile - 1) / kTile) * kPhiTileBytes, 0x00020000);
  auto issue_phi = [&](int tb, int buf) {
    char *pb = lds + C::PHI_OFF + buf * kPhiTileBytes;
    const uint32_t off = (uint32_t)(tb / kTile) * kPhiTileBytes;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int blk = 2 * wave + u;  // 1 KB blocks 0..7
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rphi, (LDS_AS void *)(pb + blk * 1024), 16,
                                               off + (uint32_t)(blk * 64 + lane) * 16, 0, 0, 0);
    }
  };

  float m[4], lsum[4];
  f32x4_t acc[C::VB];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    lsum[i] = 0.f;
  }
#pragma unroll
  for (int v = 0; v < C::VB; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_tile(t0);
  issue_phi(t0, 0);
  for (int tb = t0, it = 0; tb < t1; tb += kTile, ++it) {
    const bool more = tb + kTile < t1;
    // this tile's latents (registers) and phi rows (LDS) have landed, and
    // every wave is done with the phi buffer the next copy overwrites
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    const char *phb = lds + C::PHI_OFF + (it & 1) * kPhiTileBytes;
    // V chunks of this tile into the staged tile, then the next tile's V
    // chunks and phi rows on their way
#pragma unroll
    for (int u = 0; u < C::VLOADS; ++u) {
      const int c = lane + 64 * u;
      if (c < kTile * C::VCH) {
        const int sl = c / C::VCH, q = c % C::VCH;
        u32x2_t *dst = reinterpret_cast<u32x2_t *>(Vt + sl * C::VPITCH + 8 * q);
        dst[0] = u32x2_t{vch[u][0], vch[u][1]};
        dst[1] = u32x2_t{vch[u][2], vch[u][3]};
      }
    }
    if (more) issue_phi(tb + kTile, (it + 1) & 1);
    // K^T of the tile, two dim-tile pairs (T, T + 2) at a time
    bf16x8_t kbf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kbf[ks] = __builtin_bit_cast(bf16x8_t, kb[ks]);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      // one pair of accumulator tiles live at a time
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t a0 = {}, a1 = {};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[T][ks], kbf[ks], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[T + 2][ks], kbf[ks], a1, 0, 0, 0);
      }
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[T][C::KS], ones, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[T + 2][C::KS], ones, a1, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i0 = 32 * T + 8 * c + 4 * h2;  // first of four consecutive dims (< 64)
        // phi tile element (step 2T + c/2, lane l32 + 32 (c%2), 4 h2 + e): cos at dim
        // i0 + e, and 4 steps further sin
        const uint16_t *ph = reinterpret_cast<const uint16_t *>(phb) +
                             ((2 * T + c / 2) * 64 + l32 + 32 * (c % 2)) * 8 + 4 * h2;
        const u32x2_t cw = *reinterpret_cast<const u32x2_t *>(ph);
        const u32x2_t sw = *reinterpret_cast<const u32x2_t *>(ph + 4 * 64 * 8);
        const float co[4] = {bf16_lo(cw[0]), bf16_hi(cw[0]), bf16_lo(cw[1]), bf16_hi(cw[1])};
        const float sn[4] = {bf16_lo(sw[0]), bf16_hi(sw[0]), bf16_lo(sw[1]), bf16_hi(sw[1])};
        float r0[4], r1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = a0[4 * c + e], x1 = a1[4 * c + e];
          r0[e] = x0 * co[e] - x1 * sn[e];
          r1[e] = x0 * sn[e] + x1 * co[e];
        }
        const int ch0 = (i0 >> 3), ch1 = ((i0 + kHalf) >> 3);
        *reinterpret_cast<u32x2_t *>(Kt + l32 * kD + kswz(l32, ch0) * 8 + 4 * h2) =
            u32x2_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3])};
        *reinterpret_cast<u32x2_t *>(Kt + l32 * kD + kswz(l32, ch1) * 8 + 4 * h2) =
            u32x2_t{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
      }
    }
    if (more) {  // the latents' registers are free again: the next tile's
      load_k(tb + kTile);
      load_v(tb + kTile);
    }
    wave_lds_sync();

    // S = Q K^T: queries 4 g4 + i, slots 16 nt + l16
    f32x4_t sc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int sl = 16 * nt + l16;
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(
            Kt + sl * kD + kswz(sl, 4 * ks + g4) * 8);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kf, o, 0, 0, 0);
      }
      sc[nt] = o;
    }
    // online softmax per query row; P to LDS
    const bool ok0 = tb + l16 < t1, ok1 = tb + 16 + l16 < t1;
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = ok0 ? sc[0][i] : -INFINITY, s1 = ok1 ? sc[1][i] : -INFINITY;
      const float mx = row16_max(fmaxf(s0, s1));
      alpha[i] = 1.f;
      if (mx > m[i] + kRescaleGap) {  // row-uniform
        alpha[i] = exp2f(m[i] - mx);
        m[i] = mx;
      }
      const uint16_t p0 = f32_to_bf16_bits(ok0 ? exp2f(s0 - m[i]) : 0.f);
      const uint16_t p1 = f32_to_bf16_bits(ok1 ? exp2f(s1 - m[i]) : 0.f);
      lsum[i] = fmaf(lsum[i], alpha[i], bf16_bits_to_f32(p0) + bf16_bits_to_f32(p1));
      const int q = 4 * g4 + i;
      Pt[q * C::PPITCH + l16] = p0;
      Pt[q * C::PPITCH + 16 + l16] = p1;
    }
    wave_lds_sync();

    // acc += P C_v (queries x value columns, K = 32 slots)
    const bf16x8_t pa = *reinterpret_cast<const bf16x8_t *>(Pt + l16 * C::PPITCH + 8 * g4);
#pragma unroll
    for (int v = 0; v < C::VB; ++v) {
      const uint16_t *vb = Vt + (8 * g4) * C::VPITCH + 16 * v + l16;
      bf16x8_t bv;
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = (short)vb[e * C::VPITCH];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[v][i] *= alpha[i];
      acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, acc[v], 0, 0, 0);
    }
  }

  // ---- partials (m, l, sum p c_v) of every query ----
  if (!head_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * g4 + i;
    const float l = row16_sum(lsum[i]);
    if (q >= nq) continue;
    float *part = part_at(q);
    if (l16 == 0) {
      part[0] = m[i];
      part[1] = l;
    }
#pragma unroll
    for (int v = 0; v < C::VB; ++v) part[2 + 16 * v + l16] = acc[v][i];
  }
}

template <int RK, int RV>
hipError_t launch(const DecodeParams &p, hipStream_t st) {
  using C = Cfg<RK, RV>;
  const int groups = (p.H + kWaves - 1) / kWaves;
  const int B = p.B / p.qps;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_mq_split<RK, RV>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mq_split<RK, RV>), dim3((unsigned)((int64_t)B * groups * p.S)),
                     dim3(kThreads), C::LDS, st, p);
  return hipGetLastError();
}

}  // namespace mq

bool decode_mq_supported(int32_t d, int32_t rk, int32_t rv, int32_t Hs, int32_t H, int32_t n_q) {
  if (d != mq::kD || Hs != H || n_q < 1 || n_q > mq::kQ) return false;
  return (rk == 16 && rv == 32) || (rk == 32 && rv == 64) || (rk == 48 && rv == 80);
}

hipError_t launch_decode_mq(const DecodeParams &p, hipStream_t st) {
  if (p.rk == 16 && p.rv == 32) return mq::launch<16, 32>(p, st);
  if (p.rk == 32 && p.rv == 64) return mq::launch<32, 64>(p, st);
  if (p.rk == 48 && p.rv == 80) return mq::launch<48, 80>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace lla
