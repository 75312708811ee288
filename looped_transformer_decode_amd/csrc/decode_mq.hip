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
// bilinear form (whose matrix work grows with the number of queries).  One
// wave per head, four heads per workgroup; per 32-slot tile and wave, all on
// v_mfma_f32_16x16x32_bf16 with every operand in registers:
//  * K^T = W_up,k,t [c | 1]^T per 16-dim tile and 16-slot half, the mean
//    folded in as two extra latent components (mu split exactly into bf16
//    hi + lo) of value one.  Lane l holds slot l%16 and dims 16a + 4(l/16)
//    + 0..3, so the rotate-half partner (dim + 64, tile a + 4) sits in the
//    same lane and RoPE is applied in registers.
//  * S^T = K Q^T (slots x queries): the rotated keys of tiles a and a + 4
//    are exactly the A operand of one k-step, with the dims of a k-step
//    taken in the order the lanes hold them (the queries' B operand uses
//    the same order).  Lane l ends with query l%16 and slots 4(l/16) + 0..3
//    of each half.
//  * acc^T += C_v^T P^T (value columns x queries, K = the 32 slots): those
//    eight softmax weights per lane are the B operand as they stand (slots
//    again in lane order), C_v^T comes from the staged tile in the same
//    order by two transposing LDS reads (ds_read_b64_tr_b16) per column
//    block, and the output lane keeps query l%16, so the softmax state and
//    the rescaling of its accumulator stay in the lane.
// Latent tiles stream HBM -> LDS directly (buffer loads into LDS, no
// register staging) into a ring of two to four tiles per wave; a tile's
// 16-byte chunks are rotated within each slot record so that the 16 slots a
// read touches fall in distinct banks.  The rotation of each (slot, dim)
// comes from the RoPE table's bf16 phi tile of the 32 slots, copied into
// LDS a quarter by each wave, two buffers, one barrier per tile.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace mq {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kD = 128;
constexpr int kHalf = kD / 2;
constexpr int kTile = 32;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQ = 16;               // query columns of the MFMA tiles
constexpr float kRescaleGap = 8.0f;  // log2 domain
constexpr int kPhiTileBytes = kTile * kD * 2;  // bf16 phi rows of one 32-slot tile
constexpr int kLdsPerGroup = 80 * 1024;        // two workgroups per CU
// Cache policy of the latent loads: nontemporal (each latent is read once
// per call); the phi tiles, shared by every workgroup, use the default.
constexpr int kCachePolicyStream = 2;
#define LDS_AS __attribute__((address_space(3)))

// The largest power of two dividing both a and 16.
constexpr int gcd16(int a) {
  return (a % 16 == 0) ? 16 : (a % 8 == 0) ? 8 : (a % 4 == 0) ? 4 : (a % 2 == 0) ? 2 : 1;
}

template <int RK, int RV>
struct Cfg {
  static constexpr int R = RK + RV;
  static constexpr int CPR = R / 8;                  // 16-byte chunks per (slot, head) record
  static constexpr int KCH = RK / 8;                 // of which K latent
  static constexpr int STAGE = kTile * CPR * 16;     // one wave's tile in LDS
  static constexpr int LS = kTile * CPR / 64;        // LDS-direct loads per lane per tile
  static constexpr int NS_FIT = (kLdsPerGroup - 2 * kPhiTileBytes) / (kWaves * STAGE);
  static constexpr int NS = NS_FIT > 4 ? 4 : NS_FIT;  // ring depth (tiles per wave)
  static constexpr int PHI_OFF = kWaves * NS * STAGE;
  static constexpr int LDS = PHI_OFF + 2 * kPhiTileBytes;
  static constexpr int KS = (RK + 2 + 31) / 32;      // k-steps of K^T: latent, mu hi, mu lo
  static constexpr int VB = RV / 16;                 // value column blocks
  // chunk c of slot j sits at position (c + j / PER) % CPR of its record:
  // 16 consecutive slots then start in 16 distinct 16-byte bank groups
  static constexpr int PER = 16 / gcd16(CPR);
  static_assert(R % 16 == 0 && RK % 16 == 0 && RV % 16 == 0, "rank granularity");
  static_assert((kTile * CPR) % 64 == 0, "whole loads per tile");
  static_assert(NS >= 2, "two tiles per wave must fit");
  static_assert(LDS <= kLdsPerGroup, "LDS budget");
  static_assert(LS + 2 <= 63, "vmcnt range");
};

// Every ds read of a wave happens before it passes the next barrier; the
// signal fences keep the compiler from moving LDS accesses across it.  The
// wait leaves at most n vector-memory operations (the latest tile loads)
// outstanding.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

template <int RK, int RV>
__global__ __launch_bounds__(kThreads) void decode_mq_split(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only builtins
  using C = Cfg<RK, RV>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
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
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // ---- streaming: this wave's ring of latent tiles, the shared phi tiles ----
  const int64_t slab_bytes = (int64_t)p.N * p.Hs * C::R * 2;
  const char *slab = reinterpret_cast<const char *>(p.store) + ((int64_t)b * p.D + p.layer) * slab_bytes;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(slab), (short)0, (int)slab_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rphi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.rope_bf16), (short)0,
      ((p.N + kTile - 1) / kTile) * kPhiTileBytes, 0x00020000);
  const uint32_t srow = (uint32_t)p.Hs * C::R * 2;  // bytes per slot
  char *ring = lds + wave * C::NS * C::STAGE;
  int jn[C::LS];          // slot (in the tile) of the chunk this lane loads
  uint32_t cb[C::LS];     // its byte offset inside the slot
#pragma unroll
  for (int n = 0; n < C::LS; ++n) {
    const int P = n * 64 + lane;  // LDS chunk position in the stage
    const int j = P / C::CPR, r = P % C::CPR;
    const int c = (r + C::CPR - (j / C::PER) % C::CPR) % C::CPR;
    jn[n] = j;
    cb[n] = (uint32_t)h * (C::R * 2) + (uint32_t)c * 16;
  }
  auto issue_lat = [&](int it) {
    char *sb = ring + (it % C::NS) * C::STAGE;
    const int tb = t0 + it * kTile;
#pragma unroll
    for (int n = 0; n < C::LS; ++n) {
      // slots past the split's last repeat its last slot: every byte loaded
      // is a finite latent, and the softmax gives those slots weight zero
      const int j = min(tb + jn[n], t1 - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void *)(sb + n * 64 * 16), 16,
                                               (uint32_t)j * srow + cb[n], 0, 0,
                                               kCachePolicyStream);
    }
  };
  auto issue_phi = [&](int it) {
    char *pb = lds + C::PHI_OFF + (it & 1) * kPhiTileBytes;
    const uint32_t off = (uint32_t)((t0 + it * kTile) / kTile) * kPhiTileBytes;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int blk = 2 * wave + u;  // 1 KB blocks 0..7
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rphi, (LDS_AS void *)(pb + blk * 1024), 16,
                                               off + (uint32_t)(blk * 64 + lane) * 16, 0, 0, 0);
    }
  };
  // The first tiles stream in while the operands below are set up.
#pragma unroll
  for (int k = 0; k + 2 < C::NS; ++k)
    if (k < ntiles) issue_lat(k);
  issue_phi(0);
  if (C::NS - 2 < ntiles) issue_lat(C::NS - 2);

  // ---- B operand of S^T: rotated, scaled queries in the lanes' dim order ----
  // k-step a, lane (query l16, group g4), element e: dim 16a + 4 g4 + e
  // (e < 4) and dim 64 + 16a + 4 g4 + e - 4 (e >= 4).
  bf16x8_t qb[4];
  {
    const int qi = l16;
    const bool qok = qi < nq;
    const int qpos = min(first + qi, p.N - 1);
    const float *qrow = p.q + ((int64_t)(b * nq + (qok ? qi : 0)) * p.H + h) * kD;
    const float *cs = p.rope_f32 + (int64_t)qpos * kD;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * a + 4 * g4 + e;  // < 64
        const float c = cs[2 * i], sn = cs[2 * i + 1];
        const float x0 = qrow[i], x1 = qrow[i + kHalf];
        lo[e] = qok ? (x0 * c - x1 * sn) * p.scale_log2 : 0.f;
        hi[e] = qok ? (x0 * sn + x1 * c) * p.scale_log2 : 0.f;
      }
      const u32x4_t w = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                         pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
      qb[a] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // ---- A operand of K^T: W_up,k,t rows (dims 16 a' + l16), mu folded in ----
  // k-step ks, lane group g4: latent components 32 ks + 8 g4 + 0..7; the
  // group at component RK carries (mu_hi, mu_lo), later groups zeros.
  bf16x8_t wa[8][C::KS];
  {
    const uint16_t *W = reinterpret_cast<const uint16_t *>(p.wk) + (int64_t)h * kD * RK;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int dim = 16 * a + l16;
      const float mu = p.muk[(int64_t)h * kD + dim];
      const uint16_t mhi = f32_to_bf16_bits(mu);
      const uint16_t mlo = f32_to_bf16_bits(mu - bf16_bits_to_f32(mhi));
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        // unconditional (clamped) load, then the mu / zero groups selected
        const int k0 = 32 * ks + 8 * g4;
        u32x4_t w = *reinterpret_cast<const u32x4_t *>(W + (int64_t)dim * RK + min(k0, RK - 8));
        const uint32_t keep = k0 < RK ? ~0u : 0u;
        w[0] = (w[0] & keep) | (k0 == RK ? ((uint32_t)mhi | ((uint32_t)mlo << 16)) : 0u);
        w[1] &= keep;
        w[2] &= keep;
        w[3] &= keep;
        wa[a][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
  }

  // Byte offsets in a tile of this lane's 8-byte pieces for the transposing
  // reads of C_v: for value block v and slot half hh, lane l16 of group g4
  // reads slot 16 hh + 4 g4 + l16 / 4, columns 16 v + 4 (l16 % 4) + 0..3.
  // ds_read_b64_tr_b16 gives lane i of a 16-lane group element i % 4 of
  // the pieces of lanes i / 4 + 4 e (e = 0..3): column 16 v + i of the
  // group's four slots.
  uint32_t vofs[C::VB][2];
#pragma unroll
  for (int v = 0; v < C::VB; ++v)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int sl = 16 * hh + 4 * g4 + (l16 >> 2);
      const int c = C::KCH + 2 * v + ((l16 & 3) >> 1);
      vofs[v][hh] = (uint32_t)((sl * C::CPR + (c + sl / C::PER) % C::CPR) * 16 + 8 * (l16 & 1));
    }

  float m = -INFINITY, lsum = 0.f;  // query l16
  f32x4_t acc[C::VB];
#pragma unroll
  for (int v = 0; v < C::VB; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < ntiles; ++it) {
    const int tb = t0 + it * kTile;
    // tile it's latents (this wave) and phi rows (all waves) have landed,
    // and every wave is done with tile it - 1's buffers
    if (C::NS >= 3 && it + C::NS - 2 < ntiles)
      tile_barrier<C::LS>();
    else
      tile_barrier<0>();
    if (it + 1 < ntiles) issue_phi(it + 1);
    if (it + C::NS - 1 < ntiles) issue_lat(it + C::NS - 1);

    const char *st = ring + (it % C::NS) * C::STAGE;
    const uint32_t st_lds = (uint32_t)(uintptr_t)(LDS_AS const char *)st;
    const uint16_t *ph = reinterpret_cast<const uint16_t *>(lds + C::PHI_OFF + (it & 1) * kPhiTileBytes);

    // ---- S^T = K Q^T, one 16-slot half at a time ----
    f32x4_t sc[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const int js = 16 * sh + l16;  // slot in the tile
      const char *rec = st + js * C::CPR * 16;
      const int rot = js / C::PER;
      bf16x8_t kb[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        // every lane reads (groups past the K latent an in-record chunk whose
        // value is then replaced), so no read is conditional
        const int c = 4 * ks + g4;
        const int cr = c < C::CPR ? c : C::CPR - 1;
        u32x4_t v = *reinterpret_cast<const u32x4_t *>(rec + ((cr + rot) % C::CPR) * 16);
        if (ks == C::KS - 1) {
          const uint32_t keep = c < C::KCH ? ~0u : 0u;
          v[0] = (v[0] & keep) | (c == C::KCH ? 0x3F803F80u : 0u);
          v[1] &= keep;
          v[2] &= keep;
          v[3] &= keep;
        }
        kb[ks] = __builtin_bit_cast(bf16x8_t, v);
      }
      f32x4_t so = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          x0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a][ks], kb[ks], x0, 0, 0, 0);
          x1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a + 4][ks], kb[ks], x1, 0, 0, 0);
        }
        // phi element (k-step a, lane js + 32 (g4 / 2), 4 (g4 % 2) + e): cos of
        // frequency 16a + 4 g4 + e; four k-steps further its sin
        const uint16_t *pc = ph + ((a * 64 + js + 32 * (g4 >> 1)) * 8 + 4 * (g4 & 1));
        const u32x2_t cw = *reinterpret_cast<const u32x2_t *>(pc);
        const u32x2_t sw = *reinterpret_cast<const u32x2_t *>(pc + 4 * 64 * 8);
        const float co[4] = {bf16_lo(cw[0]), bf16_hi(cw[0]), bf16_lo(cw[1]), bf16_hi(cw[1])};
        const float sn[4] = {bf16_lo(sw[0]), bf16_hi(sw[0]), bf16_lo(sw[1]), bf16_hi(sw[1])};
        float r0[4], r1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r0[e] = x0[e] * co[e] - x1[e] * sn[e];
          r1[e] = x0[e] * sn[e] + x1[e] * co[e];
        }
        const u32x4_t kw = {pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]),
                            pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
        so = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), qb[a],
                                                     so, 0, 0, 0);
      }
      sc[sh] = so;
    }

    // ---- online softmax of query l16 over slots 16 sh + 4 g4 + i ----
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = tb + 16 * sh + 4 * g4 + i < t1;
        sv[4 * sh + i] = ok ? sc[sh][i] : -INFINITY;
        mx = fmaxf(mx, sv[4 * sh + i]);
      }
    mx = xor_max(mx);  // every tile holds a slot before t1: finite
    float alpha = 1.f;
    if (mx > m + kRescaleGap) {
      alpha = exp2f(m - mx);
      m = mx;
    }
    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // the hardware exp2 (arguments <= 8 or -inf; results below the normal
      // range flush to zero)
      pw[e] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2 * e] - m),
                          __builtin_amdgcn_exp2f(sv[2 * e + 1] - m));
      psum += bf16_lo(pw[e]) + bf16_hi(pw[e]);
    }
    lsum = fmaf(lsum, alpha, psum);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});

    // ---- acc^T += C_v^T P^T: value columns 16 v + l16, slots in lane order ----
    // two transposing LDS reads per value block: lane l16 receives column
    // 16 v + l16 of the four slots 4 g4 + 0..3 (then 16 + 4 g4 + 0..3), read
    // by the lanes of its 16-lane group as 8-byte pieces (vofs)
    uint32_t ta[2 * C::VB];
#pragma unroll
    for (int v = 0; v < C::VB; ++v) {
      ta[2 * v] = st_lds + vofs[v][0];
      ta[2 * v + 1] = st_lds + vofs[v][1];
    }
    tr_short4_t tv[2 * C::VB];
    lds_read_tr16_b64<2 * C::VB>(ta, tv);
#pragma unroll
    for (int v = 0; v < C::VB; ++v) {
      const tr_short4_t lo = tv[2 * v], hi = tv[2 * v + 1];
      const bf16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[v][i] *= alpha;
      acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, acc[v], 0, 0, 0);
    }
  }

  // ---- partials (m, l, sum p c_v) of query l16 ----
  const float l = xor_sum(lsum);
  if (!head_ok || l16 >= nq) return;
  float *part = part_at(l16);
  if (g4 == 0) {
    part[0] = m;
    part[1] = l;
  }
#pragma unroll
  for (int v = 0; v < C::VB; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[2 + 16 * v + 4 * g4 + i] = acc[v][i];
#endif
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
