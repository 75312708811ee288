// LLA-2D decode for bf16 latent stores on gfx950: one latent per token and
// layer decodes all H heads ("Looped Latent Attention: Cross-Loop KV
// Compression for Looped Transformers", Sec. 3, LLA-2D variant, with Eq. 3
// and "RoPE and reconstruction").  For sequence b, loop t and slot j <= pos:
//     k_h,j = RoPE(W_up,k,t[h] c_k,j + mu_k,t[h], j),  h = 0..H-1
//     s_h,j = scale * RoPE(q_h, pos) . k_h,j
// and the latent-space value average sum_j p_h,j c_v,j of every head.
//
// The K side is the same bilinear form as the per-head fast path, per head:
//     s_h,j = phi_j^T G_h c_k,j + phi_j^T g0_h
// (phi_j = [cos(j theta); sin(j theta)], G_h built from the rotated query
// and W_up,k,t rows of head h, g0_h from mu_k,t).  Here every head reads the
// SAME latent c_k,j, so one workgroup owns one (sequence, context split) and
// all H heads: the latent tile is streamed from HBM once and reused H times,
// which makes the path bound by the matrix cores, not by HBM.
//
// Eight waves, two per SIMD (one's vector work overlaps the other's matrix
// work); each wave holds G^T of its two heads (128 registers of packed bf16
// A operands) for the whole split.  Per 32-slot tile, wave w (heads 2w,
// 2w+1, one pair):
//  * U = G^T Phi^T on v_mfma_f32_32x32x16_bf16: r_k/16 row tiles x d/16
//    k-steps per pair.  Lane l owns slot l%32 of head 2w + l/32
//    and finds all r_k values of its head's column in its own accumulators;
//    the score is then an r_k-term dot with c_k.
//  * phi_j^T g0_h for all heads: eight v_mfma_f32_16x16x32_bf16 per tile
//    ((slot half) x (d quarter)), one per wave, partial sums exchanged
//    through LDS.
//  * online softmax per head over the 32 lanes of a half (lazy rescaling:
//    the running max moves only when a score exceeds it by kRescaleGap),
//    the weights rounded to bf16 and published in LDS.
//  * P C_v on v_mfma_f32_16x16x32_bf16: wave w owns value columns
//    16w..16w+15 of all heads (rows = heads, K = 32 slots).
// The three stages run as a software pipeline: one iteration computes the
// scores of tile it, the softmax of tile it-1 and P C_v of tile it-2, and
// the two waves of a SIMD take them in opposite orders so that matrix and
// vector work overlap.
// G is formed once per workgroup in LDS (32 latent components of every head
// at a time, transposed so that d is contiguous) and each lane then loads
// its 16-byte A fragments.
// One barrier per tile.  Latent tiles (NS = 5 LDS buffers, two in flight)
// and bf16 phi tiles (three buffers) arrive by buffer loads that write LDS
// directly; 16-byte chunks of a slot record are XOR-swizzled by slot
// (swz, swz_v) so that lanes reading different slots hit different banks.  The partial (m, l, sum p c_v) of every head goes to the
// workspace; the merge kernel applies W_up,v,t and mu_v,t batched over
// sequences.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace d2 {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kD = 128;
constexpr int kKSteps = kD / 16;
constexpr int kTile = 32;
constexpr int kPhiTileBytes = kTile * kD * 2;
constexpr int kLdsMax = 160 * 1024;
constexpr float kRescaleGap = 8.0f;
constexpr int kPPitch = 40;  // bf16 elements per head row of the P tile (80 B: bank spread)
// Store loads are nontemporal (nt): each latent is read once per call, the
// phi rows (default policy) by every workgroup.
constexpr int kCachePolicyStream = 2;

template <int RK, int RV>
struct Cfg {
  static constexpr int NW = 8;                        // waves (two per SIMD)
  static constexpr int HPW = 2;                       // heads per wave
  static constexpr int PAIRS = HPW / 2;
  static constexpr int H = NW * HPW;
  static constexpr int NT = 64 * NW;
  static constexpr int R = RK + RV;
  static constexpr int REC = 2 * R;                   // bytes per slot record
  static constexpr int CPT = REC / 16;                // 16-byte chunks per record
  static constexpr int CK = RK * 2 / 16;              // of which hold the K latent
  static constexpr int TILE_BYTES = kTile * REC;
  static constexpr int WLOADS = TILE_BYTES / 1024;    // 64-lane x 16 B loads per tile
  static constexpr int LW_MAX = (WLOADS + NW - 1) / NW;
  static constexpr int PHI_LOADS = kPhiTileBytes / 1024 / NW;
  static constexpr int MU_PIECES = 8 / NW;            // (slot half, d quarter) pieces per wave
  static constexpr int NS = 5;     // tiles it-2 .. it+2: stage C reads it-2, two in flight
  static constexpr int NPHI = 3;
  static constexpr int KT = RK / 16;
  static constexpr int VB = RV / 16 / NW;             // 16-column value blocks per wave
  static constexpr int OFF_PHI = NS * TILE_BYTES;
  static constexpr int OFF_MU = OFF_PHI + NPHI * kPhiTileBytes;
  static constexpr int MU_BUF = 4 * H * kTile * 4;    // [4 d-quarters][H][32 slots] fp32
  static constexpr int OFF_P = OFF_MU + 2 * MU_BUF;
  static constexpr int P_BUF = H * kPPitch * 2;
  static constexpr int OFF_ALPHA = OFF_P + 2 * P_BUF;
  static constexpr int OFF_AMU = OFF_ALPHA + 2 * H * 4;   // g0 A fragments [NW][pieces][64][16 B]
  static constexpr int PIPE_BYTES = OFF_AMU + NW * (8 / NW) * 64 * 16;
  static constexpr int WPITCH = kD + 8;               // LDS row pitch of G^T (elements)
  static constexpr int WSTAGE = H * 32 * WPITCH * 2;  // G^T for 32 k of every head, [h][k][i]
  static constexpr int SETUP_BYTES = WSTAGE + H * kD * 4;
  static constexpr int LDS_BYTES = PIPE_BYTES > SETUP_BYTES ? PIPE_BYTES : SETUP_BYTES;
  static_assert(H == 16, "heads = rows of the 16x16 MFMAs");
  static_assert(VB >= 1 && RV == 16 * VB * NW, "value columns split evenly over the waves");
  static_assert(RK % 32 == 0 && KT >= 2, "rank granularity (setup builds 32 k per round)");
  static_assert(CPT % 8 == 0 && CK % 8 == 0, "swizzles work on groups of 8 chunks");
  static_assert(TILE_BYTES % 1024 == 0 && PHI_LOADS >= 1 && MU_PIECES >= 1, "load split");
  static_assert(LDS_BYTES <= kLdsMax, "LDS");
  static_assert(H * (RV + 2) * 4 <= 2 * MU_BUF, "epilogue staging");
  static_assert(LW_MAX + PHI_LOADS <= 6, "vmcnt range of wait_vm_small");
  static_assert(OFF_AMU % 16 == 0 && PIPE_BYTES <= WSTAGE, "g0 fragments live below the queries");
};

// LDS placement of a slot record's 16-byte chunks.  K-latent chunks
// (lanes = 32 consecutive slots read the same chunk) are XOR-swizzled by
// swz(j); V-latent chunks (lanes = 16 columns of 4 slots 8 apart) by
// 2 ((j >> 3) & 3), which moves each 8-slot group to its own chunk pair and
// keeps the per-slot offsets of a gather a compile-time stride.
__device__ __forceinline__ int swz(int j) { return (j ^ (j >> 3)) & 7; }
__device__ __forceinline__ int swz_v(int j) { return 2 * ((j >> 3) & 3); }

// sc + sum_a u[a] * c[8 c0 + a]: the 16 latent values of chunks c0, c0+1
// of a (swizzled) slot record against one 32x32 accumulator column.  The
// accumulators are rounded to bf16 pairs and multiplied with the bf16
// latent pairs by v_dot2 (fp32 sums): half the vector instructions of
// unpacking every latent to fp32.  (The latent pairs are converted to
// uint32_t before the bit cast: a bit cast of a vector element directly
// has been miscompiled into a reuse of element 0.)
__device__ __forceinline__ float dot16(const f32x16_t &u, const char *rec, int c0, int fj,
                                       float sc) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t *>(rec + ((c0 ^ fj) * 16));
  const u32x4_t b = *reinterpret_cast<const u32x4_t *>(rec + (((c0 + 1) ^ fj) * 16));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const bf16x2_v ca = __builtin_bit_cast(bf16x2_v, (uint32_t)a[w]);
    const bf16x2_v cb = __builtin_bit_cast(bf16x2_v, (uint32_t)b[w]);
    const f32x2_v ua = {u[2 * w], u[2 * w + 1]}, ub = {u[8 + 2 * w], u[8 + 2 * w + 1]};
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_convertvector(ua, bf16x2_v), ca, sc, false);
    sc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_convertvector(ub, bf16x2_v), cb, sc, false);
  }
  return sc;
}

__device__ __forceinline__ void wait_vm_small(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(5)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
  }
}

template <int RK, int RV>
__global__ __launch_bounds__(512, 1) void decode2d_split(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<RK, RV>;
  constexpr int H = C::H, NW = C::NW, HPW = C::HPW;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x % p.S;
  const int vb = blockIdx.x / p.S;  // query (virtual sequence)

  const QuerySlot qs = query_slot(p, vb);
  const int b = qs.b, pos = qs.qpos;
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, qs.last + 1);
  float *part = p.ws + ((int64_t)vb * H * p.S + s) * (RV + 2);  // head h at + h * S * (RV + 2)
  if (t0 >= t1) {  // split entirely after the attended slots: empty partials
    for (int i = tid; i < H * (RV + 2); i += C::NT) {
      const int h = i / (RV + 2), r = i % (RV + 2);
      part[(int64_t)h * p.S * (RV + 2) + r] = (r == 0) ? -INFINITY : 0.f;
    }
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // ---- setup: rotated, scaled queries; G^T of this wave's heads; g0 rows ----
  const int row = lane & 31, khalf = lane >> 5;
  const int g4 = lane >> 4, l16 = lane & 15;
  float *qr = reinterpret_cast<float *>(lds + C::WSTAGE);  // [H][kD]
  {
    const float *rq = p.rope_f32 + (int64_t)pos * kD;
    for (int i = tid; i < H * (kD / 2); i += C::NT) {
      const int h = i / (kD / 2), ii = i % (kD / 2);
      const float *qb = p.q + ((int64_t)vb * H + h) * kD;
      const float c = rq[2 * ii], sn = rq[2 * ii + 1];
      const float a = qb[ii], bb = qb[ii + kD / 2];
      qr[h * kD + ii] = (a * c - bb * sn) * p.scale_log2;
      qr[h * kD + ii + kD / 2] = (a * sn + bb * c) * p.scale_log2;
    }
  }
  // A operands (packed bf16 pairs): row r of pair tile ti is head
  // HPW w + 2 pair + ((r >> 2) & 1), k = 16 ti + 4 (r >> 3) + (r & 3);
  // element e of k-step st is i = 16 st + 8 khalf + e.
  u32x4_t Ak[C::PAIRS][C::KT][kKSteps];
  uint16_t *gt = reinterpret_cast<uint16_t *>(lds);  // [H][32 k][WPITCH]: G^T, bf16
  // Round r forms G[h][i][k] for k in [32 r, 32 r + 32) of every head in
  // LDS (transposed, i contiguous), then every wave loads its row tiles
  // ti = 2 r, 2 r + 1 as 16-byte A fragments.
#pragma unroll
  for (int round = 0; round < C::KT / 2; ++round) {
    // 16 bytes of W_up,k,t = 8 consecutive k of one (h, i):
    //   G[i][k] = q'_i W[i][k] + q'_{i+d/2} W[i+d/2][k]      (i < d/2)
    //   G[i][k] = q'_i W[i-d/2][k] - q'_{i-d/2} W[i][k]      (i >= d/2)
    const uint16_t *w = reinterpret_cast<const uint16_t *>(p.wk) + 32 * round;
#pragma unroll 2
    for (int v = tid; v < H * kD * 4; v += C::NT) {
      const int hi = v >> 2, k0 = (v & 3) * 8;  // hi = h * kD + i
      const int h = hi / kD, i = hi % kD;
      const bool lo = i < kD / 2;
      const int ia = lo ? i : i - kD / 2, ib = lo ? i + kD / 2 : i;
      const u32x4_t wa = *reinterpret_cast<const u32x4_t *>(w + ((int64_t)h * kD + ia) * RK + k0);
      const u32x4_t wb = *reinterpret_cast<const u32x4_t *>(w + ((int64_t)h * kD + ib) * RK + k0);
      const float q1 = qr[h * kD + i];
      const float q2 = lo ? qr[h * kD + i + kD / 2] : -qr[h * kD + i - kD / 2];
      uint16_t *dst = gt + (h * 32 + k0) * C::WPITCH + i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t x = e & 1 ? (wa[e / 2] >> 16) : (wa[e / 2] & 0xFFFFu);
        const uint32_t y = e & 1 ? (wb[e / 2] >> 16) : (wb[e / 2] & 0xFFFFu);
        dst[e * C::WPITCH] = f32_to_bf16_bits(fmaf(q2, bf16_bits_to_f32(y),
                                                   q1 * bf16_bits_to_f32(x)));
      }
    }
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < C::PAIRS; ++pp) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int kk = tt * 16 + ((row >> 3) << 2) + (row & 3);  // k - 32 round
        const int h = HPW * wave + 2 * pp + ((row >> 2) & 1);
        const uint16_t *grow = gt + (h * 32 + kk) * C::WPITCH + 8 * khalf;
#pragma unroll
        for (int st = 0; st < kKSteps; ++st)
          Ak[pp][2 * round + tt][st] = *reinterpret_cast<const u32x4_t *>(grow + 16 * st);
      }
    }
    __syncthreads();
  }
  // g0 rows for the mu term: wave w computes the (slot half cb, d quarter
  // ks) pieces c = w + NW v of the eight, for all 16 heads.  They are kept
  // in LDS (read once per tile) rather than in registers.
  u32x4_t *amu_l = reinterpret_cast<u32x4_t *>(lds + C::OFF_AMU) + (wave * C::MU_PIECES) * 64 + lane;
#pragma unroll
  for (int v = 0; v < C::MU_PIECES; ++v) {
    const int c = wave + NW * v, ks = c >> 1;
    const float *qh = qr + l16 * kD;
    const float *mu = p.muk + (int64_t)l16 * kD;
    float gv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 32 * ks + 8 * g4 + e;
      gv[e] = (i < kD / 2) ? qh[i] * mu[i] + qh[i + kD / 2] * mu[i + kD / 2]
                           : qh[i] * mu[i - kD / 2] - qh[i - kD / 2] * mu[i];
    }
    u32x4_t frag;
#pragma unroll
    for (int w = 0; w < 4; ++w) frag[w] = pack_bf16x2(gv[2 * w], gv[2 * w + 1]);
    amu_l[v * 64] = frag;
  }
  __syncthreads();  // the setup LDS is reused by the pipeline

  // ---- streaming setup ----
  const int64_t slab_elems = (int64_t)p.N * C::R;
  const uint16_t *slab = reinterpret_cast<const uint16_t *>(p.store) +
                         ((int64_t)b * p.D + p.layer) * slab_elems;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(slab), (short)0, (int)(slab_elems * 2), 0x00020000);
  const int phi_tiles = (p.N + kTile - 1) / kTile;
  const __amdgpu_buffer_rsrc_t rphi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.rope_bf16), (short)0, phi_tiles * kPhiTileBytes, 0x00020000);
  // this wave's store loads: wave-load indices n = wave + u * NW < WLOADS
  const int LW = (C::WLOADS - wave + NW - 1) / NW;
  uint32_t voff[C::LW_MAX];
#pragma unroll
  for (int u = 0; u < C::LW_MAX; ++u) {
    const int P = (wave + u * NW) * 64 + lane;
    const int tj = P / C::CPT, q = P % C::CPT;
    voff[u] = tj * C::REC + (uint32_t)((q ^ (q < C::CK ? swz(tj) : swz_v(tj))) * 16);
  }
  auto issue_store = [&](int t) {
    char *sb = lds + (t % C::NS) * C::TILE_BYTES;
    const uint32_t toff = (uint32_t)(t0 + t * kTile) * C::REC;
#pragma unroll
    for (int u = 0; u < C::LW_MAX; ++u)
      if (u < LW)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (LDS_AS void *)(sb + (wave + u * NW) * 1024), 16, voff[u] + toff, 0, 0,
            kCachePolicyStream);
  };
  // phi tile (8 KB = 8 wave loads): wave w loads blocks w + NW u
  auto issue_phi = [&](int t) {
    char *pb = lds + C::OFF_PHI + (t % C::NPHI) * kPhiTileBytes;
    const uint32_t off = (uint32_t)(t0 / kTile + t) * kPhiTileBytes;
#pragma unroll
    for (int u = 0; u < C::PHI_LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rphi, (LDS_AS void *)(pb + (wave + u * NW) * 1024), 16,
          off + (uint32_t)((wave + u * NW) * 64 + lane) * 16, 0, 0, 0);
  };

  // phi_j^T g0_h for tile t into mu buffer t & 1: [ks][h][slot]
  auto mu_step = [&](int t) {
    const char *pb = lds + C::OFF_PHI + (t % C::NPHI) * kPhiTileBytes;
    float *mb = reinterpret_cast<float *>(lds + C::OFF_MU + (t & 1) * C::MU_BUF);
#pragma unroll
    for (int v = 0; v < C::MU_PIECES; ++v) {
      const int c = wave + NW * v, ks = c >> 1, cb = c & 1;
      const bf16x8_t bm = *reinterpret_cast<const bf16x8_t *>(
          pb + ((2 * ks + (g4 >> 1)) * 64 + 16 * cb + l16 + 32 * (g4 & 1)) * 16);
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, amu_l[v * 64]), bm,
                                                   o, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) mb[(ks * H + 4 * g4 + i) * kTile + 16 * cb + l16] = o[i];
    }
  };

  // P C_v of tile t for value columns 16 (VB w + v) + 0..15 of every head
  f32x4_t pv[C::VB];
#pragma unroll
  for (int v = 0; v < C::VB; ++v) pv[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto pv_step = [&](int t) {
    const uint16_t *P = reinterpret_cast<const uint16_t *>(lds + C::OFF_P + (t & 1) * C::P_BUF);
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(P + l16 * kPPitch + 8 * g4);
    const char *sb = lds + (t % C::NS) * C::TILE_BYTES;
    const f32x4_t al = *reinterpret_cast<const f32x4_t *>(
        reinterpret_cast<const float *>(lds + C::OFF_ALPHA + (t & 1) * H * 4) + 4 * g4);
    // slots past the attended ones (only in the last tile) may hold
    // anything, NaN included, so their C_v is zeroed there
    const bool full = t0 + (t + 1) * kTile <= t1;  // workgroup-uniform
#pragma unroll
    for (int v = 0; v < C::VB; ++v) {
      const int comp = RK + 16 * (C::VB * wave + v) + l16;
      // slots 8 g4 + e share swz_v = 2 g4: one base address, stride REC
      const char *gb = sb + 8 * g4 * C::REC + (((comp >> 3) ^ (2 * g4)) * 16) + (comp & 7) * 2;
      bf16x8_t bv;
      if (full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = *reinterpret_cast<const short *>(gb + e * C::REC);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sl = 8 * g4 + e;
          const uint16_t x = *reinterpret_cast<const uint16_t *>(gb + e * C::REC);
          bv[e] = (t0 + t * kTile + sl < t1) ? (short)x : (short)0;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[v][i] *= al[i];
      pv[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, pv[v], 0, 0, 0);
    }
  };

  // ---- per-lane softmax state: slot residue l%32 of head 4w + 2 pair + l/32 ----
  float m[C::PAIRS], lsum[C::PAIRS];
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) {
    m[pp] = -INFINITY;
    lsum[pp] = 0.f;
  }

  // ---- prologue ----
  issue_store(0);
  issue_phi(0);
  if (ntiles > 1) {
    issue_phi(1);
    issue_store(1);
  }
  wait_vm_small(ntiles > 1 ? C::PHI_LOADS + LW : 0);  // store(0), phi(0) have landed
  lds_barrier();  // (a __syncthreads() would also wait for store(1), phi(1))

  const int j = lane & 31;
  const int fj = swz(j);

  // Stage A(t): K-side MFMA chains of tile t and the dots with c_k -> sc.
  auto stage_scores = [&](int t, float (&sc)[C::PAIRS]) {
    const char *sb = lds + (t % C::NS) * C::TILE_BYTES;
    const char *phb = lds + C::OFF_PHI + (t % C::NPHI) * kPhiTileBytes;
    const char *rec = sb + j * C::REC;
#pragma unroll
    for (int pp = 0; pp < C::PAIRS; ++pp) {
      // phi fragments of the tile: read from LDS once per pair, reused by
      // every row tile (LDS bandwidth is as scarce as registers here)
      bf16x8_t bphi[kKSteps];
#pragma unroll
      for (int st = 0; st < kKSteps; ++st)
        bphi[st] = *reinterpret_cast<const bf16x8_t *>(phb + (st * 64 + lane) * 16);
      float acc = 0.f;
#pragma unroll
      for (int ti = 0; ti < C::KT; ++ti) {
        f32x16_t u = {};
#pragma unroll
        for (int st = 0; st < kKSteps; ++st)
          u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, Ak[pp][ti][st]),
                                                      bphi[st], u, 0, 0, 0);
        // accumulator a of row tile ti is k = 16 ti + a of this lane's head
        acc = dot16(u, rec, 2 * ti, fj, acc);
      }
      sc[pp] = acc;
    }
  };

  // Stage B(t): mu term, online softmax of every head -> P(t), alpha(t).
  auto stage_softmax = [&](int t, const float (&sc)[C::PAIRS]) {
    const float *mb = reinterpret_cast<const float *>(lds + C::OFF_MU + (t & 1) * C::MU_BUF);
    uint16_t *Pw = reinterpret_cast<uint16_t *>(lds + C::OFF_P + (t & 1) * C::P_BUF);
    float *Aw = reinterpret_cast<float *>(lds + C::OFF_ALPHA + (t & 1) * H * 4);
    const bool valid = (t0 + t * kTile + j) < t1;
#pragma unroll
    for (int pp = 0; pp < C::PAIRS; ++pp) {
      const int hsel = HPW * wave + 2 * pp + khalf;
      float s = sc[pp];
#pragma unroll
      for (int q = 0; q < 4; ++q) s += mb[(q * H + hsel) * kTile + j];
      s = valid ? s : -INFINITY;
      // online softmax of head hsel over the 32 lanes of this half
      float alpha = 1.f;
      if (__any(s > m[pp] + kRescaleGap)) {
        float tm = s;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) tm = fmaxf(tm, __shfl_xor(tm, o, 64));
        if (tm > m[pp] + kRescaleGap) {
          alpha = exp2f(m[pp] - tm);
          m[pp] = tm;
        }
      }
      const float pe = valid ? exp2f(s - m[pp]) : 0.f;
      const uint16_t pb16 = f32_to_bf16_bits(pe);
      lsum[pp] = fmaf(lsum[pp], alpha, bf16_bits_to_f32(pb16));
      Pw[hsel * kPPitch + j] = pb16;
      if (j == 0) Aw[hsel] = alpha;
    }
  };

  // Software pipeline over tiles: iteration it runs A(it) (with the mu term
  // of tile it), B(it - 1) and C(it - 2) = pv_step; one barrier per
  // iteration publishes mu(it) and P(it - 1).  The two waves that share a
  // SIMD take the stages in opposite orders (matrix work first, vector work
  // first), so that one's MFMA chains overlap the other's softmax and
  // gathers.
  const bool mfma_first = wave < NW / 2;
  float scp[C::PAIRS];  // scores of tile it - 1, waiting for stage B
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) scp[pp] = 0.f;
  for (int it = 0; it < ntiles + 2; ++it) {
    if (it + 2 < ntiles) {
      issue_phi(it + 2);
      issue_store(it + 2);
    }
    float scc[C::PAIRS];
    if (mfma_first) {
      if (it < ntiles) {
        mu_step(it);
        stage_scores(it, scc);
      }
      if (it >= 1 && it <= ntiles) stage_softmax(it - 1, scp);
      if (it >= 2) pv_step(it - 2);
    } else {
      if (it >= 1 && it <= ntiles) stage_softmax(it - 1, scp);
      if (it >= 2) pv_step(it - 2);
      if (it < ntiles) {
        mu_step(it);
        stage_scores(it, scc);
      }
    }
#pragma unroll
    for (int pp = 0; pp < C::PAIRS; ++pp) scp[pp] = scc[pp];
    wait_vm_small(it + 2 < ntiles ? C::PHI_LOADS + LW : 0);  // store(it+1), phi(it+1)
    // LDS-only barrier: a __syncthreads() would also wait for store(it+2)
    // and phi(it+2), issued at the top of this iteration, and so cut the
    // prefetch to one iteration.
    lds_barrier();
  }

  // ---- partials (m, l, sum p c_v) of every head ----
  __syncthreads();  // everyone is done with the mu buffers
  float *comb = reinterpret_cast<float *>(lds + C::OFF_MU);  // [H][RV + 2]
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) {
    float l = lsum[pp];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    const int hsel = HPW * wave + 2 * pp + khalf;
    if (j == 0) {
      comb[hsel * (RV + 2)] = m[pp];
      comb[hsel * (RV + 2) + 1] = l;
    }
  }
#pragma unroll
  for (int v = 0; v < C::VB; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      comb[(4 * g4 + i) * (RV + 2) + 2 + 16 * (C::VB * wave + v) + l16] = pv[v][i];
  __syncthreads();
  for (int i = tid; i < H * (RV + 2); i += C::NT) {
    const int h = i / (RV + 2), r = i % (RV + 2);
    part[(int64_t)h * p.S * (RV + 2) + r] = comb[i];
  }
#endif
}

template <int RK, int RV>
hipError_t launch(const DecodeParams &p, hipStream_t st) {
  using C = Cfg<RK, RV>;
  const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&decode2d_split<RK, RV>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode2d_split<RK, RV>), dim3(p.B * p.S), dim3(C::NT), C::LDS_BYTES, st,
                     p);
  return hipGetLastError();
}

}  // namespace d2

bool decode2d_mfma_supported(int32_t H, int32_t d, int32_t rk, int32_t rv) {
  return H == 16 && d == d2::kD && rk == 64 && rv == 128;
}

hipError_t launch_decode2d_mfma(const DecodeParams &p, hipStream_t st) {
  if (p.rk == 64 && p.rv == 128 && p.H == 16) return d2::launch<64, 128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace lla
