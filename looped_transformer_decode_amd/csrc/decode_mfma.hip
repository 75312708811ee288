// Per-head LLA decode for bf16 latent stores on gfx950 (the fast path).
//
// What it computes ("Looped Latent Attention: Cross-Loop KV Compression for
// Looped Transformers", Sec. 3 Eq. 3 and "RoPE and reconstruction"): for
// sequence b, head h, loop t and every slot j <= pos[b]
//     s_j = scale * RoPE(q, pos) . RoPE(W_up,k,t c_k,j + mu_k,t, j)
// followed by an online softmax and the latent-space value average
// sum_j p_j c_v,j; W_up,v,t and mu_v,t are applied once at the end (here
// when the context is not split, else by the merge kernel).
//
// How.  RoPE is a rotation by j*theta_i of each pair (i, i + d/2), so with
// phi_j = [cos(j theta); sin(j theta)] in R^d the score is bilinear in the
// rotary row phi_j and the stored latent c_j:
//     s_j = phi_j^T G c_j + phi_j^T g0,
//     G[i, k]       = q'_i W[i, k] + q'_{i+d/2} W[i+d/2, k]
//     G[i+d/2, k]   = q'_{i+d/2} W[i, k] - q'_i W[i+d/2, k]      (i < d/2)
// with q' the rotated, scaled query and g0 the same expression with mu_k,t
// in place of W[:, k].  G is built once per workgroup; per tile of 32 slots
// one MFMA chain U = G^T Phi^T (rows (head, k), columns = slots, K = d)
// yields phi_j^T G[:, k] for every slot, and the score is the rank-r_k dot
// product of U's column with the slot's latent.  Reconstruction, RoPE and
// the q.k product thereby run on the matrix cores (the K-side work is the
// same tokens x d x r_k contraction as reconstructing K), leaving the
// vector ALUs an r_k-term dot, the softmax and the r_v-term value update
// per (slot, head).  Row order of G^T is chosen so that lane l of a 32x32
// MFMA output holds all r_k values of slot l%32 for one head: lanes 0-31
// serve the first head of a pair, lanes 32-63 the second, so no cross-lane
// reduction is needed anywhere in the slot loop.
//
// Data movement.  A workgroup owns (b, head group, context split): 16 heads
// in 8 waves (two per SIMD) for r_k + r_v = 48, 8 heads in 4 waves for the
// larger ranks, whose 32-slot tiles would not fit LDS three deep.  Slot
// records of the head group are contiguous in HBM; tiles of 32 slots are
// streamed with nontemporal buffer loads that write LDS directly (no VGPR
// staging), three or two tiles deep, plus the matching 8 KB tile of bf16 phi
// rows; where LDS allows, the first tiles are already streaming while G is
// built.
// 16-byte chunks are XOR-swizzled by (slot & 7) inside each slot record so
// that the per-lane record reads (lanes = consecutive slots) hit distinct
// LDS banks.  Buffer loads past the slab return zeros, so partial tiles
// never read outside the store.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace detail {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kD = 128;             // d_head served by this path
constexpr int kKSteps = kD / 16;    // k-steps of v_mfma_f32_32x32x16_bf16
constexpr int kTile = 32;           // slots per tile (MFMA column count)
constexpr int kPhiTileBytes = kTile * kD * 2;
constexpr int kLdsMax = 160 * 1024;
constexpr float kRescaleGap = 8.0f; // log2-domain headroom before rescaling
// G^T rows in LDS: kD + 8 bf16 (272 bytes, so that consecutive rows start 16
// bytes apart in bank space) and 32 more between heads, so that the two heads
// a wave's 16-byte operand reads touch at once fall in different banks.
constexpr int kGPitch = kD + 8;
constexpr int kGHeadPad = 32;
// Cache policy of the store loads: nontemporal (nt).  Every store byte is
// read once per call; the hint keeps the stream from displacing the phi
// rows and codec matrices that all workgroups share in L2 (measured: 5.96
// -> 6.25 TB/s at the extreme-batch shape).  The phi tiles use the default.
constexpr int kCachePolicyStream = 2;

template <int RK, int RV, int HPW, int NW>
struct Cfg {
  static constexpr int HG = HPW * NW;           // heads per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int REC = (RK + RV) * 2;     // bytes per (slot, head)
  static constexpr int CPH = REC / 16;          // 16-byte chunks per head record
  static constexpr int CPT = HG * CPH;          // chunks per slot of the group
  static constexpr int TILE_BYTES = kTile * CPT * 16;
  // Store tiles are prefetched NS-1 tiles ahead; the (L2-resident) phi
  // tiles one tile ahead in two buffers of their own.
  static constexpr int NS_FIT = (kLdsMax - 2 * kPhiTileBytes) / TILE_BYTES;
  static constexpr int NS = NS_FIT > 3 ? 3 : NS_FIT;
  static constexpr int PHI_OFF = NS * TILE_BYTES;
  static constexpr int LDS_BYTES = PHI_OFF + 2 * kPhiTileBytes;
  static constexpr int LS = kTile * CPT / NT;             // store loads per thread per tile
  static constexpr int LP = (kPhiTileBytes / 16) / NT;    // phi loads per thread per tile
  static constexpr int PAIRS = HPW / 2;
  static constexpr int KT = RK / 16;            // 32-row MFMA tiles per head pair
  static constexpr int CK_CHUNKS = RK / 8;
  static constexpr int CV_CHUNKS = RV / 8;
  static_assert(HPW % 2 == 0 && HPW <= 4, "heads per wave: 2 or 4");
  static_assert(RK % 16 == 0 && RV % 8 == 0, "rank granularity");
  static_assert(CPT % 8 == 0, "swizzle works on groups of 8 chunks");
  static_assert((kTile * CPT) % NT == 0 && (kPhiTileBytes / 16) % NT == 0, "load split");
  static_assert(NS >= 2, "two store stages must fit");
  static_assert(2 * LS + LP <= 63, "vmcnt range");
  // Setup staging: G^T of the group as bf16 rows of kGPitch elements, heads
  // G_HEAD elements apart, then the g0 rows, then the rotated queries (fp32).
  // When it fits between the first store stage and the phi buffers, the
  // first store and phi tiles stream in while G is built (EARLY); otherwise
  // it starts at 0 and the tiles are issued after it.
  static constexpr int G_HEAD = RK * kGPitch + kGHeadPad;
  static constexpr int SETUP_BYTES = (HG * G_HEAD + HG * kGPitch) * 2 + HG * kD * 4;
  static constexpr bool EARLY = TILE_BYTES + SETUP_BYTES <= PHI_OFF;
  static constexpr int SETUP_OFF = EARLY ? TILE_BYTES : 0;
  static_assert(SETUP_OFF + SETUP_BYTES <= (EARLY ? PHI_OFF : LDS_BYTES), "setup staging");
  // G blocks: (head, 8 k's, 8 i's of the first half) per item
  static constexpr int ITEMS = HG * (RK / 8) * (kD / 16);
  static constexpr int P1_PER_THREAD = (HG * (kD / 2) + NT - 1) / NT;  // (head, i < 64) pairs
  static_assert(!EARLY || ITEMS <= NT, "EARLY: one G item per thread, loaded before the first tile");
  // Final reduction: the 32 lanes' rescaled (l, acc) of every head, [HG][RV+1][32],
  // the head maxima [HG], then the combined partials [HG][RV+2].
  static constexpr int RED_FLOATS = HG * (RV + 1) * 32;
  static_assert((RED_FLOATS + HG + HG * (RV + 2)) * 4 <= LDS_BYTES, "reduction staging");
  static_assert(RV % 8 == 0, "W_up,v,t rows are read as 16-byte vectors");
  static constexpr int OUT_PER_THREAD = HG * kD / NT;  // W_up,v,t outputs per thread
  static_assert(OUT_PER_THREAD * NT == HG * kD, "output split");
  // W_up,v,t rows fetched before the final reduction when they fit in 64 VGPRs
  static constexpr bool WV_AHEAD = OUT_PER_THREAD * (RV / 8) * 4 <= 64;
};

// Wait until at most n vector-memory operations are outstanding (0 <= n
// <= 63); s_waitcnt takes an immediate, so dispatch over the values.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define LLA_W(k) case k: __builtin_amdgcn_s_waitcnt(waitcnt_vm(k)); break;
#define LLA_W8(k) LLA_W(k) LLA_W(k + 1) LLA_W(k + 2) LLA_W(k + 3) LLA_W(k + 4) LLA_W(k + 5) \
    LLA_W(k + 6) LLA_W(k + 7)
    LLA_W8(0) LLA_W8(8) LLA_W8(16) LLA_W8(24) LLA_W8(32) LLA_W8(40) LLA_W8(48) LLA_W8(56)
#undef LLA_W8
#undef LLA_W
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
}

// lgkmcnt(0), other counters untouched.
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

template <int RK, int RV, int HPW, int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_split(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only builtin types
  using C = Cfg<RK, RV, HPW, NW>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int groups = p.H / C::HG;
  int bid = blockIdx.x;
  const int s = bid % p.S;
  bid /= p.S;
  const int g = bid % groups;
  const int vb = bid / groups;  // query (virtual sequence)
  const int h0 = g * C::HG;

  const QuerySlot qs = query_slot(p, vb);
  const int b = qs.b;  // stored sequence
  const int pos = qs.qpos;
  const int t0 = s * p.split_len;
  const int t1 = min(t0 + p.split_len, qs.last + 1);
  if (t0 >= t1) {  // split entirely after the attended slots: empty partials
    for (int i = tid; i < C::HG * (RV + 2); i += C::NT) {
      const int hl = i / (RV + 2), r = i % (RV + 2);
      p.ws[((int64_t)(vb * p.H + h0 + hl) * p.S + s) * (RV + 2) + r] = (r == 0) ? -INFINITY : 0.f;
    }
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // ---- tile streaming setup ----
  const int64_t slab_elems = (int64_t)p.N * p.Hs * p.R;
  const uint16_t *slab = reinterpret_cast<const uint16_t *>(p.store) +
                         ((int64_t)b * p.D + p.layer) * slab_elems;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(slab), (short)0, (int)(slab_elems * 2), 0x00020000);
  const int phi_tiles = (p.N + kTile - 1) / kTile;
  const __amdgpu_buffer_rsrc_t rphi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.rope_bf16), (short)0, phi_tiles * kPhiTileBytes, 0x00020000);
  const uint32_t tok_stride = (uint32_t)p.Hs * p.R * 2;  // bytes per slot in the slab
  const uint32_t grp_off = (uint32_t)h0 * C::REC;
  uint32_t voff[C::LS];
#pragma unroll
  for (int n = 0; n < C::LS; ++n) {
    const int P = n * C::NT + tid;           // LDS chunk this lane fills
    const int tj = P / C::CPT, qq = P % C::CPT;
    voff[n] = tj * tok_stride + grp_off + (uint32_t)((qq ^ (tj & 7)) * 16);
  }
  // Workgroups start at different tiles of their slabs (the online softmax
  // does not depend on the order): tile it of the loop is slab tile rot(it).
  // Workgroups that start together then read different parts of their slabs
  // instead of marching in step (measured: 768.7 -> 752.7 us at B = 768).
  const int tile_shift = ntiles > 1 ? (int)((blockIdx.x * 37u) % (unsigned)ntiles) : 0;
  auto rot = [&](int it) { const int t = it + tile_shift; return t < ntiles ? t : t - ntiles; };
  auto issue_store = [&](int it) {
    char *sb = lds + (it % C::NS) * C::TILE_BYTES;
    const uint32_t tile_off = (uint32_t)(t0 + rot(it) * kTile) * tok_stride;
#pragma unroll
    for (int n = 0; n < C::LS; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (LDS_AS void *)(sb + (n * C::NT + wave * 64) * 16), 16, voff[n] + tile_off, 0, 0,
          kCachePolicyStream);
  };
  auto issue_phi = [&](int it) {
    char *pb = lds + C::PHI_OFF + (it & 1) * kPhiTileBytes;
    const uint32_t phi_off = (uint32_t)(t0 / kTile + rot(it)) * kPhiTileBytes;
#pragma unroll
    for (int n = 0; n < C::LP; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rphi, (LDS_AS void *)(pb + (n * C::NT + wave * 64) * 16), 16,
          phi_off + (uint32_t)(n * C::NT + tid) * 16, 0, 0, 0);
  };


  // ---- setup: G^T and g0 of the group, bf16, in LDS ----
  // Pass 1, one thread per (head hl, i < 64): q' = RoPE(q, pos) * scale at i
  // and i + 64 into qr, g0 at i and i + 64 into g0t.  Pass 2, one item per
  // (head hl, k block k0..k0+7, i block i0..i0+7 < 64): the 16 rows W[i0 + ii]
  // and W[i0 + 64 + ii] (8 k's each, one 16-byte load per row) give the 8 x 8
  // blocks of G^T at columns i0 and i0 + 64, written as 16-byte rows.  All
  // global loads of both passes are issued first; with EARLY the first store
  // and phi tiles are issued right after them and stream in during the rest.
  uint16_t *gt = reinterpret_cast<uint16_t *>(lds + C::SETUP_OFF);  // [HG][RK][kGPitch] (+pad)
  uint16_t *g0t = gt + C::HG * C::G_HEAD;                             // [HG][kGPitch]
  float *qr = reinterpret_cast<float *>(g0t + C::HG * kGPitch);       // [HG][kD]
  {
    // Indexes past the last (head, i) pair or G item are clamped to it: every
    // load is valid and such threads write the same values to the same LDS
    // words as the thread that owns them, so no step is conditional.
    float qin[C::P1_PER_THREAD][2], mkin[C::P1_PER_THREAD][2];
    float2 csin[C::P1_PER_THREAD];
#pragma unroll
    for (int n = 0; n < C::P1_PER_THREAD; ++n) {
      const int o = min(n * C::NT + tid, C::HG * (kD / 2) - 1);
      const int hl = o / (kD / 2), i = o % (kD / 2);
      const float *qb = p.q + ((int64_t)vb * p.H + h0 + hl) * kD;
      const float *mu = p.muk + (int64_t)(h0 + hl) * kD;
      qin[n][0] = qb[i];
      qin[n][1] = qb[i + kD / 2];
      mkin[n][0] = mu[i];
      mkin[n][1] = mu[i + kD / 2];
      csin[n] = reinterpret_cast<const float2 *>(p.rope_f32 + (int64_t)pos * kD)[i];
    }
    auto item_w = [&](int j, u32x4_t (&wlo)[8], u32x4_t (&whi)[8]) {
      const int ib = j % 8, kb = (j / 8) % (RK / 8), hl = j / RK;
      const uint16_t *wb = reinterpret_cast<const uint16_t *>(p.wk) +
                           ((int64_t)(h0 + hl) * kD + 8 * ib) * RK + 8 * kb;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        wlo[ii] = *reinterpret_cast<const u32x4_t *>(wb + ii * RK);
        whi[ii] = *reinterpret_cast<const u32x4_t *>(wb + (ii + kD / 2) * RK);
      }
    };
    u32x4_t wlo[8], whi[8];
    item_w(min(tid, C::ITEMS - 1), wlo, whi);
    if constexpr (C::EARLY) {
      __builtin_amdgcn_sched_barrier(0);  // the setup loads go out before the tiles
      issue_store(0);                     // ntiles >= 1 here
      issue_phi(0);
    }
#pragma unroll
    for (int n = 0; n < C::P1_PER_THREAD; ++n) {
      const int o = min(n * C::NT + tid, C::HG * (kD / 2) - 1);
      const int hl = o / (kD / 2), i = o % (kD / 2);
      const float cn = csin[n].x, sn = csin[n].y, a = qin[n][0], bb = qin[n][1];
      const float qa = (a * cn - bb * sn) * p.scale_log2;  // q' at i
      const float qc = (a * sn + bb * cn) * p.scale_log2;  // q' at i + 64
      qr[hl * kD + i] = qa;
      qr[hl * kD + i + kD / 2] = qc;
      // g0 = G with mu_k,t in place of W[:, k]
      g0t[hl * kGPitch + i] = f32_to_bf16_bits(qa * mkin[n][0] + qc * mkin[n][1]);
      g0t[hl * kGPitch + i + kD / 2] = f32_to_bf16_bits(qc * mkin[n][0] - qa * mkin[n][1]);
    }
    lds_barrier();  // the first tiles may still be in flight
    auto item_build = [&](int j, const u32x4_t (&wlo)[8], const u32x4_t (&whi)[8]) {
      const int ib = j % 8, kb = (j / 8) % (RK / 8), hl = j / RK;
      const int i0 = 8 * ib, k0 = 8 * kb;
      float qa[8], qc[8];  // q' at i0 + ii and i0 + 64 + ii
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        qa[ii] = qr[hl * kD + i0 + ii];
        qc[ii] = qr[hl * kD + i0 + ii + kD / 2];
      }
      uint16_t *gh = gt + hl * C::G_HEAD;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        u32x4_t vlo, vhi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float glo[2], ghi[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int ii = 2 * e + h;
            const uint32_t pa = wlo[ii][kk / 2], pb = whi[ii][kk / 2];
            const float wa = (kk & 1) ? bf16_hi(pa) : bf16_lo(pa);
            const float wc = (kk & 1) ? bf16_hi(pb) : bf16_lo(pb);
            glo[h] = qa[ii] * wa + qc[ii] * wc;  // G[i0 + ii, k]
            ghi[h] = qc[ii] * wa - qa[ii] * wc;  // G[i0 + 64 + ii, k]
          }
          vlo[e] = pack_bf16x2(glo[0], glo[1]);
          vhi[e] = pack_bf16x2(ghi[0], ghi[1]);
        }
        *reinterpret_cast<u32x4_t *>(gh + (k0 + kk) * kGPitch + i0) = vlo;
        *reinterpret_cast<u32x4_t *>(gh + (k0 + kk) * kGPitch + i0 + kD / 2) = vhi;
      }
    };
    if constexpr (C::EARLY) {
      item_build(min(tid, C::ITEMS - 1), wlo, whi);
    } else {
      for (int j = tid; j < C::ITEMS; j += C::NT) {
        if (j != tid) item_w(j, wlo, whi);
        item_build(j, wlo, whi);
      }
    }
  }
  lds_barrier();

  // ---- A operands: G^T rows (per head pair) and the mu row block ----
  const int row = lane & 31, khalf = lane >> 5;
  bf16x8_t Ak[C::PAIRS][C::KT][kKSteps];
  bf16x8_t Amu[kKSteps];
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) {
#pragma unroll
    for (int ti = 0; ti < C::KT; ++ti) {
      const int hip = (row >> 2) & 1;
      const int k = ti * 16 + ((row >> 3) << 2) + (row & 3);
      const int hl = wave * HPW + 2 * pp + hip;
      const uint16_t *src = gt + hl * C::G_HEAD + k * kGPitch + 8 * khalf;
#pragma unroll
      for (int st = 0; st < kKSteps; ++st)
        Ak[pp][ti][st] = *reinterpret_cast<const bf16x8_t *>(src + 16 * st);
    }
  }
  {
    // mu rows: row 8*pp + 4*hip (pp < PAIRS) carries head wave*HPW + 2*pp + hip;
    // an output lane l then finds its head's mu term in accumulator 4*pp.
    const bool used = ((row & 3) == 0) && ((row >> 3) < C::PAIRS);
    const int hl = used ? wave * HPW + 2 * (row >> 3) + ((row >> 2) & 1) : 0;
    const uint16_t *src = g0t + hl * kGPitch + 8 * khalf;
#pragma unroll
    for (int st = 0; st < kKSteps; ++st) {
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t *>(src + 16 * st);
      Amu[st] = used ? v : bf16x8_t{};
    }
  }
  lds_barrier();  // the setup LDS area is reused by the pipeline stages

  // ---- online-softmax state: per lane (slot residue l%32, head of the pair) ----
  float m[C::PAIRS], l[C::PAIRS], acc[C::PAIRS][RV];
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) {
    m[pp] = -INFINITY;
    l[pp] = 0.f;
#pragma unroll
    for (int r = 0; r < RV; ++r) acc[pp][r] = 0.f;
  }

  // Issue order: iteration it issues phi(it+1), then store(it+NS-1), right
  // after the barrier that shows every wave is done with tile it-1 (whose
  // buffers they reuse).  The prologue issues the stores before tile NS-1
  // and phi(0), in the order the iterations would have (with EARLY, store(0)
  // and phi(0) were issued before the setup).
  if constexpr (C::EARLY) {
    for (int k = 1; k + 2 < C::NS; ++k)
      if (k < ntiles) issue_store(k);
  } else {
    for (int k = 0; k + 2 < C::NS; ++k)
      if (k < ntiles) issue_store(k);
    issue_phi(0);
  }
  if (C::NS - 2 < ntiles && (C::NS > 2 || !C::EARLY)) issue_store(C::NS - 2);

  const int tj = lane & 31;
  const int swz = tj & 7;
  for (int it = 0; it < ntiles; ++it) {
    // Wait for store(it) and phi(it): what was issued after phi(it) may stay
    // outstanding (loads complete in issue order): store(it+NS-2), issued
    // right after it.
    wait_vm(it + C::NS - 2 < ntiles && C::NS >= 3 ? C::LS : 0);
    __builtin_amdgcn_s_barrier();
    if (it + 1 < ntiles) issue_phi(it + 1);
    if (it + C::NS - 1 < ntiles) issue_store(it + C::NS - 1);

    const char *sb = lds + (it % C::NS) * C::TILE_BYTES;
    const char *phb = lds + C::PHI_OFF + (it & 1) * kPhiTileBytes;
    bf16x8_t bphi[kKSteps];
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
      bphi[st] = *reinterpret_cast<const bf16x8_t *>(phb + (st * 64 + lane) * 16);

    f32x16_t umu = {};
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
      umu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Amu[st], bphi[st], umu, 0, 0, 0);

    const bool valid = (t0 + rot(it) * kTile + tj) < t1;
    const char *rec = sb + tj * C::CPT * 16;
#pragma unroll
    for (int pp = 0; pp < C::PAIRS; ++pp) {
      f32x16_t u[C::KT];
#pragma unroll
      for (int ti = 0; ti < C::KT; ++ti) {
        u[ti] = f32x16_t{};
#pragma unroll
        for (int st = 0; st < kKSteps; ++st)
          u[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak[pp][ti][st], bphi[st], u[ti], 0, 0, 0);
      }
      const int hl = wave * HPW + 2 * pp + (lane >> 5);
      const int q0 = hl * C::CPH;
      u32x4_t ck[C::CK_CHUNKS];
#pragma unroll
      for (int c = 0; c < C::CK_CHUNKS; ++c)
        ck[c] = *reinterpret_cast<const u32x4_t *>(rec + ((q0 + c) ^ swz) * 16);
      float sc = umu[4 * pp];
#pragma unroll
      for (int ti = 0; ti < C::KT; ++ti) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          // k = ti*16 + 4*gg + e, e = 0..3: chunk k/8, dwords (k%8)/2
          const u32x4_t cc = ck[(ti * 16 + 4 * gg) / 8];
          const int dw = ((4 * gg) % 8) / 2;
          sc = fmaf(u[ti][4 * gg + 0], bf16_lo(cc[dw]), sc);
          sc = fmaf(u[ti][4 * gg + 1], bf16_hi(cc[dw]), sc);
          sc = fmaf(u[ti][4 * gg + 2], bf16_lo(cc[dw + 1]), sc);
          sc = fmaf(u[ti][4 * gg + 3], bf16_hi(cc[dw + 1]), sc);
        }
      }
      if (valid) {
        if (sc > m[pp] + kRescaleGap) {
          const float f = exp2f(m[pp] - sc);
          l[pp] *= f;
#pragma unroll
          for (int r = 0; r < RV; ++r) acc[pp][r] *= f;
          m[pp] = sc;
        }
        const float pe = exp2f(sc - m[pp]);
        l[pp] += pe;
#pragma unroll
        for (int c = 0; c < C::CV_CHUNKS; ++c) {
          const u32x4_t cv =
              *reinterpret_cast<const u32x4_t *>(rec + ((q0 + C::CK_CHUNKS + c) ^ swz) * 16);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[pp][8 * c + 2 * w] = fmaf(pe, bf16_lo(cv[w]), acc[pp][8 * c + 2 * w]);
            acc[pp][8 * c + 2 * w + 1] = fmaf(pe, bf16_hi(cv[w]), acc[pp][8 * c + 2 * w + 1]);
          }
        }
      }
    }
  }

  // ---- combine the 32 lane states of every head and write the partial ----
  // The head's maximum M over its 32 lanes (xor butterfly inside the half
  // wave); every lane rescales its (l, acc) to M, and the 32 lanes are summed
  // through LDS by one thread per partial value.
  u32x4_t wpre[C::WV_AHEAD ? C::OUT_PER_THREAD : 1][RV / 8];
  float mupre[C::WV_AHEAD ? C::OUT_PER_THREAD : 1];
  if constexpr (C::WV_AHEAD) {
    if (p.write_out) {  // W_up,v,t rows and mu_v,t of this thread's outputs, ahead of use
#pragma unroll
      for (int n = 0; n < C::OUT_PER_THREAD; ++n) {
        const int o = n * C::NT + tid, hl = o / kD, i = o % kD;
        const u32x4_t *wrow = reinterpret_cast<const u32x4_t *>(
            reinterpret_cast<const uint16_t *>(p.wv) + ((int64_t)(h0 + hl) * kD + i) * RV);
#pragma unroll
        for (int r8 = 0; r8 < RV / 8; ++r8) wpre[n][r8] = wrow[r8];
        mupre[n] = p.muv[(int64_t)(h0 + hl) * kD + i];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __syncthreads();  // every wave is done reading the last tile's buffers
  float *red = reinterpret_cast<float *>(lds);  // [HG][RV + 1][32]: rescaled l, acc
  float *hmax = red + C::RED_FLOATS;            // [HG]
  float *comb = hmax + C::HG;                   // [HG][RV + 2], one context split
#pragma unroll
  for (int pp = 0; pp < C::PAIRS; ++pp) {
    float M = m[pp];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float f = m[pp] == -INFINITY ? 0.f : exp2f(m[pp] - M);
    const int hl = wave * HPW + 2 * pp + (lane >> 5);
    float *dst = red + hl * (RV + 1) * 32 + (lane & 31);
    dst[0] = l[pp] * f;
#pragma unroll
    for (int r = 0; r < RV; ++r) dst[(r + 1) * 32] = acc[pp][r] * f;
    if ((lane & 31) == 0) hmax[hl] = M;
  }
  __syncthreads();
  for (int o = tid; o < C::HG * (RV + 2); o += C::NT) {
    const int hl = o / (RV + 2), r = o % (RV + 2);
    float v;
    if (r == 0) {
      v = hmax[hl];
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(red + (hl * (RV + 1) + r - 1) * 32);
      float4 t = src[0];
#pragma unroll
      for (int c = 1; c < 8; ++c) {
        const float4 u = src[c];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
      }
      v = (t.x + t.y) + (t.z + t.w);
    }
    if (p.write_out)
      comb[o] = v;
    else
      p.ws[((int64_t)(vb * p.H + h0 + hl) * p.S + s) * (RV + 2) + r] = v;
  }
  if (p.write_out) {
    // A single split holds the whole softmax: apply W_up,v,t and mu_v,t here
    // (no merge launch).  out = W_up,v,t (acc / l) + mu_v,t, one thread per
    // output element, the bf16 row of W_up,v,t read as 16-byte vectors.
    __syncthreads();
#pragma unroll
    for (int n = 0; n < C::OUT_PER_THREAD; ++n) {
      const int o = n * C::NT + tid, hl = o / kD, i = o % kD;
      const float *c = comb + hl * (RV + 2);
      const u32x4_t *wrow = reinterpret_cast<const u32x4_t *>(
          reinterpret_cast<const uint16_t *>(p.wv) + ((int64_t)(h0 + hl) * kD + i) * RV);
      float a = 0.f;
#pragma unroll
      for (int r8 = 0; r8 < RV / 8; ++r8) {
        const u32x4_t wv = C::WV_AHEAD ? wpre[C::WV_AHEAD ? n : 0][r8] : wrow[r8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaf(bf16_lo(wv[e]), c[2 + 8 * r8 + 2 * e], a);
          a = fmaf(bf16_hi(wv[e]), c[3 + 8 * r8 + 2 * e], a);
        }
      }
      const float mu = C::WV_AHEAD ? mupre[C::WV_AHEAD ? n : 0] : p.muv[(int64_t)(h0 + hl) * kD + i];
      const int64_t oi = ((int64_t)vb * p.H + h0 + hl) * kD + i;
      p.out[oi] = fmaf(a, 1.0f / c[1], mu);
    }
  }
#endif
}

template <int RK, int RV, int HPW, int NW>
hipError_t launch(const DecodeParams &p, hipStream_t st) {
  using C = Cfg<RK, RV, HPW, NW>;
  const int groups = p.H / C::HG;
  const dim3 grid(p.B * groups * p.S);
  const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&decode_mfma_split<RK, RV, HPW, NW>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mfma_split<RK, RV, HPW, NW>), grid, dim3(C::NT), C::LDS_BYTES, st, p);
  return hipGetLastError();
}

}  // namespace detail

using namespace detail;

// Shapes served by the fast path and the template instance for each.
bool decode_mfma_supported(int32_t H, int32_t d, int32_t rk, int32_t rv, int32_t Hs) {
  if (d != kD || Hs != H) return false;
  const int32_t hg = decode_mfma_group_heads(rk, rv);
  return hg > 0 && H % hg == 0;
}

int32_t decode_mfma_group_heads(int32_t rk, int32_t rv) {
  if (rk == 16 && rv == 32) return Cfg<16, 32, 2, 8>::HG;
  if (rk == 32 && rv == 64) return Cfg<32, 64, 2, 4>::HG;
  if (rk == 48 && rv == 80) return Cfg<48, 80, 2, 4>::HG;
  return 0;
}

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t st) {
  if (p.rk == 16 && p.rv == 32) return launch<16, 32, 2, 8>(p, st);
  if (p.rk == 32 && p.rv == 64) return launch<32, 64, 2, 4>(p, st);
  if (p.rk == 48 && p.rv == 80) return launch<48, 80, 2, 4>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace lla
