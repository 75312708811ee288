// Append-time encoder for many new rows ("Looped Latent Attention:
// Cross-Loop KV Compression for Looped Transformers", Sec. 3 Eq. 2):
// c = (x - mu) W_down for every new token, stored head and axis, bf16 stores.
//
// The arithmetic is that of the register-streamed encoder: c = x W_down -
// mu W_down on v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums), mu
// split exactly into three bf16 parts (hi + mid + lo) that occupy three rows
// of one extra MFMA row tile, the latent rounded once to bf16 (nearest, ties
// to even).
//
// Data movement.  A workgroup of four waves owns 128 rows (two 16-row tiles
// per wave) of one (stored head, axis) and every column of that axis's
// latent.  The stacked length K is walked in chunks of 64; the 128 x rows and
// the 64 W_down rows of a chunk are copied from HBM into one stage of a
// four-deep LDS ring by LDS-direct buffer loads (no registers, no vector
// instructions), so three chunks are in flight while one is multiplied (a
// fifth stage measured 5% slower, a third 0-15% slower).
// W_down stays in its own [k][column] layout and the k-contiguous B
// fragments are read with the transposing LDS read.  The hi / mid / lo parts
// of mu are formed once per workgroup into LDS.  Workgroups are numbered so
// that the row blocks of one W_down slice run on the same XCD (consecutive
// workgroups go to consecutive XCDs): the slice is read from HBM once and
// then served by that XCD's L2.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace encst {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
#define ENC_LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;                // rows per workgroup
constexpr int kKc = 64;                           // contraction chunk
constexpr int kXPieces = kRows * kKc * 2 / 16;    // 16-byte pieces of x per chunk
constexpr int kXL = kXPieces / kThreads;          // LDS-direct loads of x per lane and chunk
constexpr int kMaxK = 2048;
constexpr int kMuPitch = kMaxK * 2 + 64;          // bytes between the mu part rows
constexpr int kLdsMax = 160 * 1024;
// x is read once: streamed (the same cache-policy bits as the decode
// kernels' latent stream); W_down is re-read by the other row blocks.
constexpr int kPolicyStream = 2;

template <int NT>
struct Cfg {
  static constexpr int WCH = 2 * NT;                  // 16-byte chunks of one W_down row (16 NT columns)
  static constexpr int PITCH = (WCH + 3) / 4 * 4;     // chunks per row in LDS (pad chunks hold copies)
  static constexpr int WL = kKc * PITCH / kThreads;   // LDS-direct loads of W_down per lane and chunk
  static constexpr int LS = kXL + WL;                 // loads per lane and chunk
  static constexpr int W_OFF = kXPieces * 16;
  static constexpr int STAGE = W_OFF + kKc * PITCH * 16;
  static constexpr int NS_FIT = (kLdsMax - 3 * kMuPitch) / STAGE;
  static constexpr int NS = NS_FIT > 4 ? 4 : NS_FIT;  // ring depth
  static constexpr int MU_OFF = NS * STAGE;
  static constexpr int LDS = MU_OFF + 3 * kMuPitch;
  static_assert(NT >= 1 && NT <= 5, "ten transposing reads per k-step at most");
  static_assert((kKc * PITCH) % kThreads == 0, "whole loads of W_down");
  static_assert(NS >= 3, "ring depth");
  static_assert((NS - 2) * LS <= 63, "vmcnt range");
  static_assert(LDS <= kLdsMax, "LDS budget");
};

// Rotation (in chunks) of W_down row kr inside its PITCH-chunk LDS row, so
// that the transposing reads of a half-wave (four rows of each of two
// 8-row groups, 32 bytes per row) hit distinct banks.
template <int PITCH>
__device__ __forceinline__ int w_rot(int kr) {
  if constexpr (PITCH % 8 == 4)
    return 2 * (kr >> 3);
  else if constexpr (PITCH % 16 == 8)
    return (kr & 3) + 4 * (kr >> 3);
  else
    return 2 * (kr & 3) + 8 * (kr >> 3);
}

// Waits until at most N of this wave's vector-memory operations are
// outstanding and its LDS accesses are complete, then joins the workgroup
// barrier; the signal fences keep the compiler from moving LDS accesses
// across it.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Part `which` (0 = hi, 1 = mid, 2 = lo) of the exact three-way bf16 split
// of a float32 value.
__device__ __forceinline__ uint32_t split3(float v, int which) {
  const uint16_t h = f32_to_bf16_bits(v);
  if (which == 0) return h;
  const float r1 = v - bf16_bits_to_f32(h);  // exact
  const uint16_t m = f32_to_bf16_bits(r1);
  if (which == 1) return m;
  return f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));  // exact remainder
}

template <int NT>
__device__ __forceinline__ void body(const EncodeParams &p, int axis, int hs, int rb, char *lds) {
  using C = Cfg<NT>;
  constexpr int R = 16 * NT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, rr = lane & 15;
  const int M = p.B * p.n_new, K = p.K, nc = K / kKc;
  const int row0 = rb * kRows;

  // ---- mu: lane t splits mu[8t .. 8t+7] ----
  const float *mu = p.mu[axis] + (int64_t)hs * K;
  const int m8 = min(tid, K / 8 - 1);
  const float4 m0 = reinterpret_cast<const float4 *>(mu)[2 * m8];
  const float4 m1 = reinterpret_cast<const float4 *>(mu)[2 * m8 + 1];

  // ---- the ring: per-lane source offsets of the LDS-direct loads ----
  // x piece P = n * 256 + tid: row P / 8 of the block, LDS position P % 8;
  // chunk c of a row sits at position (c + row / 2) % 8, so the 16 rows of
  // an A-fragment read start in 16 distinct 16-byte bank groups.
  const int64_t xrow_el = (int64_t)p.Hs * K;  // elements between consecutive rows
  const uint16_t *xbase =
      reinterpret_cast<const uint16_t *>(p.x[axis]) + (int64_t)row0 * xrow_el + (int64_t)hs * K;
  const int rows_here = min(kRows, M - row0);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(xbase), (short)0, (int)(((int64_t)(rows_here - 1) * xrow_el + K) * 2),
      0x00020000);
  uint32_t xo[kXL];
#pragma unroll
  for (int n = 0; n < kXL; ++n) {
    const int P = n * kThreads + tid;
    const int row = P >> 3, pos = P & 7;
    const int c = (pos - (row >> 1)) & 7;
    const int rowc = min(row, rows_here - 1);  // rows past M: a valid row, never stored
    xo[n] = (uint32_t)(((int64_t)rowc * xrow_el + c * 8) * 2);
  }
  // W_down piece P = n * 256 + tid: row kr = P / PITCH of the chunk, LDS
  // position P % PITCH; chunk cw of a row sits at (cw + w_rot(kr)) % PITCH,
  // and the pad positions (cw >= WCH) load a copy of chunk cw - WCH.
  const uint16_t *wbase = reinterpret_cast<const uint16_t *>(p.wd[axis]) + (int64_t)hs * K * R;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(wbase), (short)0, K * R * 2, 0x00020000);
  uint32_t wo[C::WL];
#pragma unroll
  for (int n = 0; n < C::WL; ++n) {
    const int P = n * kThreads + tid;
    const int kr = P / C::PITCH, pos = P % C::PITCH;
    int cw = (pos - w_rot<C::PITCH>(kr) % C::PITCH + C::PITCH) % C::PITCH;
    if (cw >= C::WCH) cw -= C::WCH;
    wo[n] = (uint32_t)((kr * R + cw * 8) * 2);
  }
  auto issue = [&](int it) {
    char *sb = lds + (it % C::NS) * C::STAGE;
    const uint32_t xk = (uint32_t)it * kKc * 2;
    const uint32_t wk = (uint32_t)it * kKc * R * 2;
#pragma unroll
    for (int n = 0; n < kXL; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (ENC_LDS_AS void *)(sb + (n * kThreads + wave * 64) * 16), 16, xo[n] + xk, 0, 0,
          kPolicyStream);
#pragma unroll
    for (int n = 0; n < C::WL; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (ENC_LDS_AS void *)(sb + C::W_OFF + (n * kThreads + wave * 64) * 16), 16, wo[n] + wk,
          0, 0, 0);
  };
#pragma unroll
  for (int k = 0; k + 1 < C::NS; ++k)
    if (k < nc) issue(k);

  // The compiler issues the mu loads after the ring's first chunks and waits
  // for all of them here; copying mu by LDS-direct loads too, so that only
  // the first chunk is waited for, measured no faster.
  char *mus = lds + C::MU_OFF;
  if (tid < K / 8) {
    const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      u32x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = split3(mv[2 * e], part) | (split3(mv[2 * e + 1], part) << 16);
      *reinterpret_cast<u32x4_t *>(mus + part * kMuPitch + tid * 16) = pk;
    }
  }

  // ---- per-lane LDS offsets of the fragments ----
  // A (x): row 32 wave + 16 mt + rr, k = 32 ks + 8 g + 0..7 (chunk 4 ks + g)
  uint32_t ao[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = 32 * wave + 16 * mt + rr;
      ao[mt][ks] = (uint32_t)((row * 8 + ((4 * ks + g + (row >> 1)) & 7)) * 16);
    }
  // B (W_down), transposing reads: for k-step ks and tile nt, lane rr of
  // group g addresses the 8-byte piece of row 32 ks + 8 g + rr / 4 (and four
  // rows further for the upper half of the fragment), columns 16 nt +
  // 4 (rr % 4) + 0..3, so that lane i of the group receives column 16 nt + i
  // of those four rows.  The rotation of a row depends on kr % 4 and kr / 8
  // only, so the upper half is 4 PITCH chunks further.
  uint32_t bo[2][NT];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int kr = 32 * ks + 8 * g + (rr >> 2);
      const int cw = 2 * nt + ((rr & 3) >> 1);
      bo[ks][nt] = (uint32_t)(C::W_OFF + (kr * C::PITCH + (cw + w_rot<C::PITCH>(kr)) % C::PITCH) * 16 +
                              8 * (rr & 1));
    }
  // mu A fragment: rows 0..2 of the tile are the hi / mid / lo parts
  const uint32_t muo = (uint32_t)(min(rr, 2) * kMuPitch + g * 16);
  const uint32_t mukeep = rr < 3 ? ~0u : 0u;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(ENC_LDS_AS char *)lds;

  f32x4_t acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int NB = (NT + 3) / 4;  // mu W_down: wave w owns the tiles nt with nt % 4 == w
  f32x4_t accb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) accb[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < nc; ++it) {
    // chunk it has landed (every wave's loads) and every wave is done with
    // chunk it - 1, whose stage the next issue overwrites
    const int ahead = min(nc - 1 - it, C::NS - 2);  // chunks issued after this one
    if (ahead == C::NS - 2)
      ring_barrier<(C::NS - 2) * C::LS>();
    else if (ahead == 2)
      ring_barrier<2 * C::LS>();
    else if (ahead == 1)
      ring_barrier<C::LS>();
    else
      ring_barrier<0>();
    if (it + C::NS - 1 < nc) issue(it + C::NS - 1);

    const uint32_t stage = (uint32_t)((it % C::NS) * C::STAGE);
    const char *sb = lds + stage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) a[mt] = *reinterpret_cast<const bf16x8_t *>(sb + ao[mt][ks]);
      u32x4_t mw = *reinterpret_cast<const u32x4_t *>(mus + muo + (it * kKc + 32 * ks) * 2);
      mw[0] &= mukeep;
      mw[1] &= mukeep;
      mw[2] &= mukeep;
      mw[3] &= mukeep;
      const bf16x8_t amu = __builtin_bit_cast(bf16x8_t, mw);
      uint32_t ta[2 * NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ta[2 * nt] = lds_base + stage + bo[ks][nt];
        ta[2 * nt + 1] = ta[2 * nt] + 4 * C::PITCH * 16;
      }
      tr_short4_t tv[2 * NT];
      lds_read_tr16_b64<2 * NT>(ta, tv);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const tr_short4_t lo = tv[2 * nt], hi = tv[2 * nt + 1];
        const bf16x8_t bw = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], bw, acc[mt][nt], 0, 0, 0);
        if (nt % 4 == wave)
          accb[nt / 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(amu, bw, accb[nt / 4], 0, 0, 0);
      }
    }
  }

  // ---- mu W_down: rows 0..2 of the mu tile live in lanes 0..15 ----
  __syncthreads();  // every wave is done with the ring
  float *bias = reinterpret_cast<float *>(lds);  // [R]
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int nt = 4 * i + wave;
    if (nt < NT && g == 0) bias[nt * 16 + rr] = (accb[i][2] + accb[i][1]) + accb[i][0];
  }
  __syncthreads();

  // ---- c = x W - mu W, rounded to bf16, written at the token's slot ----
  uint16_t *st = reinterpret_cast<uint16_t *>(p.store);
  const int koff = axis ? p.rk : 0;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 32 * wave + 16 * mt + 4 * g + i;
      if (row >= M) continue;
      const int b = row / p.n_new, jn = row % p.n_new;
      const int64_t slot = (int64_t)p.start[b] + jn;  // start is caller data
      if (slot < 0 || slot >= p.N) continue;
      uint16_t *dst = st + ((((int64_t)b * p.D + p.layer) * p.N + slot) * p.Hs + hs) * p.R + koff;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        dst[nt * 16 + rr] = f32_to_bf16_bits(acc[mt][nt][i] - bias[nt * 16 + rr]);
    }
  }
}

// Workgroup L runs item I = (pair, row block), pair = 2 * head + axis.  When
// the item count is a multiple of eight, XCD x = L % 8 runs the consecutive
// items x * items / 8 ...: whole groups of row blocks of one pair.
template <int NTK, int NTV>
__global__ __launch_bounds__(kThreads, 1) void encode_stream(EncodeParams p, int nrb) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only builtins
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int L = blockIdx.x, items = gridDim.x;
  const int I = (items % 8 == 0) ? (L % 8) * (items / 8) + L / 8 : L;
  const int pair = I / nrb, rb = I % nrb;
  const int hs = pair >> 1;
  if ((pair & 1) == 0)
    body<NTK>(p, 0, hs, rb, lds);
  else
    body<NTV>(p, 1, hs, rb, lds);
#endif
}

template <int NTK, int NTV>
hipError_t launch(const EncodeParams &p, hipStream_t st) {
  const int M = p.B * p.n_new;
  const int nrb = (M + kRows - 1) / kRows;
  const size_t lds = Cfg<NTK>::LDS > Cfg<NTV>::LDS ? Cfg<NTK>::LDS : Cfg<NTV>::LDS;
  const void *fn = reinterpret_cast<const void *>(&encode_stream<NTK, NTV>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((encode_stream<NTK, NTV>), dim3(nrb * 2 * p.Hs), dim3(kThreads), lds, st, p, nrb);
  return hipGetLastError();
}

}  // namespace encst

// The streamed form needs K a multiple of 64 and at most 2048 (the mu parts
// of the whole length sit in LDS), 32-bit byte offsets inside one
// workgroup's 128 rows of x and inside one head's W_down, one of the rank
// pairs it is instantiated for, and enough workgroups to fill the chip.
bool encode_stream_supported(const EncodeParams &p) {
  const int M = p.B * p.n_new;
  const int64_t xspan = ((int64_t)(encst::kRows - 1) * p.Hs * p.K + p.K) * 2;
  const bool ranks = (p.rk == 16 && p.rv == 32) || (p.rk == 32 && p.rv == 64) ||
                     (p.rk == 48 && p.rv == 80);
  const int64_t items = (int64_t)((M + encst::kRows - 1) / encst::kRows) * 2 * p.Hs;
  return ranks && p.K % encst::kKc == 0 && p.K <= encst::kMaxK && xspan < ((int64_t)1 << 31) &&
         (int64_t)p.K * p.rv * 2 < ((int64_t)1 << 31) && items >= 128;
}

hipError_t launch_encode_stream(const EncodeParams &p, hipStream_t st) {
  if (p.rk == 16) return encst::launch<1, 2>(p, st);
  if (p.rk == 32) return encst::launch<2, 4>(p, st);
  return encst::launch<3, 5>(p, st);
}

}  // namespace lla
