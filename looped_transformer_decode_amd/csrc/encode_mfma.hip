// Append-time encoder on the matrix cores, for bf16 stores ("Looped Latent
// Attention: Cross-Loop KV Compression for Looped Transformers", Sec. 3
// Eq. 2):  c = (x - mu) W_down  for every new token, stored head and axis.
//
// The product is split as c = x W_down - mu W_down.  x and W_down are bf16,
// so x W_down runs on v_mfma_f32_16x16x32_bf16 with exact products and fp32
// sums.  mu is float32 and not representable in bf16; it is split exactly
// into three bf16 parts (mu = hi + mid + lo, 8 + 8 + 8 significand bits),
// which occupy three rows of one extra MFMA row tile, so mu W_down is also
// formed from exact products.  The latent is rounded once to bf16 (nearest,
// ties to even).
//
// Work split.  A workgroup of four waves owns (row block, stored head, axis,
// column group); each wave owns MT tiles of 16 rows (rows = (sequence, new
// token)).  With few row blocks (LLA-2D, small batches) the variant at the
// end of this file splits the contraction over the waves instead; with many
// rows the form in encode_stream.hip (x and W_down through an LDS ring)
// takes over.  The
// stacked length K is walked in chunks of 128.  Rows of x stream from HBM
// straight into registers: within a chunk, lane group g = lane/16 reads 64
// contiguous bytes of its row, and the contraction index is permuted
// accordingly (step s, group g, element e <-> k = 32 g + 8 s + e), so every
// row is read in whole 256-byte segments.  The W_down chunk of the head is
// shared by the four waves: it is loaded once per workgroup and written to
// LDS transposed ([column][k], padded rows) so that each lane's B fragment
// is one 16-byte read; the three bf16 parts of the mu chunk go to LDS with
// it.  While chunk c is multiplied, x of chunk c+2 and W_down of chunk c+1
// are in flight.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace detail {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int kKc = 128;           // contraction chunk
constexpr int kPitch = kKc + 8;    // LDS row pitch of the transposed W_down chunk (elements)
constexpr int kThreads = 256;
constexpr int kMaxNT = 8;          // r <= 128

__host__ __device__ constexpr size_t encode_lds_bytes(int r) {
  return 2 * (size_t)r * kPitch * 2   // W_down chunk, two buffers
         + 2 * 3 * kKc * 2            // hi / mid / lo parts of the mu chunk, two buffers
         + (size_t)r * 4;             // mu W_down
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Part `which` (0 = hi, 1 = mid, 2 = lo) of the exact three-way bf16 split
// of a float32 value.
__device__ __forceinline__ uint16_t split3(float v, int which) {
  const uint16_t h = f32_to_bf16_bits(v);
  if (which == 0) return h;
  const float r1 = v - bf16_bits_to_f32(h);  // exact
  const uint16_t m = f32_to_bf16_bits(r1);
  if (which == 1) return m;
  return f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));  // exact remainder
}

template <int MT, int NT>
// Columns [col0, col0 + 16 NT) of the latents of one axis (rfull wide).
__device__ __forceinline__ void encode_body(const EncodeParams &p, int axis, int col0, char *lds) {
  constexpr int R = NT * 16;
  constexpr int PAIRS = kKc / 2 * (R / 8);        // (k pair, 8-column group) units per chunk
  constexpr int PPT = (PAIRS + kThreads - 1) / kThreads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, rr = lane & 15;
  const int hs = blockIdx.y;
  const int M = p.B * p.n_new;
  const int K = p.K;
  const int nc = K / kKc;
  const int row0 = (blockIdx.x * 4 + wave) * (16 * MT);

  uint16_t *wt = reinterpret_cast<uint16_t *>(lds);                       // [2][R][kPitch]
  uint16_t *mus = wt + 2 * R * kPitch;                                     // [2][3][kKc]
  float *bias = reinterpret_cast<float *>(mus + 2 * 3 * kKc);              // [R]

  const int rfull = axis ? p.rv : p.rk;
  const uint16_t *wd =
      reinterpret_cast<const uint16_t *>(p.wd[axis]) + (int64_t)hs * K * rfull + col0;
  const float *mu = p.mu[axis] + (int64_t)hs * K;
  const u32x4_t *xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = min(row0 + mt * 16 + rr, M - 1);  // rows past M: read a valid row, never stored
    xrow[mt] = reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint16_t *>(p.x[axis]) +
                                                 ((int64_t)row * p.Hs + hs) * K) + 4 * g;
  }

  // ---- staging of one W_down / mu chunk: global -> registers -> LDS ----
  u32x4_t wreg[PPT][2];
  float4 mureg;
  auto fetch_w = [&](int c) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < PAIRS) {
        const int kp = v / (R / 8), n0 = (v % (R / 8)) * 8;
        const u32x4_t *src =
            reinterpret_cast<const u32x4_t *>(wd + (int64_t)(c * kKc + 2 * kp) * rfull + n0);
        wreg[i][0] = src[0];
        wreg[i][1] = src[rfull / 8];
      }
    }
    if (tid < kKc / 4) mureg = reinterpret_cast<const float4 *>(mu + c * kKc)[tid];
  };
  auto store_w = [&](int buf) {
    uint16_t *w = wt + buf * R * kPitch;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int v = tid + i * kThreads;
      if (v < PAIRS) {
        const int kp = v / (R / 8), n0 = (v % (R / 8)) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (wreg[i][0][e / 2] >> ((e & 1) * 16)) & 0xFFFFu;
          const uint32_t hi = (wreg[i][1][e / 2] >> ((e & 1) * 16)) & 0xFFFFu;
          *reinterpret_cast<uint32_t *>(w + (n0 + e) * kPitch + 2 * kp) = lo | (hi << 16);
        }
      }
    }
    if (tid < kKc / 4) {
      const float mv[4] = {mureg.x, mureg.y, mureg.z, mureg.w};
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        uint2 pk;
        pk.x = split3(mv[0], part) | ((uint32_t)split3(mv[1], part) << 16);
        pk.y = split3(mv[2], part) | ((uint32_t)split3(mv[3], part) << 16);
        *reinterpret_cast<uint2 *>(mus + (buf * 3 + part) * kKc + 4 * tid) = pk;
      }
    }
  };

  // ---- accumulators ----
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // mu W_down: wave w owns the column tiles nt with nt % 4 == w
  constexpr int NB = (NT + 3) / 4;
  f32x4_t accb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) accb[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t xa[3][MT][4];
  auto fetch_x = [&](int c, u32x4_t (&dst)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[mt][s] = __builtin_nontemporal_load(xrow[mt] + c * 16 + s);
  };

  auto compute = [&](int buf, const u32x4_t (&xc)[MT][4]) {
    const uint16_t *w = wt + buf * R * kPitch;
    // rows 0..2 of the mu tile: hi / mid / lo parts of mu; other rows zero
    const uint16_t *mrow = mus + (buf * 3 + (rr < 3 ? rr : 0)) * kKc;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t mz = {0u, 0u, 0u, 0u};
      const bf16x8_t amu =
          as_bf16x8(rr < 3 ? *reinterpret_cast<const u32x4_t *>(mrow + 32 * g + 8 * s) : mz);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t bw =
            *reinterpret_cast<const bf16x8_t *>(w + (nt * 16 + rr) * kPitch + 32 * g + 8 * s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xc[mt][s]), bw,
                                                                 acc[mt][nt], 0, 0, 0);
        if (nt % 4 == wave)
          accb[nt / 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(amu, bw, accb[nt / 4], 0, 0, 0);
      }
    }
  };

  // ---- pipeline over chunks ----
  // x is fetched two chunks ahead (three register buffers, so the loop is
  // unrolled by three), W_down / mu one chunk ahead through registers into
  // the other LDS buffer.  Loads complete in issue order: storing W_down
  // chunk c+1 waits only for loads issued before it, never for x of c+2.
  auto step = [&](int c, const u32x4_t (&cur)[MT][4], u32x4_t (&ahead)[MT][4]) {
    if (c + 2 < nc) fetch_x(c + 2, ahead);
    compute(c & 1, cur);
    if (c + 1 < nc) store_w((c + 1) & 1);
    if (c + 2 < nc) fetch_w(c + 2);
    __syncthreads();
  };
  fetch_w(0);
  fetch_x(0, xa[0]);
  if (nc > 1) fetch_x(1, xa[1]);
  store_w(0);
  if (nc > 1) fetch_w(1);
  __syncthreads();
  for (int c = 0; c < nc; c += 3) {
    step(c, xa[0], xa[2]);
    if (c + 1 >= nc) break;
    step(c + 1, xa[1], xa[0]);
    if (c + 2 >= nc) break;
    step(c + 2, xa[2], xa[1]);
  }

  // ---- mu W_down: rows 0..2 of the mu tile live in lanes 0..15 ----
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int nt = 4 * i + wave;
    if (nt < NT && g == 0) bias[nt * 16 + rr] = (accb[i][2] + accb[i][1]) + accb[i][0];
  }
  __syncthreads();

  // ---- c = x W - mu W, rounded to bf16, written at the token's slot ----
  uint16_t *st = reinterpret_cast<uint16_t *>(p.store);
  const int koff = (axis ? p.rk : 0) + col0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + mt * 16 + 4 * g + i;
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

// NTK / NTV: column tiles per workgroup of the K and V latents.
// blockIdx.z enumerates the column groups: gk groups of the K latent, then
// those of the V latent.
template <int MT, int NTK, int NTV>
__global__ __launch_bounds__(kThreads, 2) void encode_mfma(EncodeParams p, int gk) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int z = blockIdx.z;
  if (z < gk)
    encode_body<MT, NTK>(p, 0, z * 16 * NTK, lds);
  else
    encode_body<MT, NTV>(p, 1, (z - gk) * 16 * NTV, lds);
#endif
}

template <int MT, int NTK, int NTV>
hipError_t launch(const EncodeParams &p, hipStream_t st) {
  const int M = p.B * p.n_new;
  const int gk = p.rk / (16 * NTK);
  const int gv = p.rv / (16 * NTV);
  const size_t lds = encode_lds_bytes(16 * (NTK > NTV ? NTK : NTV));
  const void *fn = reinterpret_cast<const void *>(&encode_mfma<MT, NTK, NTV>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int rows = 4 * 16 * MT;
  const dim3 grid((M + rows - 1) / rows, p.Hs, gk + gv);
  hipLaunchKernelGGL((encode_mfma<MT, NTK, NTV>), grid, dim3(kThreads), lds, st, p, gk);
  return hipGetLastError();
}

// ---- few row blocks: the contraction split over the waves ----
// With few row blocks (LLA-2D, small batches) a workgroup of the kernel
// above walks all K / 128 chunks one after another, and that chain of load
// round trips sets its time.  Here a workgroup owns one tile of 16 rows and
// one 16-column tile; wave w of kSkWaves takes chunks w, w + kSkWaves, ...,
// stages each W_down chunk (transposed) and its mu parts in LDS of its own,
// keeps its own partial products, and the partials are summed through LDS at
// the end.  Each wave's chain is kSkWaves times shorter.  (Eight waves
// measured 7% faster than four at the LLA-2D shape; what remains is the
// re-reading of x by every column tile and of W_down by every row tile.)
constexpr int kSkWaves = 8;
constexpr int kSkStages = 3;  // chunks of x / W_down / mu a wave has in flight

__host__ __device__ constexpr size_t encode_sk_wave_lds() {
  return 2 * 16 * kPitch * 2    // W_down chunk, transposed, two buffers
         + 2 * 3 * kKc * 2;     // hi / mid / lo parts of the mu chunk, two buffers
}

__global__ __launch_bounds__(64 * kSkWaves) void encode_mfma_splitk(EncodeParams p, int gk) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, rr = lane & 15;
  const int z = blockIdx.z, axis = z < gk ? 0 : 1;
  const int col0 = (axis ? z - gk : z) * 16;
  const int hs = blockIdx.y;
  const int M = p.B * p.n_new, K = p.K, nc = K / kKc;
  const int rfull = axis ? p.rv : p.rk;
  const int row = min((int)blockIdx.x * 16 + rr, M - 1);  // rows past M: read, never stored
  const u32x4_t *xrow = reinterpret_cast<const u32x4_t *>(
                            reinterpret_cast<const uint16_t *>(p.x[axis]) +
                            ((int64_t)row * p.Hs + hs) * K) + 4 * g;
  const uint16_t *wd =
      reinterpret_cast<const uint16_t *>(p.wd[axis]) + (int64_t)hs * K * rfull + col0;
  const float *mu = p.mu[axis] + (int64_t)hs * K;
  uint16_t *wt = reinterpret_cast<uint16_t *>(lds + wave * encode_sk_wave_lds());  // [2][16][kPitch]
  uint16_t *mus = wt + 2 * 16 * kPitch;                                          // [2][3][kKc]

  // this wave's chunks: c = wave + kSkWaves i, i < nw
  const int nw = nc > wave ? (nc - wave + kSkWaves - 1) / kSkWaves : 0;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
  if (nw > 0) {  // wave-uniform
    // Stage s holds chunk i: the 64 bytes of x this lane multiplies (row rr,
    // k = 32 g + 8 q + e), W_down rows 2 lane and 2 lane + 1 of the 16
    // columns, and mu at k = 2 lane, 2 lane + 1.  Past the wave's last chunk
    // the loads repeat it (no branch around a load).
    u32x4_t xs[kSkStages][4], ws[kSkStages][4];
    float2 ms[kSkStages];
    auto fetch = [&](int i, int st) {
      const int c = wave + kSkWaves * min(i, nw - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[st][q] = xrow[c * 16 + q];
      const u32x4_t *src =
          reinterpret_cast<const u32x4_t *>(wd + (int64_t)(c * kKc + 2 * lane) * rfull);
      ws[st][0] = src[0];
      ws[st][1] = src[1];
      ws[st][2] = src[rfull / 8];
      ws[st][3] = src[rfull / 8 + 1];
      ms[st] = *reinterpret_cast<const float2 *>(mu + c * kKc + 2 * lane);
    };
    auto stage_lds = [&](int buf, int st) {  // W_down transposed ([column][k]) and mu parts
      uint16_t *w = wt + buf * 16 * kPitch;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int sh = (n & 1) * 16;
        const uint32_t lo = (ws[st][n / 8][(n % 8) / 2] >> sh) & 0xFFFFu;
        const uint32_t hi = (ws[st][2 + n / 8][(n % 8) / 2] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint32_t *>(w + n * kPitch + 2 * lane) = lo | (hi << 16);
      }
#pragma unroll
      for (int part = 0; part < 3; ++part)
        *reinterpret_cast<uint32_t *>(mus + (buf * 3 + part) * kKc + 2 * lane) =
            split3(ms[st].x, part) | ((uint32_t)split3(ms[st].y, part) << 16);
    };
    auto compute = [&](int buf, int st) {
      const uint16_t *w = wt + buf * 16 * kPitch;
      const uint16_t *mrow = mus + (buf * 3 + (rr < 3 ? rr : 0)) * kKc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t mz = {0u, 0u, 0u, 0u};
        const bf16x8_t amu =
            as_bf16x8(rr < 3 ? *reinterpret_cast<const u32x4_t *>(mrow + 32 * g + 8 * q) : mz);
        const bf16x8_t bw =
            *reinterpret_cast<const bf16x8_t *>(w + rr * kPitch + 32 * g + 8 * q);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xs[st][q]), bw, acc, 0, 0, 0);
        accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(amu, bw, accb, 0, 0, 0);
      }
    };
    // every LDS region is the wave's own: a wave-level wait orders its
    // writes before its reads, and LDS operations of one wave run in order
    auto step = [&](int i, int st) {
      stage_lds(i & 1, st);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      compute(i & 1, st);
      fetch(i + kSkStages, st);
    };
#pragma unroll
    for (int st = 0; st < kSkStages; ++st) fetch(st, st);
    // whole groups of kSkStages steps without a branch (a branch inside
    // would leave the compiler's count of outstanding loads inexact and make
    // it wait for all of them), then the remainder
    const int full = nw / kSkStages * kSkStages;
    for (int i0 = 0; i0 < full; i0 += kSkStages) {
#pragma unroll
      for (int j = 0; j < kSkStages; ++j) step(i0 + j, j);
    }
#pragma unroll
    for (int j = 0; j + 1 < kSkStages; ++j)
      if (full + j < nw) step(full + j, j);
  }

  // ---- sum the partials; c = x W - mu W, rounded once ----
  __syncthreads();  // every wave is done with its staging buffers
  float *red = reinterpret_cast<float *>(lds);   // [waves][64 lanes][4]
  float *redb = red + kSkWaves * 64 * 4;         // [waves][16 columns]
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
  // mu W_down: rows 0..2 of the mu tile (hi, mid, lo parts) sit in lanes 0..15
  if (g == 0) redb[wave * 16 + rr] = (accb[2] + accb[1]) + accb[0];
  __syncthreads();
  if (wave != 0) return;
  float bias = 0.f;
#pragma unroll
  for (int w = 0; w < kSkWaves; ++w) bias += redb[w * 16 + rr];
  uint16_t *st = reinterpret_cast<uint16_t *>(p.store);
  const int koff = (axis ? p.rk : 0) + col0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) a += red[(w * 64 + lane) * 4 + i];
    const int r = (int)blockIdx.x * 16 + 4 * g + i;
    if (r >= M) continue;
    const int b = r / p.n_new, jn = r % p.n_new;
    const int64_t slot = (int64_t)p.start[b] + jn;  // start is caller data
    if (slot < 0 || slot >= p.N) continue;
    st[((((int64_t)b * p.D + p.layer) * p.N + slot) * p.Hs + hs) * p.R + koff + rr] =
        f32_to_bf16_bits(a - bias);
  }
#endif
}

hipError_t launch_splitk(const EncodeParams &p, hipStream_t st) {
  const int M = p.B * p.n_new;
  const int gk = p.rk / 16, gv = p.rv / 16;
  const size_t lds = kSkWaves * encode_sk_wave_lds();
  static_assert(kSkWaves * encode_sk_wave_lds() >= kSkWaves * 64 * 4 * 4 + kSkWaves * 16 * 4,
                "the partial sums reuse the staging LDS");
  const void *fn = reinterpret_cast<const void *>(&encode_mfma_splitk);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((M + 15) / 16, p.Hs, gk + gv);
  hipLaunchKernelGGL(encode_mfma_splitk, grid, dim3(64 * kSkWaves), lds, st, p, gk);
  return hipGetLastError();
}

}  // namespace detail

using namespace detail;

bool encode_mfma_supported(const EncodeParams &p, int dtype) {
  auto al = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
  return dtype == LLA_DT_BF16 && p.rk % 16 == 0 && p.rv % 16 == 0 && p.rk <= 16 * kMaxNT &&
         p.rv <= 16 * kMaxNT && p.K % kKc == 0 && al(p.x[0]) && al(p.x[1]) && al(p.wd[0]) &&
         al(p.wd[1]) && al(p.mu[0]) && al(p.mu[1]);
}

hipError_t launch_encode_mfma(const EncodeParams &p, hipStream_t st) {
  const int M = p.B * p.n_new;
  const int k = p.rk / 16, v = p.rv / 16;
  const int64_t blocks1 = (int64_t)((M + 63) / 64) * p.Hs;  // workgroups per column group
  // Few row blocks (small batch, LLA-2D): one 16-row, 16-column tile per
  // workgroup, the contraction split over its waves.
  if (blocks1 * 2 < 128) return launch_splitk(p, st);
  // Many rows: the streamed form (x and W_down through an LDS ring).
  if (encode_stream_supported(p)) return launch_encode_stream(p, st);
  // Two row tiles per wave when that still gives a full wave of workgroups
  // (only the smallest ranks: larger ones would spill at two waves per SIMD).
  const bool two = (int64_t)((M + 127) / 128) * p.Hs * 2 >= 256;
  if (two && k == 1 && v == 2) return launch<2, 1, 2>(p, st);
  if (k == 1 && v == 2) return launch<1, 1, 2>(p, st);
  if (k == 2 && v == 4) return launch<1, 2, 4>(p, st);
  if (k == 3 && v == 5) return launch<1, 3, 5>(p, st);
  return launch<1, 1, 1>(p, st);  // any other ranks: one 16-column tile per workgroup
}

}  // namespace lla
