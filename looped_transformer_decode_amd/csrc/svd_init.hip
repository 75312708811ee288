// SVD codec initialisation ("Looped Latent Attention: Cross-Loop KV
// Compression for Looped Transformers", Sec. 3, initialisation and
// conversion): for every codec g (one per layer, head and axis) and the N
// calibration rows x_n in R^K (K = T * width) of its stacked loop vectors,
//     mu     = (1/N) sum_n x_n                 (the per-loop means, stacked)
//     W_down = the top-r right singular vectors of X - 1 mu^T
//     W_up,t = rows [t*width, (t+1)*width) of W_down (its loop-t slice).
//
// The right singular vectors of the centred matrix are the eigenvectors of
// its Gram matrix C = (X - 1 mu^T)^T (X - 1 mu^T), and the singular values
// the square roots of C's eigenvalues.  They are found by block subspace
// iteration on C with m = r + p >= r vectors (p extra vectors speed up the
// convergence of the r-th one):
//     Q <- orth(C Q)                 (CholeskyQR2, small matrices in fp64)
// and a final Rayleigh-Ritz step: the m x m matrix Q^T C Q is diagonalised
// by cyclic Jacobi rotations in fp64 and the r leading Ritz vectors give
// W_down.  Large products (the Gram matrix, C Q, Q R^-1, Q U) are fp32 tiled
// GEMMs; the small ones (Y^T Y, Q^T C Q) accumulate in fp64.
#include <algorithm>
#include <cmath>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace svd {
inline size_t align256_(size_t v) { return (v + 255) / 256 * 256; }
// The small fp64 Gram products are formed in this many row ranges, whose
// partial m x m matrices their consumers add as they load them.
constexpr int kSmallGramParts = 4;
}  // namespace svd

SvdLayout svd_layout(int32_t G, int32_t K, int32_t m, int32_t r) {
  SvdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = svd::align256_(off + bytes);
    return o;
  };
  L.gram = take((size_t)G * K * K * 4);
  L.q = take((size_t)G * K * m * 4);
  L.y = take((size_t)G * K * m * 4);
  L.small = take((size_t)G * m * m * 8 * svd::kSmallGramParts);
  L.rinv = take((size_t)G * m * m * 4);
  L.u = take((size_t)G * m * m * 8);
  L.evals = take((size_t)G * m * 8);
  L.order = take((size_t)G * m * 4);
  L.usel = take((size_t)G * m * r * 4);
  L.w = take((size_t)G * K * r * 4);
  L.total = off;
  return L;
}

namespace svd {
namespace {

constexpr int kT = 64;        // GEMM output tile
constexpr int kBK = 16;       // GEMM k-chunk
constexpr int kThreads = 256;
constexpr size_t kMaxLds = 160 * 1024;  // dynamic LDS one gfx950 workgroup may use

// Operands of the tiled GEMM, element (g, row, col).
struct MatF32 {
  const float *p;
  int64_t sg, s0, s1;
  int n0, n1;
  __device__ float operator()(int g, int a, int b) const {
    return (a < n0 && b < n1) ? p[g * sg + (int64_t)a * s0 + (int64_t)b * s1] : 0.f;
  }
};
// Centred calibration data, x laid out [N][G][K].  Transposed (feature,
// sample) for the Gram matrix's left operand, (sample, feature) for its right.
template <typename E, bool FEATURE_ROWS>
struct Centred {
  const E *x;
  const float *mu;
  int G, N, K;
  __device__ float operator()(int g, int a, int b) const {
    const int f = FEATURE_ROWS ? a : b, n = FEATURE_ROWS ? b : a;
    if (f >= K || n >= N) return 0.f;
    return load_elem(x, ((int64_t)n * G + g) * K + f) - mu[(int64_t)g * K + f];
  }
};

// C[g][i][j] = sum_k A(g, i, k) B(g, k, j), i < M, j < Nn.  64 x 64 output
// tile per block.  The operands are staged in LDS in chunks of 16 k (through
// the loaders, which centre or bound-check element by element); the four
// waves each multiply one 32 x 32 quarter of the tile on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32: exact fp32 products, fp32 sums), with the
// next chunk's elements loaded into registers while the current one is
// multiplied.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
template <class LA, class LB>
__global__ __launch_bounds__(kThreads) void gemm(LA A, LB B, float *C, int64_t c_sg, int ldc, int M,
                                                 int Nn, int Kd) {
  __shared__ __align__(16) float As[2][kBK][kT + 4];
  __shared__ __align__(16) float Bs[2][kBK][kT + 4];
  const int g = blockIdx.z, i0 = blockIdx.y * kT, j0 = blockIdx.x * kT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;  // this wave's 32 x 32 quarter
  constexpr int PER = kBK * kT / kThreads;   // elements per thread per operand and chunk
  float ra[PER], rb[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + kThreads * q, kk = e / kT, ii = e % kT;
      ra[q] = A(g, i0 + ii, k0 + kk);
      rb[q] = B(g, k0 + kk, j0 + ii);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + kThreads * q, kk = e / kT, ii = e % kT;
      As[buf][kk][ii] = ra[q];
      Bs[buf][kk][ii] = rb[q];
    }
  };
  f32x16_t acc = {};
  fetch(0);
  stage(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < Kd; k0 += kBK) {
    const bool more = k0 + kBK < Kd;
    if (more) fetch(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 2) {
      // A: row wi*32 + lane%32, k = kk + lane/32;  B: column wj*32 + lane%32
      const float a = As[buf][kk + (lane >> 5)][wi * 32 + (lane & 31)];
      const float b = Bs[buf][kk + (lane >> 5)][wj * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // accumulator r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
  const int j = j0 + wj * 32 + (lane & 31);
  if (j < Nn) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (i < M) C[g * c_sg + (int64_t)i * ldc + j] = acc[r];
    }
  }
}

// C[g][i][j] = sum_k X[g][k][i] Y[g][k][j] for a narrow right-hand side
// (Nn <= 32 NB columns), both operands k-major with rows of 16-byte vectors:
// the subspace iteration's C Q (C symmetric, so its rows serve as X's) and
// the Rayleigh-Ritz product.  A block takes 128 rows and every column; wave
// w multiplies rows 32 w .. 32 w + 31 against the NB column tiles, so each
// A fragment read from LDS feeds NB independent v_mfma_f32_32x32x2_f32
// chains.  Chunks of 32 k are staged in LDS as 16-byte vectors, the next
// chunk loaded into registers while the current one is multiplied.
typedef float f32x4_v __attribute__((ext_vector_type(4)));
constexpr int kTnK = 32;
// RW row tiles of 32 per block (4, or 2 for narrow products, which then run
// more blocks per CU); the 4 / RW waves of a row tile share its NB column
// tiles.
template <int NB, int RW>
struct TnCfg {
  static constexpr int ROWS = 32 * RW;                     // rows of the block
  static constexpr int WPR = 4 / RW;                       // waves per row tile
  static constexpr int NBW = NB / WPR;                     // column tiles per wave
  static constexpr int NC = 32 * NB;                       // columns of the block
  // LDS row pitches (floats), 32 banks apart modulo 64: the two k rows one
  // operand read touches (lanes 0-31, 32-63) fall in disjoint banks
  static constexpr int AP = ROWS + (ROWS % 64 == 32 ? 0 : 32), BP = NC + (NC % 64 == 32 ? 0 : 32);
  static constexpr int AV = kTnK * ROWS / 4 / kThreads;    // A vectors per thread and chunk
  static constexpr int BV = (kTnK * NC / 4 + kThreads - 1) / kThreads;
  static constexpr int LDS = 2 * kTnK * (AP + BP) * 4;
  static_assert(AV * kThreads * 4 == kTnK * ROWS, "A load split");
  static_assert(NBW * WPR == NB, "column tiles split evenly over a row tile's waves");
};
template <int NB, int RW>
__global__ __launch_bounds__(kThreads) void gemm_tn(const float *X, int64_t x_sg, int ldx,
                                                    const float *Y, int64_t y_sg, int ldy,
                                                    float *C, int64_t c_sg, int ldc, int M,
                                                    int Nn, int Kd) {
  using T = TnCfg<NB, RW>;
  constexpr int kTnRows = T::ROWS;
  const int wr = (threadIdx.x >> 6) / T::WPR, wc = (threadIdx.x >> 6) % T::WPR;
  extern __shared__ __align__(16) float tn[];
  float *As = tn;                          // [2][kTnK][AP]
  float *Bs = tn + 2 * kTnK * T::AP;       // [2][kTnK][BP]
  const int g = blockIdx.y, i0 = blockIdx.x * kTnRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *Xg = X + g * x_sg, *Yg = Y + g * y_sg;
  f32x4_v ra[T::AV], rb[T::BV];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < T::AV; ++q) {
      const int e = tid + kThreads * q, kk = e / (kTnRows / 4), c4 = 4 * (e % (kTnRows / 4));
      const bool ok = k0 + kk < Kd && i0 + c4 < M;
      ra[q] = ok ? *reinterpret_cast<const f32x4_v *>(Xg + (int64_t)(k0 + kk) * ldx + i0 + c4)
                 : f32x4_v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < T::BV; ++q) {
      const int e = tid + kThreads * q, kk = e / (T::NC / 4), c4 = 4 * (e % (T::NC / 4));
      const bool ok = e < kTnK * T::NC / 4 && k0 + kk < Kd && c4 < Nn;
      rb[q] = ok ? *reinterpret_cast<const f32x4_v *>(Yg + (int64_t)(k0 + kk) * ldy + c4)
                 : f32x4_v{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < T::AV; ++q) {
      const int e = tid + kThreads * q, kk = e / (kTnRows / 4), c4 = 4 * (e % (kTnRows / 4));
      *reinterpret_cast<f32x4_v *>(As + (buf * kTnK + kk) * T::AP + c4) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < T::BV; ++q) {
      const int e = tid + kThreads * q, kk = e / (T::NC / 4), c4 = 4 * (e % (T::NC / 4));
      if (e < kTnK * T::NC / 4)
        *reinterpret_cast<f32x4_v *>(Bs + (buf * kTnK + kk) * T::BP + c4) = rb[q];
    }
  };
  f32x16_t acc[T::NBW];
#pragma unroll
  for (int nb = 0; nb < T::NBW; ++nb) acc[nb] = f32x16_t{};
  fetch(0);
  stage(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < Kd; k0 += kTnK) {
    const bool more = k0 + kTnK < Kd;
    if (more) fetch(k0 + kTnK);
    const float *Ab = As + buf * kTnK * T::AP + 32 * wr + (lane & 31);
    const float *Bb = Bs + buf * kTnK * T::BP + 32 * T::NBW * wc + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < kTnK; kk += 2) {
      // A: row 32 wave + lane % 32, k = kk + lane / 32;  B: column 32 nb + lane % 32
      const int kr = kk + (lane >> 5);
      const float a = Ab[kr * T::AP];
#pragma unroll
      for (int nb = 0; nb < T::NBW; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bb[kr * T::BP + 32 * nb], acc[nb], 0, 0,
                                                       0);
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // accumulator r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int nb = 0; nb < T::NBW; ++nb) {
    const int j = 32 * (T::NBW * wc + nb) + (lane & 31);
    if (j >= Nn) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 32 * wr + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (i < M) C[g * c_sg + (int64_t)i * ldc + j] = acc[nb][r];
    }
  }
}

// Gram matrix tiles: 128 x 128 outputs, samples staged in chunks of 32.
constexpr int kGT = 128;  // output tile
constexpr int kGN = 32;   // samples per chunk
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

// Gram matrix of the centred calibration rows, C[g] = Xc^T Xc with
// Xc[n][f] = x[n][g][f] - mu[g][f], on the bf16 matrix cores to fp32
// accuracy.  Every centred value y = x - mu (fp32) is split exactly into
// three bf16 parts, y = h + m + l (8 significant bits each: h = bf16(y),
// m = bf16(y - h), l = bf16(y - h - m)), and a product y_a y_b is formed from
// the six partial products whose size reaches 2^-24 |y_a y_b|: hh, hm, mh,
// mm, hl, lh (the dropped ml, lm, ll are below it, as an fp32 product's own
// rounding is); products are exact and sums fp32.  Six
// v_mfma_f32_32x32x16_bf16 take the place of eight v_mfma_f32_32x32x2_f32 per
// 32 x 32 block and 16 samples, at 32 against 64 cycles each.
// C is symmetric: only the 128 x 128 tiles (ti, tj) with ti <= tj are
// computed, those off the diagonal also written transposed; four waves, each
// a 64 x 64 quarter of the tile as 2 x 2 blocks of 32 x 32.  The
// operands want 8 consecutive samples of one feature per lane, so chunks of
// 32 samples are staged feature-major, one plane per part, in one buffer
// (two workgroups per CU; the next chunk waits in registers); a thread loads
// the 8 features of its 16-byte vector for two adjacent samples and writes
// each feature's pair as one 4-byte word.  Feature f of the tile sits in LDS
// row (f % 8) 16 + f / 8, so that the rows one such write touches across a
// wave fall in distinct banks; the tile goes out through LDS, where the
// permutation is undone and both stores are coalesced.
constexpr int kG3P = kGN + 8;                             // bf16 per LDS row (80 bytes)
constexpr int kG3Plane = kGT * kG3P;                      // bf16 per plane
// one staging buffer [operand][part][row][sample] (two workgroups per CU),
// or the output tile [kGT][kGT + 1] fp32, whichever is larger
constexpr int kGram3Lds = 2 * 3 * kG3Plane * 2 > kGT * (kGT + 1) * 4 ? 2 * 3 * kG3Plane * 2
                                                                     : kGT * (kGT + 1) * 4;
__device__ __forceinline__ int g3_row(int f) { return (f & 7) * (kGT / 8) + (f >> 3); }
__device__ __forceinline__ int g3_feature(int r) { return (r % (kGT / 8)) * 8 + r / (kGT / 8); }
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short g3_bf16x8_t;

template <typename E>
__global__ __launch_bounds__(kThreads) void gram3(const E *x, const float *mu, int G, int N, int K,
                                                   float *C) {
  extern __shared__ __align__(16) uint16_t g3[];
  const int T = (K + kGT - 1) / kGT;
  int t = blockIdx.x, ti = 0;
  while (t >= T - ti) {  // upper-triangle tile (ti, tj), ti <= tj
    t -= T - ti;
    ++ti;
  }
  const int tj = ti + t, g = blockIdx.y;
  const int i0 = ti * kGT, j0 = tj * kGT;
  const bool diag = ti == tj;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  // features f8 .. f8 + 7 of the tile, samples 2 np and 2 np + 1 of a chunk
  const int f8 = (tid % (kGT / 8)) * 8, np = tid / (kGT / 8);
  const int fa = i0 + f8, fb = j0 + f8;
  float mua[8], mub[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mua[e] = fa + e < K ? mu[(int64_t)g * K + fa + e] : 0.f;
    mub[e] = fb + e < K ? mu[(int64_t)g * K + fb + e] : 0.f;
  }
  const bool fa_ok = fa < K, fb_ok = fb < K;  // K % 8 == 0: whole vectors in or out
  const int fa_c = fa_ok ? fa : 0, fb_c = fb_ok ? fb : 0;
  constexpr int NV = sizeof(E) == 2 ? 1 : 2;
  u32x4_v ra[2][NV], rb[2][NV];
  auto fetch = [&](int n0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = min(n0 + 2 * np + q, N - 1);
      const int64_t row = ((int64_t)n * G + g) * K;
      const u32x4_v *pa = reinterpret_cast<const u32x4_v *>(x + row + fa_c);
      const u32x4_v *pb = reinterpret_cast<const u32x4_v *>(x + row + (diag ? fa_c : fb_c));
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        ra[q][v] = pa[v];
        rb[q][v] = pb[v];
      }
    }
  };
  auto unpack = [&](const u32x4_v (&raw)[NV], float (&dst)[8]) {
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = bf16_lo(raw[0][e]);
        dst[2 * e + 1] = bf16_hi(raw[0][e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = __uint_as_float(raw[e / 4][e % 4]);
    }
  };
  // the two samples' centred values of 8 features -> three planes of pairs
  auto put = [&](uint16_t *plane0, const float (&y0)[8], const float (&y1)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float h0 = bf16_bits_to_f32(f32_to_bf16_bits(y0[e]));
      const float h1 = bf16_bits_to_f32(f32_to_bf16_bits(y1[e]));
      const float r0 = y0[e] - h0, r1 = y1[e] - h1;
      const float m0 = bf16_bits_to_f32(f32_to_bf16_bits(r0));
      const float m1 = bf16_bits_to_f32(f32_to_bf16_bits(r1));
      uint32_t *w = reinterpret_cast<uint32_t *>(plane0 + g3_row(f8 + e) * kG3P + 2 * np);
      w[0] = pack_bf16x2(h0, h1);
      w[kG3Plane / 2] = pack_bf16x2(m0, m1);
      w[kG3Plane] = pack_bf16x2(r0 - m0, r1 - m1);
    }
  };
  auto stage = [&](int n0) {
    uint16_t *pa = g3, *pb = pa + 3 * kG3Plane;
    float va[2][8], vb[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool nok = n0 + 2 * np + q < N;
      unpack(ra[q], va[q]);
      unpack(rb[q], vb[q]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        va[q][e] = nok && fa_ok ? va[q][e] - mua[e] : 0.f;
        vb[q][e] = nok && fb_ok ? vb[q][e] - mub[e] : 0.f;
      }
    }
    put(pa, va[0], va[1]);
    if (!diag) put(pb, vb[0], vb[1]);
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16_t{};
  fetch(0);
  stage(0);
  __syncthreads();
  for (int n0 = 0; n0 < N; n0 += kGN) {
    const bool more = n0 + kGN < N;
    if (more) fetch(n0 + kGN);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the products
    const uint16_t *pa = g3;
    const uint16_t *pb = diag ? pa : pa + 3 * kG3Plane;
#pragma unroll
    for (int ks = 0; ks < kGN / 16; ++ks) {
      // lane: row (feature slot) lane % 32 of its block, samples 16 ks + 8 (lane / 32) ..
      const int off = (lane & 31) * kG3P + 16 * ks + 8 * (lane >> 5);
      g3_bf16x8_t A[2][3], B[2][3];
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
          A[a][pt] = *reinterpret_cast<const g3_bf16x8_t *>(
              pa + pt * kG3Plane + (wi * 64 + 32 * a) * kG3P + off);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          B[b][pt] = *reinterpret_cast<const g3_bf16x8_t *>(
              pb + pt * kG3Plane + (wj * 64 + 32 * b) * kG3P + off);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          f32x16_t c = acc[a][b];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][0], B[b][2], c, 0, 0, 0);  // h l
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][2], B[b][0], c, 0, 0, 0);  // l h
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][1], B[b][1], c, 0, 0, 0);  // m m
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][0], B[b][1], c, 0, 0, 0);  // h m
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][1], B[b][0], c, 0, 0, 0);  // m h
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a][0], B[b][0], c, 0, 0, 0);  // h h
          acc[a][b] = c;
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // and are waited for only after them
    __syncthreads();                    // every wave is done with this chunk
    if (more) stage(n0 + kGN);
    __syncthreads();
  }
  // accumulator r of block (a, b): LDS rows 64 wi + 32 a + 8 (r / 4) +
  // 4 (lane / 32) + r % 4 and 64 wj + 32 b + lane % 32, i.e. the features
  // g3_feature() of those; the tile [fi][fj] goes through LDS
  float *tr = reinterpret_cast<float *>(g3);  // [kGT][kGT + 1]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 64 * wi + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int jl = 64 * wj + 32 * b + (lane & 31);
        tr[g3_feature(il) * (kGT + 1) + g3_feature(jl)] = acc[a][b][r];
      }
  __syncthreads();
  float *Cg = C + (int64_t)g * K * K;
  for (int e = tid; e < kGT * kGT; e += kThreads) {
    const int il = e / kGT, jl = e % kGT;  // C[i][j], consecutive j per lane
    if (i0 + il < K && j0 + jl < K) Cg[(int64_t)(i0 + il) * K + j0 + jl] = tr[il * (kGT + 1) + jl];
  }
  if (diag) return;  // workgroup-uniform
  for (int e = tid; e < kGT * kGT; e += kThreads) {
    const int jl = e / kGT, il = e % kGT;  // C[j][i] = tile[i][j], consecutive i per lane
    if (j0 + jl < K && i0 + il < K) Cg[(int64_t)(j0 + jl) * K + i0 + il] = tr[il * (kGT + 1) + jl];
  }
}


// mu[g][f] = (1/N) sum_n x[n][g][f] in fp64: a block covers 32 features;
// its 8 row groups (n = r, r + 8, ...) sum in parallel and are added in a
// fixed order at the end.
// mu[g][f] = (1/N) sum_n x[n][g][f] (fp64 sums) for rows of whole 16-byte
// vectors: a block takes 64 features of one codec; its threads read one
// vector of a row each (the block's rows 128 contiguous bytes), row groups
// of a block take every (256 / vectors per row)-th row, four rows in flight,
// with one fp64 sum per feature, and the groups' sums are added through LDS
// in a fixed order.
constexpr int kMeanVF = 64;  // features per block
template <typename E>
__global__ __launch_bounds__(kThreads) void column_mean_vec(const E *x, int G, int N, int K,
                                                            float *mu) {
  constexpr int VEC = 16 / (int)sizeof(E);   // features per 16-byte vector
  constexpr int VPR = kMeanVF / VEC;         // vectors per row of the block
  constexpr int RG = kThreads / VPR;         // row groups
  __shared__ double part[RG][kMeanVF];
  const int g = blockIdx.y, v = threadIdx.x % VPR, rg = threadIdx.x / VPR;
  const int f0 = blockIdx.x * kMeanVF + v * VEC;
  const bool ok = f0 < K;  // K % VEC == 0: whole vectors in or out
  double s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.0;
  auto add = [&](const u32x4_v &w) {
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[2 * e] += (double)bf16_lo(w[e]);
        s[2 * e + 1] += (double)bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += (double)__uint_as_float(w[e]);
    }
  };
  if (ok) {
    const u32x4_v *base = reinterpret_cast<const u32x4_v *>(x + (int64_t)g * K + f0);
    const int64_t rs = (int64_t)G * K / VEC;  // 16-byte words per row
    int n = rg;
    for (; n + 3 * RG < N; n += 4 * RG) {
      u32x4_v w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = base[(int64_t)(n + u * RG) * rs];
#pragma unroll
      for (int u = 0; u < 4; ++u) add(w[u]);
    }
    for (; n < N; n += RG) add(base[(int64_t)n * rs]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[rg][v * VEC + e] = s[e];
  __syncthreads();
  if (threadIdx.x < kMeanVF) {
    const int f = blockIdx.x * kMeanVF + threadIdx.x;
    double t = 0.0;
    for (int r = 0; r < RG; ++r) t += part[r][threadIdx.x];
    if (f < K) mu[(int64_t)g * K + f] = (float)(t / N);
  }
}

constexpr int kMeanF = 32, kMeanR = kThreads / kMeanF;
template <typename E>
__global__ __launch_bounds__(kThreads) void column_mean(const E *x, int G, int N, int K, float *mu) {
  __shared__ double part[kMeanR][kMeanF];
  const int g = blockIdx.y, fx = threadIdx.x % kMeanF, ry = threadIdx.x / kMeanF;
  const int f = blockIdx.x * kMeanF + fx;
  double s = 0.0;
  if (f < K)
    for (int n = ry; n < N; n += kMeanR) s += load_elem(x, ((int64_t)n * G + g) * K + f);
  part[ry][fx] = s;
  __syncthreads();
  if (ry == 0 && f < K) {
    double t = 0.0;
#pragma unroll
    for (int r = 0; r < kMeanR; ++r) t += part[r][fx];
    mu[(int64_t)g * K + f] = (float)(t / N);
  }
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) at counter i: the
// starting block of the iteration, uniform in [-1, 1).
__device__ __forceinline__ float start_value(uint64_t i) {
  uint64_t z = (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (float)((double)(z >> 11) * 0x1.0p-52 - 1.0);
}

__global__ __launch_bounds__(kThreads) void start_block(float *Q, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    Q[i] = start_value((uint64_t)i);
}

// out[part][g][i][j] = sum over the part's rows k of P[g][k][i] * R[g][k][j]
// in fp64 (P, R: [K][m] fp32; parts of kSmallGramParts row ranges, so that
// a few codecs still fill the GPU; the consumers add the parts in order).
// Block = (32 x 32 output tile, g and part), eight waves: wave w multiplies quadrant
// w % 4 over half w / 4 of every chunk of 64 k, one v_mfma_f64_16x16x4f64
// per four k (fp32 products are exact in fp64, the sums are fp64); the two
// halves are added through LDS at the end.  Chunks are staged in LDS as
// whole 128-byte rows, the next chunk loaded into registers while the
// current one is multiplied.  With sym (P == R) only tiles on and above the
// diagonal run, and each entry i <= j is also written at (j, i), so that the
// result is exactly symmetric.
// Operand lanes: A row l % 16 and B column l % 16 of the quadrant at
// k = 4 s + l / 16; accumulator entry e: row l / 16 + 4 e, column l % 16 (the
// f64 form interleaves its rows, unlike the f32 16x16x4 form's 4 (l / 16) + e).
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kSgThreads = 512;
constexpr int kSgT = 32;   // output tile
constexpr int kSgK = 64;   // k per chunk
constexpr int kSgPer = kSgK * kSgT / kSgThreads;  // elements per thread, operand and chunk
__global__ __launch_bounds__(kSgThreads) void small_gram64(const float *P, const float *R, int K,
                                                           int m, int sym, double *out) {
  if (sym && blockIdx.y > blockIdx.x) return;
  __shared__ float As[2][kSgK][kSgT + 1], Bs[2][kSgK][kSgT + 1];
  __shared__ double part[4][4][64];
  const int g = blockIdx.z / kSmallGramParts, sp = blockIdx.z % kSmallGramParts;
  const int i0 = blockIdx.y * kSgT, j0 = blockIdx.x * kSgT;
  // this part's rows [kb, ke), whole chunks of kSgK (an empty range writes zeros)
  const int span = ((K + kSmallGramParts - 1) / kSmallGramParts + kSgK - 1) / kSgK * kSgK;
  const int kb = sp * span, ke = min(K, kb + span);
  out += (int64_t)sp * (gridDim.z / kSmallGramParts) * m * m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kl = lane >> 4;
  const int qi = (wave >> 1) & 1, qj = wave & 1, kh = wave >> 2;
  const float *Pg = P + (int64_t)g * K * m, *Rg = R + (int64_t)g * K * m;
  float ra[kSgPer], rb[kSgPer];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < kSgPer; ++q) {
      const int e = tid + kSgThreads * q, kk = k0 + e / kSgT, c = e % kSgT;
      ra[q] = kk < ke && i0 + c < m ? Pg[(int64_t)kk * m + i0 + c] : 0.f;
      rb[q] = kk < ke && j0 + c < m ? Rg[(int64_t)kk * m + j0 + c] : 0.f;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kSgPer; ++q) {
      const int e = tid + kSgThreads * q;
      As[buf][e / kSgT][e % kSgT] = ra[q];
      Bs[buf][e / kSgT][e % kSgT] = rb[q];
    }
  };
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
  fetch(kb);
  stage(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += kSgK) {
    const bool more = k0 + kSgK < ke;
    if (more) fetch(k0 + kSgK);
#pragma unroll
    for (int s = 0; s < kSgK / 8; ++s) {
      const int kk = kh * (kSgK / 2) + 4 * s + kl;
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)As[buf][kk][qi * 16 + (lane & 15)],
                                                 (double)Bs[buf][kk][qj * 16 + (lane & 15)], acc,
                                                 0, 0, 0);
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if (kh)
    for (int e = 0; e < 4; ++e) part[wave & 3][e][lane] = acc[e];
  __syncthreads();
  if (!kh) {
    const int j = j0 + qj * 16 + (lane & 15);
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + qi * 16 + kl + 4 * e;
      const double v = acc[e] + part[wave][e][lane];
      if (i >= m || j >= m) continue;
      if (!sym) {
        out[((int64_t)g * m + i) * m + j] = v;
      } else if (i <= j) {
        out[((int64_t)g * m + i) * m + j] = v;
        out[((int64_t)g * m + j) * m + i] = v;
      }
    }
  }
}

// Cholesky A = L L^T of one codec's m x m matrix (fp64, with a tiny diagonal
// shift so that a rank-deficient block cannot break it), then
// Rinv = (L^T)^-1 = X^T with X = L^-1, the factor that makes Y Rinv
// orthonormal.  The array M holds L in its lower triangle and X transposed
// in its strict upper one (X[i][c] at (c, i); X starts as the identity).
// Thread (ty, tx) of a 16 x 16 block keeps the entries (r, col) with
// r = ty + 16 a and col = tx + 16 b (a, b < Q, 16 Q >= m) in registers.
// Step j: the owners of column j publish it to LDS (one barrier, two
// buffers); every thread reads the pivot and the entries of its rows and
// columns at once, forms 1 / d = 1 / sqrt(M[j][j]) itself (hardware
// reciprocal square root, two Newton steps) and w = column j / d,
// w[j] = 1 / d: column j of L scaled below the diagonal, row j of X above
// it.  Forward elimination of L (trailing update l_rj l_colj) and of the
// identity (X[col][r] -= l_colj X[j][r], r <= j) are then one update
// M[r][col] -= w[r] w[col], col > j.  It also reaches the upper entries
// j < r < col, which are not yet X's; row j is zeroed before its update, so
// those start from zero when they become X's, and L's rows left of the
// diagonal, no longer read once their column is published, may hold
// anything.  The owners of column j then store w there (final: 1 / d on the
// diagonal, which is Rinv's).
constexpr int kCholThreads = 256;
constexpr int kCholT = 16;  // kCholT x kCholT threads
template <int Q>
__global__ __launch_bounds__(kCholThreads) void chol_inv(const double *A, int m, float *Rinv) {
  __shared__ double buf[2][Q * kCholT];
  const int g = blockIdx.x, tid = threadIdx.x, ty = tid / kCholT, tx = tid % kCholT;
  const double *Ag = A + (int64_t)g * m * m;
  const int64_t pst = (int64_t)gridDim.x * m * m;  // between the small Gram parts
  auto a_at = [&](int r, int c) {
    double v = Ag[(int64_t)r * m + c];
#pragma unroll
    for (int sp = 1; sp < kSmallGramParts; ++sp) v += Ag[sp * pst + (int64_t)r * m + c];
    return v;
  };
  double v[Q][Q];
#pragma unroll
  for (int a = 0; a < Q; ++a)
#pragma unroll
    for (int b = 0; b < Q; ++b) {
      const int r = ty + kCholT * a, col = tx + kCholT * b;
      v[a][b] = r < m && col <= r ? a_at(r, col) : 0.0;
    }
  // the diagonal, from its owners (ty == tx, a == b), for the shift
  if (ty == tx) {
#pragma unroll
    for (int a = 0; a < Q; ++a)
      if (ty + kCholT * a < m) buf[0][ty + kCholT * a] = v[a][a];
  }
  __syncthreads();
  double dmax = 0.0;
  for (int i = 0; i < m; ++i) dmax = fmax(dmax, buf[0][i]);
  const double shift = 1e-13 * dmax + 1e-300;
  __syncthreads();  // step 0 publishes into the same buffer
  // j = 16 jo + jl: the block jo is a constant in each unrolled copy, so the
  // owners' slots are known and the finished column blocks b < jo (w = 0)
  // are skipped
#pragma unroll
  for (int jo = 0; jo < Q; ++jo) {
#pragma unroll 1
    for (int jl = 0; jl < kCholT; ++jl) {
      const int j = kCholT * jo + jl;
      if (j >= m) break;
      double *bj = buf[j & 1];
      const bool owner = tx == jl;
      if (owner) {
#pragma unroll
        for (int a = 0; a < Q; ++a)
          if (ty + kCholT * a < m) bj[ty + kCholT * a] = v[a][jo];
      }
      __syncthreads();
      const double piv = bj[j];
      double br[Q], bc[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        br[q] = bj[min(ty + kCholT * q, m - 1)];
        bc[q] = bj[min(tx + kCholT * q, m - 1)];
      }
      const double x = fmax(piv + shift, shift);
      double inv = __builtin_amdgcn_rsq(x);
#pragma unroll
      for (int it = 0; it < 2; ++it) inv = fma(0.5 * inv, fma(-x * inv, inv, 1.0), inv);
      double wr[Q], wc[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        wr[q] = q == jo && ty == jl ? inv : br[q] * inv;
        wc[q] = q > jo || (q == jo && tx > jl) ? bc[q] * inv : 0.0;
      }
      if (ty == jl) {
#pragma unroll
        for (int b = jo; b < Q; ++b) v[jo][b] = 0.0;
      }
#pragma unroll
      for (int a = 0; a < Q; ++a)
#pragma unroll
        for (int b = jo; b < Q; ++b) v[a][b] = fma(-wr[a], wc[b], v[a][b]);
      if (owner) {
#pragma unroll
        for (int a = 0; a < Q; ++a) v[a][jo] = wr[a];
      }
    }
  }
  // Rinv[c][i] = X[i][c]: M[c][i] above the diagonal, 1 / l_cc on it
  float *Rg = Rinv + (int64_t)g * m * m;
#pragma unroll
  for (int a = 0; a < Q; ++a)
#pragma unroll
    for (int b = 0; b < Q; ++b) {
      const int r = ty + kCholT * a, col = tx + kCholT * b;
      if (r < m && col < m) Rg[(int64_t)r * m + col] = col >= r ? (float)v[a][b] : 0.f;
    }
}

// Symmetric eigenproblem of one codec's m x m matrix B (fp64, in LDS) by
// cyclic Jacobi rotations; disjoint pairs of a round-robin schedule rotate in
// parallel.  One round applies B <- J^T B J and U <- U J in a single pass:
// the entries in rows (a, b) of one pair and columns (a', b') of another
// depend only on those four entries and the two rotations, so each thread
// takes such 2 x 2 blocks (rows first, then columns, as two sequential
// passes would) and its column pair's slice of U.  B is zero-padded to an
// even order; the odd player's pair rotates by the identity.  U sits in LDS
// when both matrices fit (kLdsU), else in the workspace.  Writes the
// eigenvalues, the order that sorts them descending (ties by index), and
// Usel[k][j] = U[k][order[j]] (j < r, fp32) for the final GEMM.
constexpr int kJacThreads = 1024;
constexpr int kJacWaves = kJacThreads / 64;
__host__ __device__ constexpr size_t jacobi_lds(int m, bool lds_u) {
  return (size_t)(m + (m & 1)) * (m + (m & 1)) * 8 + (lds_u ? (size_t)m * m * 8 : 0) +
         (size_t)(m + (m & 1)) * 8 + (size_t)2 * kJacWaves * 8 + (size_t)(m + (m & 1)) * 4;
}
template <bool kLdsU>
__global__ __launch_bounds__(kJacThreads) void jacobi(const double *B, int m, int sweeps,
                                                      double *Uws, double *evals, int *order,
                                                      int r, float *Usel) {
  // S [mp][mp], U [m][m] (kLdsU), rotations cs [npair][2], wave sums
  // [2][kJacWaves], pairs pr [npair][2] (at the end: the order)
  extern __shared__ double S[];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int mp = m + (m & 1);  // players; index m (odd m) is the zero pad
  const int npair = mp / 2;
  double *U = kLdsU ? S + mp * mp : Uws + (int64_t)g * m * m;
  double *cs = S + mp * mp + (kLdsU ? m * m : 0);
  double *red = cs + 2 * npair;
  int *pr = reinterpret_cast<int *>(red + 2 * kJacWaves);
  const double *Bg = B + (int64_t)g * m * m;
  const int64_t pst = (int64_t)gridDim.x * m * m;  // between the small Gram parts
  auto b_at = [&](int i, int j) {
    double v = Bg[i * m + j];
#pragma unroll
    for (int sp = 1; sp < kSmallGramParts; ++sp) v += Bg[sp * pst + i * m + j];
    return v;
  };
  for (int e = tid; e < mp * mp; e += kJacThreads) {
    const int i = e / mp, j = e % mp;
    S[e] = i < m && j < m ? 0.5 * (b_at(i, j) + b_at(j, i)) : 0.0;  // exact symmetry
  }
  for (int e = tid; e < m * m; e += kJacThreads) U[e] = e / m == e % m ? 1.0 : 0.0;
  // this thread's column pair, and its first row pair / row of U
  const int rpp = kJacThreads / npair;
  const bool active = tid < rpp * npair;
  const int k2 = tid % npair, r0 = tid / npair;
  __syncthreads();
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int rd = 0; rd < mp - 1; ++rd) {
      if (tid < npair) {
        const int a = (rd + tid) % (mp - 1), b = tid == 0 ? mp - 1 : (rd + mp - 1 - tid) % (mp - 1);
        double c = 1.0, s = 0.0;
        if (b < m) {
          const double app = S[a * mp + a], aqq = S[b * mp + b], apq = S[a * mp + b];
          if (fabs(apq) > 1e-300 && fabs(apq) > 1e-18 * (fabs(app) + fabs(aqq))) {
            const double tau = (aqq - app) / (2.0 * apq);
            const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
          }
        }
        cs[2 * tid] = c;
        cs[2 * tid + 1] = s;
        pr[2 * tid] = a;
        pr[2 * tid + 1] = b;
      }
      __syncthreads();
      if (active) {
        const int a2 = pr[2 * k2], b2 = pr[2 * k2 + 1];
        const double c2 = cs[2 * k2], s2 = cs[2 * k2 + 1];
        for (int k = r0; k < npair; k += rpp) {
          const int a = pr[2 * k], b = pr[2 * k + 1];
          const double c = cs[2 * k], s = cs[2 * k + 1];
          double *Sa = S + a * mp, *Sb = S + b * mp;
          const double xaa = Sa[a2], xab = Sa[b2], xba = Sb[a2], xbb = Sb[b2];
          const double yaa = c * xaa - s * xba, yab = c * xab - s * xbb;  // rows
          const double yba = s * xaa + c * xba, ybb = s * xab + c * xbb;
          Sa[a2] = c2 * yaa - s2 * yab;  // columns
          Sa[b2] = s2 * yaa + c2 * yab;
          Sb[a2] = c2 * yba - s2 * ybb;
          Sb[b2] = s2 * yba + c2 * ybb;
        }
        if (b2 < m) {
          for (int i = r0; i < m; i += rpp) {
            const double ua = U[i * m + a2], ub = U[i * m + b2];
            U[i * m + a2] = c2 * ua - s2 * ub;
            U[i * m + b2] = s2 * ua + c2 * ub;
          }
        }
      }
      __syncthreads();
    }
    // stop once the off-diagonal part is negligible against the diagonal
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < mp * mp; e += kJacThreads) {
      const double v = S[e] * S[e];
      if (e / mp == e % mp) dia += v; else off += v;
    }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      dia += __shfl_xor(dia, o);
    }
    if ((tid & 63) == 0) {
      red[tid >> 6] = off;
      red[kJacWaves + (tid >> 6)] = dia;
    }
    __syncthreads();
    off = dia = 0.0;
    for (int w = 0; w < kJacWaves; ++w) {
      off += red[w];
      dia += red[kJacWaves + w];
    }
    if (off <= 1e-24 * dia) break;  // the same decision in every thread
  }
  // rank of each eigenvalue, descending, ties (and NaN, ranked last) by index
  for (int i = tid; i < m; i += kJacThreads) {
    const double li = S[i * (mp + 1)], ki = li == li ? li : -INFINITY;
    int rank = 0;
    for (int j = 0; j < m; ++j) {
      const double lj = S[j * (mp + 1)], kj = lj == lj ? lj : -INFINITY;
      rank += kj > ki || (kj == ki && j < i);
    }
    pr[rank] = i;  // no thread reads the pairs any more
    order[(int64_t)g * m + rank] = i;
    evals[(int64_t)g * m + i] = li;
  }
  __syncthreads();
  for (int e = tid; e < m * r; e += kJacThreads) {
    const int k = e / r, j = e % r;
    Usel[((int64_t)g * m + k) * r + j] = (float)U[k * m + pr[j]];
  }
}

// Column j of W (fp32 [G][K][r]): sign fixed so that its entry of largest
// magnitude is positive, rounded into w_down [G][K][r] and the loop slices
// w_up [T][G][width][r]; sigma_j = sqrt(max(lambda_j, 0)).
template <typename E>
__global__ __launch_bounds__(kThreads) void finalize(const float *W, const double *evals,
                                                     const int *order, int G, int K, int m, int r,
                                                     int T, int width, E *w_down, E *w_up,
                                                     float *sigma) {
  __shared__ float best_v[kThreads];
  __shared__ int best_i[kThreads];
  const int j = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const float *Wg = W + (int64_t)g * K * r;
  float bv = -1.f;
  int bi = 0;
  for (int k = tid; k < K; k += kThreads) {
    const float a = fabsf(Wg[(int64_t)k * r + j]);
    if (a > bv) {
      bv = a;
      bi = k;
    }
  }
  best_v[tid] = bv;
  best_i[tid] = bi;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (tid < h) {
      const float o = best_v[tid + h];
      const int oi = best_i[tid + h];
      if (o > best_v[tid] || (o == best_v[tid] && oi < best_i[tid])) {
        best_v[tid] = o;
        best_i[tid] = oi;
      }
    }
    __syncthreads();
  }
  const float sgn = Wg[(int64_t)best_i[0] * r + j] < 0.f ? -1.f : 1.f;
  for (int k = tid; k < K; k += kThreads) {
    const float v = sgn * Wg[(int64_t)k * r + j];
    store_elem(w_down, ((int64_t)g * K + k) * r + j, v);
    const int t = k / width, i = k % width;
    store_elem(w_up, (((int64_t)t * G + g) * width + i) * r + j, v);
  }
  if (tid == 0 && sigma) {
    const double lam = evals[(int64_t)g * m + order[(int64_t)g * m + j]];
    sigma[(int64_t)g * r + j] = (float)sqrt(fmax(lam, 0.0));
  }
}

template <class LA, class LB>
hipError_t launch_gemm(const LA &A, const LB &B, float *C, int64_t c_sg, int ldc, int G, int M,
                       int Nn, int Kd, hipStream_t st) {
  const dim3 grid((Nn + kT - 1) / kT, (M + kT - 1) / kT, G);
  hipLaunchKernelGGL((gemm<LA, LB>), grid, dim3(kThreads), 0, st, A, B, C, c_sg, ldc, M, Nn, Kd);
  return hipGetLastError();
}

template <int NB, int RW = 4>
hipError_t launch_gemm_tn_nb(const float *X, int64_t x_sg, int ldx, const float *Y, int64_t y_sg,
                             int ldy, float *C, int64_t c_sg, int ldc, int G, int M, int Nn,
                             int Kd, hipStream_t st) {
  using T = TnCfg<NB, RW>;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tn<NB, RW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_tn<NB, RW>), dim3((M + T::ROWS - 1) / T::ROWS, G), dim3(kThreads),
                     T::LDS, st, X, x_sg, ldx, Y, y_sg, ldy, C, c_sg, ldc, M, Nn, Kd);
  return hipGetLastError();
}
// Needs M, Nn, ldx, ldy multiples of 4, 16-byte aligned X and Y, Nn <= 128.
hipError_t launch_gemm_tn(const float *X, int64_t x_sg, int ldx, const float *Y, int64_t y_sg,
                          int ldy, float *C, int64_t c_sg, int ldc, int G, int M, int Nn, int Kd,
                          hipStream_t st) {
  const int nb = (Nn + 31) / 32;
  if (nb <= 1) return launch_gemm_tn_nb<1>(X, x_sg, ldx, Y, y_sg, ldy, C, c_sg, ldc, G, M, Nn, Kd, st);
  if (nb == 2)
    return launch_gemm_tn_nb<2, 2>(X, x_sg, ldx, Y, y_sg, ldy, C, c_sg, ldc, G, M, Nn, Kd, st);
  if (nb == 3) return launch_gemm_tn_nb<3>(X, x_sg, ldx, Y, y_sg, ldy, C, c_sg, ldc, G, M, Nn, Kd, st);
  return launch_gemm_tn_nb<4>(X, x_sg, ldx, Y, y_sg, ldy, C, c_sg, ldc, G, M, Nn, Kd, st);
}

MatF32 mat(const float *p, int64_t sg, int64_t s0, int64_t s1, int n0, int n1) {
  return MatF32{p, sg, s0, s1, n0, n1};
}


}  // namespace

template <typename E>
static hipError_t run(const SvdParams &p, hipStream_t st) {
  const int G = p.G, N = p.N, K = p.K, m = p.m, r = p.r;
  const SvdLayout L = svd_layout(G, K, m, r);
  char *ws = reinterpret_cast<char *>(p.ws);
  float *C = reinterpret_cast<float *>(ws + L.gram);
  float *Q = reinterpret_cast<float *>(ws + L.q);
  float *Y = reinterpret_cast<float *>(ws + L.y);
  double *Sm = reinterpret_cast<double *>(ws + L.small);
  float *Rinv = reinterpret_cast<float *>(ws + L.rinv);
  double *U = reinterpret_cast<double *>(ws + L.u);
  double *ev = reinterpret_cast<double *>(ws + L.evals);
  int *order = reinterpret_cast<int *>(ws + L.order);
  float *Usel = reinterpret_cast<float *>(ws + L.usel);
  float *W = reinterpret_cast<float *>(ws + L.w);
  const E *x = reinterpret_cast<const E *>(p.x);
  hipError_t e;
#define LLA_TRY(call)                   \
  if ((e = (call)) != hipSuccess) return e;

  if (K % (16 / (int)sizeof(E)) == 0 && ((uintptr_t)x & 15u) == 0)  // rows of 16-byte vectors
    hipLaunchKernelGGL(column_mean_vec<E>, dim3((K + kMeanVF - 1) / kMeanVF, G), dim3(kThreads), 0,
                       st, x, G, N, K, p.mu);
  else
    hipLaunchKernelGGL(column_mean<E>, dim3((K + kMeanF - 1) / kMeanF, G), dim3(kThreads), 0, st,
                       x, G, N, K, p.mu);
  LLA_TRY(hipGetLastError());
  // Gram matrix of the centred rows: C = Xc^T Xc  (K x K, contraction over N)
  if (K % 8 == 0 && ((uintptr_t)x & 15u) == 0) {  // whole 16-byte feature vectors
    const int T = (K + kGT - 1) / kGT;
    LLA_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(gram3<E>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kGram3Lds));
    hipLaunchKernelGGL(gram3<E>, dim3((unsigned)(T * (T + 1) / 2), G), dim3(kThreads), kGram3Lds,
                       st, x, p.mu, G, N, K, C);
    LLA_TRY(hipGetLastError());
  } else {
    LLA_TRY(launch_gemm(Centred<E, true>{x, p.mu, G, N, K}, Centred<E, false>{x, p.mu, G, N, K},
                        C, (int64_t)K * K, K, G, K, K, N, st));
  }
  const int64_t qn = (int64_t)G * K * m;
  hipLaunchKernelGGL(start_block, dim3((unsigned)std::min<int64_t>((qn + kThreads - 1) / kThreads, 65536)),
                     dim3(kThreads), 0, st, Q, qn);
  LLA_TRY(hipGetLastError());

  // U joins the matrix in LDS while both fit the 160 KB of a gfx950
  // workgroup (m <= 100); the matrix alone fits up to m = 128
  const bool jac_u_lds = jacobi_lds(m, true) <= kMaxLds;
  const size_t jac_lds = jacobi_lds(m, jac_u_lds);
  const void *jac = jac_u_lds ? reinterpret_cast<const void *>(jacobi<true>)
                              : reinterpret_cast<const void *>(jacobi<false>);
  LLA_TRY(hipFuncSetAttribute(jac, hipFuncAttributeMaxDynamicSharedMemorySize, (int)jac_lds));
  const dim3 sg_grid((m + kSgT - 1) / kSgT, (m + kSgT - 1) / kSgT, G * kSmallGramParts);
  // C is symmetric: its rows are read as columns (coalesced)
  const MatF32 Ct = mat(C, (int64_t)K * K, 1, K, K, K);
  // dst = C src (C symmetric, so its rows serve as the k-major left operand)
  const bool tn = K % 4 == 0 && m % 4 == 0 && m <= 128 && ((uintptr_t)C & 15) == 0 &&
                  ((uintptr_t)Q & 15) == 0 && ((uintptr_t)Y & 15) == 0;
  auto c_times = [&](const float *src, float *dst) -> hipError_t {
    if (!tn)
      return launch_gemm(Ct, mat(src, (int64_t)K * m, m, 1, K, m), dst, (int64_t)K * m, m, G, K,
                         m, K, st);
    return launch_gemm_tn(C, (int64_t)K * K, K, src, (int64_t)K * m, m, dst, (int64_t)K * m, m, G,
                          K, m, K, st);
  };
  auto orthonormalise = [&](float *src, float *dst) -> hipError_t {
    // CholeskyQR: dst = src R^-1 with src^T src = R^T R
    hipLaunchKernelGGL(small_gram64, sg_grid, dim3(kSgThreads), 0, st, src, src, K, m, 1, Sm);
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    const int q = (m + kCholT - 1) / kCholT;  // m <= 128
    if (q <= 2)
      hipLaunchKernelGGL(chol_inv<2>, dim3(G), dim3(kCholThreads), 0, st, Sm, m, Rinv);
    else if (q <= 4)
      hipLaunchKernelGGL(chol_inv<4>, dim3(G), dim3(kCholThreads), 0, st, Sm, m, Rinv);
    else if (q <= 6)
      hipLaunchKernelGGL(chol_inv<6>, dim3(G), dim3(kCholThreads), 0, st, Sm, m, Rinv);
    else
      hipLaunchKernelGGL(chol_inv<8>, dim3(G), dim3(kCholThreads), 0, st, Sm, m, Rinv);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    return launch_gemm(mat(src, (int64_t)K * m, m, 1, K, m), mat(Rinv, (int64_t)m * m, m, 1, m, m),
                       dst, (int64_t)K * m, m, G, K, m, m, st);
  };
  LLA_TRY(orthonormalise(Q, Y));
  LLA_TRY(orthonormalise(Y, Q));
  for (int it = 0; it < p.iters; ++it) {
    LLA_TRY(c_times(Q, Y));
    LLA_TRY(orthonormalise(Y, Q));   // CholeskyQR2: twice
    LLA_TRY(orthonormalise(Q, Y));
    float *t = Q;  // the orthonormal block is now in Y
    Q = Y;
    Y = t;
  }
  // Rayleigh-Ritz: B = Q^T C Q, B = U diag(lambda) U^T, W = Q U[:, leading r]
  LLA_TRY(c_times(Q, Y));
  hipLaunchKernelGGL(small_gram64, sg_grid, dim3(kSgThreads), 0, st, Q, Y, K, m, 0, Sm);
  LLA_TRY(hipGetLastError());
  if (jac_u_lds)
    hipLaunchKernelGGL(jacobi<true>, dim3(G), dim3(kJacThreads), jac_lds, st, Sm, m, p.sweeps, U, ev,
                       order, r, Usel);
  else
    hipLaunchKernelGGL(jacobi<false>, dim3(G), dim3(kJacThreads), jac_lds, st, Sm, m, p.sweeps, U,
                       ev, order, r, Usel);
  LLA_TRY(hipGetLastError());
  LLA_TRY(launch_gemm(mat(Q, (int64_t)K * m, m, 1, K, m), mat(Usel, (int64_t)m * r, r, 1, m, r), W,
                      (int64_t)K * r, r, G, K, r, m, st));
  hipLaunchKernelGGL(finalize<E>, dim3(r, G), dim3(kThreads), 0, st, W, ev, order, G, K, m, r, p.T,
                     p.width, reinterpret_cast<E *>(p.w_down), reinterpret_cast<E *>(p.w_up),
                     p.sigma);
  return hipGetLastError();
#undef LLA_TRY
}

}  // namespace svd

hipError_t launch_svd_init(const SvdParams &p, int dtype, hipStream_t st) {
  return dtype == LLA_DT_F32 ? svd::run<float>(p, st) : svd::run<bf16_t>(p, st);
}

}  // namespace lla
