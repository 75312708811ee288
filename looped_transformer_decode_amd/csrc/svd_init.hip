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
  L.small = take((size_t)G * m * m * 8);
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

// Gram matrix of the centred calibration rows, C[g] = Xc^T Xc with
// Xc[n][f] = x[n][g][f] - mu[g][f], on the fp32 matrix cores.  C is
// symmetric: only the 128 x 128 tiles (ti, tj) with ti <= tj are computed,
// and those off the diagonal are also written transposed (through LDS, so
// that both stores are coalesced).  Four waves, each a 64 x 64 quarter of
// the tile as 2 x 2 blocks of v_mfma_f32_32x32x2_f32.  Samples are staged in
// LDS in chunks of 32, centred and in fp32, feature-contiguous; the next
// chunk is loaded into registers while the current one is multiplied.
constexpr int kGT = 128;  // output tile
constexpr int kGN = 32;   // samples per chunk
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
constexpr int kGP = kGT + 4;
constexpr int kGramLds = 2 * 2 * kGN * kGP * 4;  // [buf][operand][n][feature] fp32
static_assert(kGT * (kGT + 1) * 4 <= kGramLds, "the transposed store reuses the staging LDS");

template <typename E>
__global__ __launch_bounds__(kThreads) void gram(const E *x, const float *mu, int G, int N, int K,
                                                  float *C) {
  extern __shared__ __align__(16) float gs[];
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
  // This thread loads features f8 .. f8 + 7 of the tile (one 16-byte vector
  // of bf16, or two of fp32) of chunk rows nr and nr + 16.  Loads are never
  // conditional (indices are clamped, values past N or K zeroed afterwards),
  // so that they all go out before the first is waited for.
  const int f8 = (tid % (kGT / 8)) * 8, nr = tid / (kGT / 8);
  const int fa = i0 + f8, fb = j0 + f8;
  float mua[8], mub[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mua[e] = fa + e < K ? mu[(int64_t)g * K + fa + e] : 0.f;
    mub[e] = fb + e < K ? mu[(int64_t)g * K + fb + e] : 0.f;
  }
  const bool fa_ok = fa < K, fb_ok = fb < K;  // K % 8 == 0: whole vectors in or out
  const int fa_c = fa_ok ? fa : 0, fb_c = fb_ok ? fb : 0;
  // raw 16-byte vectors of the two rows (bf16: one per row, fp32: two),
  // converted and centred only when staged, after the chunk's products
  constexpr int NV = sizeof(E) == 2 ? 1 : 2;
  u32x4_v ra[2][NV], rb[2][NV];
  auto fetch = [&](int n0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = min(n0 + nr + 16 * q, N - 1);
      const int64_t row = ((int64_t)n * G + g) * K;
      const u32x4_v *pa = reinterpret_cast<const u32x4_v *>(x + row + fa_c);
      const u32x4_v *pb = reinterpret_cast<const u32x4_v *>(x + row + (diag ? fa_c : fb_c));
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        ra[q][v] = pa[v];
        rb[q][v] = pb[v];  // on the diagonal a second copy of the same features (unused)
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
  auto stage = [&](int buf, int n0) {
    float *sa = gs + (buf * 2) * kGN * kGP, *sb = sa + kGN * kGP;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool nok = n0 + nr + 16 * q < N;
      float va[8], vb[8];
      unpack(ra[q], va);
      unpack(rb[q], vb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        va[e] = nok && fa_ok ? va[e] - mua[e] : 0.f;
        vb[e] = nok && fb_ok ? vb[e] - mub[e] : 0.f;
      }
      float *da = sa + (nr + 16 * q) * kGP + f8;
      *reinterpret_cast<float4 *>(da) = make_float4(va[0], va[1], va[2], va[3]);
      *reinterpret_cast<float4 *>(da + 4) = make_float4(va[4], va[5], va[6], va[7]);
      if (!diag) {
        float *db = sb + (nr + 16 * q) * kGP + f8;
        *reinterpret_cast<float4 *>(db) = make_float4(vb[0], vb[1], vb[2], vb[3]);
        *reinterpret_cast<float4 *>(db + 4) = make_float4(vb[4], vb[5], vb[6], vb[7]);
      }
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16_t{};
  fetch(0);
  stage(0, 0);
  __syncthreads();
  int buf = 0;
  for (int n0 = 0; n0 < N; n0 += kGN) {
    const bool more = n0 + kGN < N;
    if (more) fetch(n0 + kGN);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the products
    const float *sa = gs + (buf * 2) * kGN * kGP;
    const float *sb = diag ? sa : sa + kGN * kGP;
#pragma unroll
    for (int kk = 0; kk < kGN; kk += 2) {
      const int r = (kk + (lane >> 5)) * kGP + (lane & 31);
      float av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = sa[r + wi * 64 + 32 * a];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = sb[r + wj * 64 + 32 * b];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // and are waited for only after them
    if (more) stage(buf ^ 1, n0 + kGN);
    __syncthreads();
    buf ^= 1;
  }
  // tile rows i (features of the first operand), columns j: accumulator r of
  // block (a, b) is row 64 wi + 32 a + 8 (r / 4) + 4 (lane / 32) + r % 4,
  // column 64 wj + 32 b + lane % 32
  float *Cg = C + (int64_t)g * K * K;
  float *tr = gs;  // [kGT][kGT + 1]: the tile, for the transposed store
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 64 * wi + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int jl = 64 * wj + 32 * b + (lane & 31);
        if (i0 + il < K && j0 + jl < K) Cg[(int64_t)(i0 + il) * K + j0 + jl] = acc[a][b][r];
        if (!diag) tr[il * (kGT + 1) + jl] = acc[a][b][r];
      }
  if (diag) return;  // workgroup-uniform
  __syncthreads();
  for (int e = tid; e < kGT * kGT; e += kThreads) {
    const int jl = e / kGT, il = e % kGT;  // C[j][i] = tile[i][j], consecutive i per lane
    if (j0 + jl < K && i0 + il < K) Cg[(int64_t)(j0 + jl) * K + i0 + il] = tr[il * (kGT + 1) + jl];
  }
}

// mu[g][f] = (1/N) sum_n x[n][g][f] in fp64: a block covers 32 features;
// its 8 row groups (n = r, r + 8, ...) sum in parallel and are added in a
// fixed order at the end.
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

// out[g][i][j] = sum_k P[g][k][i] * R[g][k][j] in fp64 (P, R: [K][m] fp32).
// Block = (16 x 16 output tile, g); k in chunks of 64 through LDS.
__global__ __launch_bounds__(kThreads) void small_gram64(const float *P, const float *R, int K,
                                                         int m, double *out) {
  __shared__ float Ps[64][17], Rs[64][17];
  const int g = blockIdx.z, i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  const float *Pg = P + (int64_t)g * K * m, *Rg = R + (int64_t)g * K * m;
  double acc = 0.0;
  for (int k0 = 0; k0 < K; k0 += 64) {
    for (int e = tid; e < 64 * 16; e += kThreads) {
      const int kk = e / 16, c = e % 16, k = k0 + kk;
      Ps[kk][c] = (k < K && i0 + c < m) ? Pg[(int64_t)k * m + i0 + c] : 0.f;
      Rs[kk][c] = (k < K && j0 + c < m) ? Rg[(int64_t)k * m + j0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) acc = fma((double)Ps[kk][ti], (double)Rs[kk][tj], acc);
    __syncthreads();
  }
  if (i0 + ti < m && j0 + tj < m) out[((int64_t)g * m + i0 + ti) * m + j0 + tj] = acc;
}

// Cholesky A = L L^T of one codec's m x m matrix (fp64, in LDS, with a tiny
// diagonal shift so that a rank-deficient block cannot break it), then
// Rinv = (L^T)^-1, the factor that makes Y Rinv orthonormal.
// Factorisation step j: every thread forms the pivot itself and updates its
// (row, column) share of the trailing lower triangle, scaling column j on the
// fly; after the step's one barrier the column is stored scaled (the next
// step reads none of it).
__global__ __launch_bounds__(kThreads) void chol_inv(const double *A, int m, float *Rinv) {
  extern __shared__ double L[];  // [m][m]
  const int g = blockIdx.x, tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const double *Ag = A + (int64_t)g * m * m;
  for (int e = tid; e < m * m; e += kThreads) L[e] = Ag[e];
  __syncthreads();
  double dmax = 0.0;
  for (int i = 0; i < m; ++i) dmax = fmax(dmax, L[i * m + i]);
  const double shift = 1e-13 * dmax + 1e-300;
  for (int j = 0; j < m; ++j) {
    const double djj = sqrt(fmax(L[j * m + j] + shift, shift));
    const double inv = 1.0 / djj;
    for (int i = j + 1 + ty; i < m; i += 16) {
      const double lij = L[i * m + j] * inv;
      for (int k = j + 1 + tx; k <= i; k += 16) L[i * m + k] -= lij * (L[k * m + j] * inv);
    }
    __syncthreads();
    for (int i = j + tid; i < m; i += kThreads) L[i * m + j] = i == j ? djj : L[i * m + j] * inv;
  }
  __syncthreads();
  // Linv (lower triangular) goes into the unused upper triangle, transposed:
  // Linv[i][c] (i > c) at [c][i]; thread c forms column c from the rows of L
  // and its own earlier entries, all in LDS.
  float *Rg = Rinv + (int64_t)g * m * m;
  for (int c = tid; c < m; c += kThreads) {
    const double inv_cc = 1.0 / L[c * m + c];
    Rg[(int64_t)c * m + c] = (float)inv_cc;
    const double *Lc = L + c * m;  // this column's Linv entries, at [c][k]
    for (int i = c + 1; i < m; ++i) {
      const double *Li = L + i * m;
      // four independent partial sums: the LDS reads of one step need not
      // wait for the previous step's sum
      double s0 = Li[c] * inv_cc, s1 = 0.0, s2 = 0.0, s3 = 0.0;
      int k = c + 1;
      for (; k + 3 < i; k += 4) {
        s0 += Li[k] * Lc[k];
        s1 += Li[k + 1] * Lc[k + 1];
        s2 += Li[k + 2] * Lc[k + 2];
        s3 += Li[k + 3] * Lc[k + 3];
      }
      for (; k < i; ++k) s0 += Li[k] * Lc[k];
      const double v = -((s0 + s1) + (s2 + s3)) / Li[i];
      L[c * m + i] = v;
      Rg[(int64_t)c * m + i] = (float)v;  // Rinv[c][i] = Linv[i][c]
    }
    for (int i = 0; i < c; ++i) Rg[(int64_t)c * m + i] = 0.f;
  }
}

// Symmetric eigenproblem of one codec's m x m matrix B (fp64, in LDS) by
// cyclic Jacobi rotations; disjoint pairs of a round-robin schedule rotate in
// parallel.  Writes the eigenvectors (columns of U, fp64, global), the
// eigenvalues and the order that sorts them descending.
__global__ __launch_bounds__(kThreads) void jacobi(const double *B, int m, int sweeps, double *U,
                                                   double *evals, int *order) {
  extern __shared__ double S[];  // [m][m], rotations [mp/2][2], sums [2][256], pairs [mp/2][2]
  const int g = blockIdx.x, tid = threadIdx.x;
  const int mp = m + (m & 1);  // players; index m (odd m) sits the round out
  const int npair = mp / 2;
  double *cs = S + m * m;
  double *red = cs + 2 * npair;
  int *pr = reinterpret_cast<int *>(red + 2 * kThreads);
  const double *Bg = B + (int64_t)g * m * m;
  double *Ug = U + (int64_t)g * m * m;
  for (int e = tid; e < m * m; e += kThreads) {
    const int i = e / m, j = e % m;
    S[e] = 0.5 * (Bg[e] + Bg[j * m + i]);  // exact symmetry
    Ug[e] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int rd = 0; rd < mp - 1; ++rd) {
      for (int k = tid; k < npair; k += kThreads) {
        int a = (rd + k) % (mp - 1), b = k == 0 ? mp - 1 : (rd + mp - 1 - k) % (mp - 1);
        double c = 1.0, s = 0.0;
        if (a < m && b < m) {
          const double app = S[a * m + a], aqq = S[b * m + b], apq = S[a * m + b];
          if (fabs(apq) > 1e-300 && fabs(apq) > 1e-18 * (fabs(app) + fabs(aqq))) {
            const double tau = (aqq - app) / (2.0 * apq);
            const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
          }
        } else {
          a = b = -1;
        }
        cs[2 * k] = c;
        cs[2 * k + 1] = s;
        pr[2 * k] = a;
        pr[2 * k + 1] = b;
      }
      __syncthreads();
      for (int e = tid; e < npair * m; e += kThreads) {  // rows: B <- J^T B
        const int k = e / m, j = e % m, a = pr[2 * k], b = pr[2 * k + 1];
        if (a < 0) continue;
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double xa = S[a * m + j], xb = S[b * m + j];
        S[a * m + j] = c * xa - s * xb;
        S[b * m + j] = s * xa + c * xb;
      }
      __syncthreads();
      for (int e = tid; e < npair * m; e += kThreads) {  // columns: B <- B J, U <- U J
        const int k = e / m, i = e % m, a = pr[2 * k], b = pr[2 * k + 1];
        if (a < 0) continue;
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double xa = S[i * m + a], xb = S[i * m + b];
        S[i * m + a] = c * xa - s * xb;
        S[i * m + b] = s * xa + c * xb;
        const double ua = Ug[(int64_t)i * m + a], ub = Ug[(int64_t)i * m + b];
        Ug[(int64_t)i * m + a] = c * ua - s * ub;
        Ug[(int64_t)i * m + b] = s * ua + c * ub;
      }
      __syncthreads();
    }
    // stop once the off-diagonal part is negligible against the diagonal
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < m * m; e += kThreads) {
      const double v = S[e] * S[e];
      if (e / m == e % m) dia += v; else off += v;
    }
    red[tid] = off;
    red[kThreads + tid] = dia;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
      if (tid < h) {
        red[tid] += red[tid + h];
        red[kThreads + tid] += red[kThreads + tid + h];
      }
      __syncthreads();
    }
    const bool done = red[0] <= 1e-24 * red[kThreads];
    __syncthreads();
    if (done) break;
  }
  if (tid == 0) {
    for (int i = 0; i < m; ++i) order[(int64_t)g * m + i] = i;
    for (int i = 0; i < m; ++i) {  // selection sort, descending
      int best = i;
      for (int j = i + 1; j < m; ++j)
        if (S[order[(int64_t)g * m + j] * (m + 1)] > S[order[(int64_t)g * m + best] * (m + 1)])
          best = j;
      const int t = order[(int64_t)g * m + i];
      order[(int64_t)g * m + i] = order[(int64_t)g * m + best];
      order[(int64_t)g * m + best] = t;
    }
    for (int i = 0; i < m; ++i) evals[(int64_t)g * m + i] = S[i * (m + 1)];
  }
}

// Usel[g][k][j] = U[g][k][order[j]], j < r (fp32 for the final GEMM).
__global__ __launch_bounds__(kThreads) void select_vectors(const double *U, const int *order, int m,
                                                           int r, float *Usel) {
  const int g = blockIdx.x;
  for (int e = threadIdx.x; e < m * r; e += kThreads) {
    const int k = e / r, j = e % r;
    Usel[((int64_t)g * m + k) * r + j] = (float)U[((int64_t)g * m + k) * m + order[(int64_t)g * m + j]];
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

  hipLaunchKernelGGL(column_mean<E>, dim3((K + kMeanF - 1) / kMeanF, G), dim3(kThreads), 0, st,
                     x, G, N, K, p.mu);
  LLA_TRY(hipGetLastError());
  // Gram matrix of the centred rows: C = Xc^T Xc  (K x K, contraction over N)
  if (K % 8 == 0 && ((uintptr_t)x & 15u) == 0) {  // whole 16-byte feature vectors
    const int T = (K + kGT - 1) / kGT;
    LLA_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(gram<E>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kGramLds));
    hipLaunchKernelGGL(gram<E>, dim3((unsigned)(T * (T + 1) / 2), G), dim3(kThreads), kGramLds, st,
                       x, p.mu, G, N, K, C);
    LLA_TRY(hipGetLastError());
  } else {
    LLA_TRY(launch_gemm(Centred<E, true>{x, p.mu, G, N, K}, Centred<E, false>{x, p.mu, G, N, K},
                        C, (int64_t)K * K, K, G, K, K, N, st));
  }
  const int64_t qn = (int64_t)G * K * m;
  hipLaunchKernelGGL(start_block, dim3((unsigned)std::min<int64_t>((qn + kThreads - 1) / kThreads, 65536)),
                     dim3(kThreads), 0, st, Q, qn);
  LLA_TRY(hipGetLastError());

  const size_t chol_lds = (size_t)m * m * 8;
  const size_t jac_lds = (size_t)m * m * 8 + (size_t)(m + 1) * 8 + (size_t)2 * kThreads * 8 +
                         (size_t)(m + 1) * 4;
  // both fit the 160 KB a gfx950 workgroup may use (m <= 128)
  LLA_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(chol_inv),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)chol_lds));
  LLA_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(jacobi),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)jac_lds));
  const dim3 sg_grid((m + 15) / 16, (m + 15) / 16, G);
  // C is symmetric: its rows are read as columns (coalesced)
  const MatF32 Ct = mat(C, (int64_t)K * K, 1, K, K, K);
  auto orthonormalise = [&](float *src, float *dst) -> hipError_t {
    // CholeskyQR: dst = src R^-1 with src^T src = R^T R
    hipLaunchKernelGGL(small_gram64, sg_grid, dim3(kThreads), 0, st, src, src, K, m, Sm);
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(chol_inv, dim3(G), dim3(kThreads), chol_lds, st, Sm, m, Rinv);
    if ((e2 = hipGetLastError()) != hipSuccess) return e2;
    return launch_gemm(mat(src, (int64_t)K * m, m, 1, K, m), mat(Rinv, (int64_t)m * m, m, 1, m, m),
                       dst, (int64_t)K * m, m, G, K, m, m, st);
  };
  LLA_TRY(orthonormalise(Q, Y));
  LLA_TRY(orthonormalise(Y, Q));
  for (int it = 0; it < p.iters; ++it) {
    LLA_TRY(launch_gemm(Ct, mat(Q, (int64_t)K * m, m, 1, K, m), Y, (int64_t)K * m, m, G, K, m, K, st));
    LLA_TRY(orthonormalise(Y, Q));   // CholeskyQR2: twice
    LLA_TRY(orthonormalise(Q, Y));
    float *t = Q;  // the orthonormal block is now in Y
    Q = Y;
    Y = t;
  }
  // Rayleigh-Ritz: B = Q^T C Q, B = U diag(lambda) U^T, W = Q U[:, leading r]
  LLA_TRY(launch_gemm(Ct, mat(Q, (int64_t)K * m, m, 1, K, m), Y, (int64_t)K * m, m, G, K, m, K, st));
  hipLaunchKernelGGL(small_gram64, sg_grid, dim3(kThreads), 0, st, Q, Y, K, m, Sm);
  LLA_TRY(hipGetLastError());
  hipLaunchKernelGGL(jacobi, dim3(G), dim3(kThreads), jac_lds, st, Sm, m, p.sweeps, U, ev, order);
  LLA_TRY(hipGetLastError());
  hipLaunchKernelGGL(select_vectors, dim3(G), dim3(kThreads), 0, st, U, order, m, r, Usel);
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
