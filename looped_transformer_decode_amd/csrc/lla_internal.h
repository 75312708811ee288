// Internal declarations shared by the host API (lla_api.cpp) and the HIP
// kernel files.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "lla.h"

namespace lla {

// Byte layout of the opaque RoPE table produced by lla_rope_table_fill():
//   [0, f32_bytes)            float32 cos/sin, [N][d/2][2]
//   [bf16_off, +bf16_bytes)   bfloat16 phi operand tiles for the MFMA decode:
//                             per 32-slot tile, [d/16 k-steps][64 lanes][8],
//                             element (s, lane, e) = phi[32*tile + lane%32][i],
//                             i = 16*s + 8*(lane/32) + e, with
//                             phi[j][i] = cos(j*theta_i) for i < d/2 and
//                             sin(j*theta_{i-d/2}) otherwise.
struct RopeLayout {
  size_t f32_bytes;
  size_t bf16_off;
  size_t bf16_bytes;
  size_t total;
};
RopeLayout rope_layout(int32_t n_ctx, int32_t d_head);

// Arguments of one decode call, resolved and validated on the host.
struct DecodeParams {
  const void *store;       // base of the whole store
  int32_t B, D, N, H, Hs;  // Hs = stored heads (H or 1)
  int32_t R, rk, rv, d;    // R = rk + rv
  int32_t layer;
  const float *q;          // [B, H, d]
  const void *wk;          // [H*d, rk]  (per-head [H, d, rk] is the same memory)
  const void *wv;          // [H*d, rv]
  const float *muk;        // [H*d]
  const float *muv;        // [H*d]
  const int32_t *pos;      // [B]
  const float *rope_f32;   // [N][d/2][2]
  const uint16_t *rope_bf16;
  float scale_log2;        // softmax scale * log2(e)
  float *ws;               // partials [B, H, S, rv + 2]
  int32_t S;               // context splits
  int32_t split_len;       // slots per split (multiple of 32)
  float *out;              // [B, H, d]
  // Multi-query / in-flight calls: the B above counts queries (virtual
  // sequences); query vb reads store sequence vb / qps.  With inflight set,
  // query i = vb % qps of sequence b sits at position pos[b] + i and attends
  // store slots < pos[b] only (its own loop-t keys are still in flight).
  int32_t qps;
  int32_t inflight;
  int32_t write_out;       // the split kernel applies W_up,v,t itself (one split)
  int32_t w_lds;           // merge kernels: W_up,v,t of the head staged in LDS
};

// Which store sequence a (virtual) query reads, its rotary position, and the
// last store slot it attends (-1: none).
struct QuerySlot {
  int32_t b, qpos, last;
};
__device__ __forceinline__ QuerySlot query_slot(const DecodeParams &p, int32_t vb) {
  const int32_t b = vb / p.qps;
  const int32_t base = p.pos[b];
  if (p.inflight) {
    const int32_t first = min(max(base, 0), p.N);
    return {b, min(first + (vb - b * p.qps), p.N - 1), first - 1};
  }
  const int32_t q = min(max(base, 0), p.N - 1);
  return {b, q, q};
}

// LDS of the in-flight merge (floats unless noted): rotated keys [nq][d];
// rotated queries [nq][d], which the store numerators [rv][nq_pad] (query
// count padded to whole groups of 8) replace once the scores are formed;
// in-flight scores [nq][nq], per-query store M, L and softmax factors
// [nq][4], split weights [nq][S];
// then, 16-byte aligned, W_up,v,t of the head as [d] rows of w_pitch dwords
// (an odd count, so that consecutive rows start in different banks).
// base: bytes without the W rows; with_w: bytes with them.
struct InflightMergeLds {
  int32_t qa_floats;  // floats of the query / numerator region
  int32_t nq_pad;
  int32_t w_off;    // floats before the W rows
  int32_t w_pitch;  // dwords per W row
  size_t base, with_w;
};
constexpr size_t kInflightMergeLdsMax = 160 * 1024;
__host__ __device__ inline InflightMergeLds inflight_merge_lds(int32_t nq, int32_t d, int32_t rv,
                                                               int32_t S, int32_t esize) {
  InflightMergeLds l;
  l.nq_pad = (nq + 7) / 8 * 8;
  const size_t qa = (size_t)nq * d > (size_t)l.nq_pad * rv ? (size_t)nq * d : (size_t)l.nq_pad * rv;
  const size_t f = (size_t)nq * d + qa + (size_t)nq * nq + 4 * (size_t)nq + (size_t)nq * S;
  l.qa_floats = (int32_t)qa;
  l.base = 4 * f;
  l.w_off = (int32_t)((f + 3) / 4 * 4);
  l.w_pitch = ((rv * esize + 3) / 4) | 1;
  l.with_w = 4 * ((size_t)l.w_off + (size_t)d * l.w_pitch);
  return l;
}

// LDS of the LLA-2D merge (floats unless noted): merged averages [8][rv],
// split weights [8][S], merged sums [8]; then, 16-byte aligned, W_up,v,t of
// the head as [d] rows of w_pitch dwords (odd).  base: bytes without the W
// rows; with_w: bytes with them (used up to kBatchedMergeWLdsMax).
struct BatchedMergeLds {
  int32_t w_off;    // floats before the W rows
  int32_t w_pitch;  // dwords per W row
  size_t base, with_w;
};
constexpr size_t kBatchedMergeWLdsMax = 64 * 1024;
__host__ __device__ inline BatchedMergeLds batched_merge_lds(int32_t d, int32_t rv, int32_t S,
                                                             int32_t esize) {
  BatchedMergeLds l;
  const size_t f = (size_t)8 * rv + (size_t)8 * S + 8;
  l.base = 4 * f;
  l.w_off = (int32_t)((f + 3) / 4 * 4);
  l.w_pitch = ((rv * esize + 3) / 4) | 1;
  l.with_w = 4 * ((size_t)l.w_off + (size_t)d * l.w_pitch);
  return l;
}

struct EncodeParams {
  void *store;
  int32_t B, D, N, Hs, R, rk, rv;
  int32_t layer;
  int32_t K;               // T * width: length of the stacked vector
  int32_t n_new;
  const void *x[2];        // [B, n_new, Hs, K] per axis
  const float *mu[2];      // [Hs, K]
  const void *wd[2];       // [Hs, K, r]
  const int32_t *start;    // [B]
};

// Heads one merge block covers: one thread per output element of 256, and
// the merged latent averages of those heads (hpb * rv floats) within 32 KB.
__host__ __device__ inline int32_t merge_heads_per_block(int32_t d, int32_t rv) {
  int32_t h = d >= 256 ? 1 : 256 / d;
  const int32_t cap = 8192 / rv;
  if (h > cap) h = cap;
  return h < 1 ? 1 : h;
}

// Uncompressed K/V cache [B, D, L, N, H, 2, d]: geometry and one call's
// arguments (decode, reconstruct-to-cache or raw append).
struct KvParams {
  void *cache;
  int32_t B, D, L, N, H, d;
  int32_t layer, cache_loop;
  const float *rope_f32;   // [N][d/2][2]
  // decode
  const float *q;          // [B, H, d]
  const int32_t *pos;      // [B]
  float scale_log2;
  float *ws;               // partials [B, H, S, d + 2]
  int32_t S, split_len;
  float *out;              // [B, H, d]
  // reconstruct-to-cache: slots [slot0, slot0 + n) of the latent store
  const void *store;
  int32_t Hs, rk, rv, R;
  const void *wk, *wv;     // [H*d, rk], [H*d, rv]
  const float *muk, *muv;  // [H*d]
  int32_t slot0, n;
  // raw append
  const float *k, *v;      // [B, n, H, d]
  const int32_t *start;    // [B]
};

// SVD codec initialisation: G codecs, N calibration rows of K = T * width.
struct SvdParams {
  int32_t G, N, K, T, width, r, m;  // m = r + oversampling: the iterated block
  int32_t iters, sweeps;
  const void *x;        // [N, G, K]
  float *mu;            // [G, K]
  void *w_down;         // [G, K, r]
  void *w_up;           // [T, G, width, r]
  float *sigma;         // [G, r] or null
  void *ws;
};
// Byte offsets of the SVD workspace regions.
struct SvdLayout {
  size_t gram, q, y, small, rinv, u, evals, order, usel, w, total;
};
SvdLayout svd_layout(int32_t G, int32_t K, int32_t m, int32_t r);
hipError_t launch_svd_init(const SvdParams &p, int dtype, hipStream_t s);

// Launchers (return the launch status).  dtype is lla_dtype_t.
hipError_t launch_decode_valu(const DecodeParams &p, int dtype, hipStream_t s);
hipError_t launch_decode_merge(const DecodeParams &p, int dtype, hipStream_t s);
hipError_t launch_decode_merge_batched(const DecodeParams &p, int dtype, hipStream_t s);
// In-flight merge: store partials of every query + the exact causal term of
// the n_q in-flight tokens (k_new, v_new: [B, n_q, H, d] fp32).  B_real is
// the number of stored sequences.
hipError_t launch_decode_merge_inflight(const DecodeParams &p, int32_t B_real, const float *k_new,
                                        const float *v_new, int dtype, hipStream_t s);
bool decode2d_mfma_supported(int32_t H, int32_t d, int32_t rk, int32_t rv);
hipError_t launch_decode2d_mfma(const DecodeParams &p, hipStream_t s);
bool decode_mfma_supported(int32_t H, int32_t d, int32_t rk, int32_t rv, int32_t Hs);
// Heads one fast-path workgroup covers (0 if the ranks have no instance).
int32_t decode_mfma_group_heads(int32_t rk, int32_t rv);
hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t s);
// Multi-query store pass (reconstruct first): all n_q <= 16 queries of a
// sequence per workgroup; writes the same partials as launch_decode_mfma.
bool decode_mq_supported(int32_t d, int32_t rk, int32_t rv, int32_t Hs, int32_t H, int32_t n_q);
hipError_t launch_decode_mq(const DecodeParams &p, hipStream_t s);
hipError_t launch_encode_valu(const EncodeParams &p, int dtype, hipStream_t s);
bool encode_mfma_supported(const EncodeParams &p, int dtype);
hipError_t launch_encode_mfma(const EncodeParams &p, hipStream_t s);
bool encode_stream_supported(const EncodeParams &p);
hipError_t launch_encode_stream(const EncodeParams &p, hipStream_t s);
bool kv_decode_supported(int32_t d, int dtype);
int32_t kv_heads_per_group(int32_t d, int dtype);
hipError_t launch_kv_decode(const KvParams &p, int dtype, hipStream_t s);
bool kv_fill_mfma_supported(int32_t d, int32_t rk, int32_t rv);
hipError_t launch_kv_fill(const KvParams &p, int dtype, bool mfma, hipStream_t s);
hipError_t launch_kv_append(const KvParams &p, int dtype, hipStream_t s);

}  // namespace lla
