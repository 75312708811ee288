// Host side of the LLA C ABI: argument validation, sizes, the exact
// compression ratio, the RoPE table, and dispatch to the HIP kernels.
// Every check runs before any launch; nothing here allocates device memory
// or synchronises the device.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>

#include "lla.h"
#include "lla_internal.h"

namespace lla {

RopeLayout rope_layout(int32_t n_ctx, int32_t d_head) {
  RopeLayout L{};
  L.f32_bytes = (size_t)n_ctx * (size_t)d_head * sizeof(float);
  L.bf16_off = (L.f32_bytes + 255) / 256 * 256;
  const size_t tiles = ((size_t)n_ctx + 31) / 32;
  L.bf16_bytes = (d_head % 16 == 0) ? tiles * 32 * (size_t)d_head * 2 : 0;
  L.total = L.bf16_off + L.bf16_bytes;
  return L;
}

}  // namespace lla

namespace {

using lla::DecodeParams;
using lla::EncodeParams;

bool mul_ok(size_t a, size_t b, size_t *out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

size_t elt_size(int32_t dtype) { return dtype == LLA_DT_F32 ? 4 : 2; }

int32_t store_heads(const lla_store_t *s) { return s->variant == LLA_2D ? 1 : s->heads; }

// Element count of the store, or 0 on overflow.
size_t store_elems(const lla_store_t *s) {
  size_t n = 1;
  const size_t dims[5] = {(size_t)s->batch, (size_t)s->layers, (size_t)s->max_ctx,
                          (size_t)store_heads(s), (size_t)s->r_k + (size_t)s->r_v};
  for (size_t v : dims)
    if (!mul_ok(n, v, &n)) return 0;
  return n;
}

// float64 -> bfloat16 bits, round to nearest, ties to even, in one step.
uint16_t f64_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
  int e = 0;
  std::frexp(v, &e);
  if (e < -125) e = -125;
  const double q = std::ldexp(1.0, e - 8);
  const double r = std::nearbyint(v / q) * q;  // default rounding mode: ties to even
  const float f = (float)r;                    // exact: r has at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// Context splits that fill whole rounds of resident workgroups: the S in
// [1, max_s] with the least ceil(per_split * S / slots) / S (the work one
// workgroup slot sees per unit of context), ties going to the fewest splits
// (less setup and merging).  `slots` = workgroups the GPU runs at once.
int32_t fill_rounds(int64_t per_split, int64_t slots, int64_t max_s) {
  int64_t best = 1;
  double best_cost = 1e300;
  for (int64_t S = 1; S <= max_s; ++S) {
    const double cost = (double)((per_split * S + slots - 1) / slots) / (double)S;
    if (cost < best_cost * (1.0 - 1e-9)) {
      best_cost = cost;
      best = S;
    }
  }
  return (int32_t)best;
}

bool mq_path(const lla_store_t *s, int32_t n_q);

int32_t auto_splits(const lla_store_t *s, bool mfma, int32_t n_q = 1) {
  // The fast-path kernels hold one workgroup per CU (the LLA-2D one and the
  // per-head one fill the LDS), the multi-query one two; each split at least
  // 256 slots long.  The generic path: about eight workgroups per CU.
  constexpr int64_t kCUs = 256;
  const bool is2d = s->variant == LLA_2D;
  const int64_t max_s = std::max<int64_t>(1, s->max_ctx / 256);
  if (mfma && is2d) return fill_rounds(s->batch, kCUs, max_s);
  if (mfma && n_q > 1 && mq_path(s, n_q))
    return fill_rounds((int64_t)s->batch * ((s->heads + 3) / 4), 2 * kCUs, max_s);
  if (mfma)
    return fill_rounds((int64_t)s->batch * (s->heads / lla::decode_mfma_group_heads(s->r_k, s->r_v)),
                       kCUs, max_s);
  const int64_t per_split = (int64_t)s->batch * s->heads;
  int64_t S = (2048 + per_split - 1) / per_split;
  if (S > max_s) S = max_s;
  return (int32_t)std::max<int64_t>(1, S);
}

bool use_mfma(const lla_store_t *s) {
  if (s->dtype != LLA_DT_BF16) return false;
  if (s->variant == LLA_2D) return lla::decode2d_mfma_supported(s->heads, s->d_head, s->r_k, s->r_v);
  return lla::decode_mfma_supported(s->heads, s->d_head, s->r_k, s->r_v, store_heads(s));
}

bool mq_path(const lla_store_t *s, int32_t n_q) {
  return s->variant == LLA_PER_HEAD && n_q > 1 &&
         lla::decode_mq_supported(s->d_head, s->r_k, s->r_v, store_heads(s), s->heads, n_q);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kMaxInflight = 32;  // in-flight tokens per call (merge kernel LDS)

// n_q queries per stored sequence; with k_new / v_new (in-flight call) query
// i of sequence b sits at pos[b] + i and the in-flight tokens are merged in.
lla_status_t decode_impl(const lla_store_t *st, int32_t want_variant, int32_t layer,
                         int32_t loop, const float *q, const void *wk, const void *wv,
                         const float *muk, const float *muv, const int32_t *pos,
                         const void *rope, float scale, float *out, void *ws, size_t ws_bytes,
                         int32_t n_splits, hipStream_t stream, int32_t n_q = 1,
                         const float *k_new = nullptr, const float *v_new = nullptr) {
  lla_status_t e = lla_store_check(st);
  if (e != LLA_OK) return e;
  if (st->variant != want_variant) return LLA_E_VARIANT;
  if (!st->data || !q || !wk || !wv || !muk || !muv || !pos || !rope || !out) return LLA_E_NULL;
  const bool inflight = k_new != nullptr || v_new != nullptr;
  if (inflight && (!k_new || !v_new)) return LLA_E_NULL;
  if (n_q < 1) return LLA_E_RANGE;
  if (n_q > kMaxInflight || (!inflight && n_q != 1)) return LLA_E_UNSUPPORTED;
  if (inflight && st->d_head > 256) return LLA_E_UNSUPPORTED;
  // (query, head) row indices are 32-bit in the kernels
  if ((int64_t)st->batch * n_q * st->heads > INT32_MAX) return LLA_E_OVERFLOW;
  if (layer < 0 || layer >= st->layers || loop < 0 || loop >= st->loops) return LLA_E_RANGE;
  if (n_splits < 0 || n_splits > st->max_ctx) return LLA_E_RANGE;
  if (std::isnan(scale) || std::isinf(scale)) return LLA_E_RANGE;
  const bool mfma = use_mfma(st) && aligned16(st->data) && aligned16(wk) && aligned16(wv) &&
                    aligned16(rope);
  if (!mfma) {
    if (st->d_head > 256 || st->r_k > 128 || st->r_v > 256 ||
        (size_t)st->d_head * st->r_k > 8192)
      return LLA_E_UNSUPPORTED;
  } else {
    // 32-bit buffer offsets address one (sequence, layer) slab
    const uint64_t slab = (uint64_t)st->max_ctx * store_heads(st) * (st->r_k + st->r_v) * 2;
    if (slab >= (1ull << 31)) return LLA_E_UNSUPPORTED;
  }
  const int32_t S = n_splits ? n_splits : auto_splits(st, mfma, inflight ? n_q : 1);
  if (inflight) {  // the in-flight merge keeps every query's rows in LDS (160 KB)
    const lla::InflightMergeLds lay = lla::inflight_merge_lds(
        n_q, st->d_head, st->r_v, S, st->dtype == LLA_DT_F32 ? 4 : 2);
    if (lay.base > lla::kInflightMergeLdsMax) return LLA_E_UNSUPPORTED;
  }
  size_t need = lla_decode_workspace_bytes(st, S);
  if (!mul_ok(need, (size_t)n_q, &need)) return LLA_E_OVERFLOW;
  if (!ws) return LLA_E_WORKSPACE;
  if (need == 0 || ws_bytes < need) return LLA_E_WORKSPACE;

  DecodeParams p{};
  p.store = st->data;
  p.B = st->batch * n_q;  // queries
  p.qps = n_q;
  p.inflight = inflight ? 1 : 0;
  p.D = st->layers;
  p.N = st->max_ctx;
  p.H = st->heads;
  p.Hs = store_heads(st);
  p.rk = st->r_k;
  p.rv = st->r_v;
  p.R = st->r_k + st->r_v;
  p.d = st->d_head;
  p.layer = layer;
  p.q = q;
  p.wk = wk;
  p.wv = wv;
  p.muk = muk;
  p.muv = muv;
  p.pos = pos;
  const lla::RopeLayout rl = lla::rope_layout(st->max_ctx, st->d_head);
  p.rope_f32 = reinterpret_cast<const float *>(rope);
  p.rope_bf16 = reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(rope) + rl.bf16_off);
  const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)st->d_head));
  p.scale_log2 = (float)((double)sc * 1.4426950408889634);
  p.ws = reinterpret_cast<float *>(ws);
  p.S = S;
  const int32_t per = (st->max_ctx + S - 1) / S;
  p.split_len = (per + 31) / 32 * 32;
  p.out = out;

  const bool is2d = st->variant == LLA_2D;
  p.write_out = (mfma && !is2d && S == 1 && !inflight) ? 1 : 0;
  const bool mq = mfma && inflight && mq_path(st, n_q);
  hipError_t he = !mfma ? lla::launch_decode_valu(p, st->dtype, stream)
                  : is2d ? lla::launch_decode2d_mfma(p, stream)
                  : mq   ? lla::launch_decode_mq(p, stream)
                         : lla::launch_decode_mfma(p, stream);
  if (he != hipSuccess) return LLA_E_HIP;
  if (p.write_out) return LLA_OK;  // the split kernel applied W_up,v,t itself
  he = inflight ? lla::launch_decode_merge_inflight(p, st->batch, k_new, v_new, st->dtype, stream)
       : is2d   ? lla::launch_decode_merge_batched(p, st->dtype, stream)
                : lla::launch_decode_merge(p, st->dtype, stream);
  return he == hipSuccess ? LLA_OK : LLA_E_HIP;
}

lla_status_t encode_impl(const lla_store_t *st, int32_t want_variant, int32_t layer,
                         const void *xk, const void *xv, const float *muk, const float *muv,
                         const void *wdk, const void *wdv, const int32_t *start, int32_t n_new,
                         hipStream_t stream) {
  lla_status_t e = lla_store_check(st);
  if (e != LLA_OK) return e;
  if (st->variant != want_variant) return LLA_E_VARIANT;
  if (layer < 0 || layer >= st->layers) return LLA_E_RANGE;
  if (n_new < 0 || n_new > st->max_ctx) return LLA_E_RANGE;
  if (n_new == 0) return LLA_OK;
  if (!st->data || !xk || !xv || !muk || !muv || !wdk || !wdv || !start) return LLA_E_NULL;
  if (st->r_k > 128 || st->r_v > 128) return LLA_E_UNSUPPORTED;
  const int64_t width = (int64_t)st->d_head * (st->variant == LLA_2D ? st->heads : 1);
  const int64_t K = width * st->loops;
  if (K > INT32_MAX || (int64_t)st->batch * n_new > INT32_MAX) return LLA_E_OVERFLOW;
  EncodeParams p{};
  p.store = st->data;
  p.B = st->batch;
  p.D = st->layers;
  p.N = st->max_ctx;
  p.Hs = store_heads(st);
  p.rk = st->r_k;
  p.rv = st->r_v;
  p.R = st->r_k + st->r_v;
  p.layer = layer;
  p.K = (int32_t)K;
  p.n_new = n_new;
  p.x[0] = xk;
  p.x[1] = xv;
  p.mu[0] = muk;
  p.mu[1] = muv;
  p.wd[0] = wdk;
  p.wd[1] = wdv;
  p.start = start;
  const hipError_t he = lla::encode_mfma_supported(p, st->dtype)
                            ? lla::launch_encode_mfma(p, stream)
                            : lla::launch_encode_valu(p, st->dtype, stream);
  return he == hipSuccess ? LLA_OK : LLA_E_HIP;
}


// The RoPE table for (N, d, base), layout lla::RopeLayout.
lla_status_t fill_rope_table(int32_t N, int32_t d, float rope_base, void *host_table,
                             size_t bytes) {
  if (!host_table) return LLA_E_NULL;
  const lla::RopeLayout L = lla::rope_layout(N, d);
  if (bytes < L.total) return LLA_E_WORKSPACE;
  const int32_t half = d / 2;
  const double base = (double)rope_base;
  float *f = reinterpret_cast<float *>(host_table);
  for (int32_t j = 0; j < N; ++j)
    for (int32_t i = 0; i < half; ++i) {
      const double ang = (double)j * std::pow(base, -2.0 * i / d);
      f[((size_t)j * half + i) * 2] = (float)std::cos(ang);
      f[((size_t)j * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  std::memset(reinterpret_cast<char *>(host_table) + L.f32_bytes, 0, L.bf16_off - L.f32_bytes);
  if (L.bf16_bytes) {
    uint16_t *h = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(host_table) + L.bf16_off);
    const int32_t ksteps = d / 16, tiles = (N + 31) / 32;
    for (int32_t t = 0; t < tiles; ++t)
      for (int32_t st = 0; st < ksteps; ++st)
        for (int32_t lane = 0; lane < 64; ++lane)
          for (int32_t e8 = 0; e8 < 8; ++e8) {
            const int32_t j = 32 * t + lane % 32;
            const int32_t i = 16 * st + 8 * (lane / 32) + e8;
            const int32_t ii = i < half ? i : i - half;
            const double ang = (double)j * std::pow(base, -2.0 * ii / d);
            const double v = i < half ? std::cos(ang) : std::sin(ang);
            h[(((size_t)t * ksteps + st) * 64 + lane) * 8 + e8] = f64_to_bf16(v);
          }
  }
  return LLA_OK;
}

// ---- uncompressed K/V cache -------------------------------------------------
size_t kv_elems(const lla_kv_cache_t *c) {
  size_t n = 1;
  const size_t dims[7] = {(size_t)c->batch, (size_t)c->layers, (size_t)c->loops,
                          (size_t)c->max_ctx, (size_t)c->heads, 2, (size_t)c->d_head};
  for (size_t v : dims)
    if (!mul_ok(n, v, &n)) return 0;
  return n;
}

int32_t kv_auto_splits(const lla_kv_cache_t *c) {
  // one round of one workgroup per CU, each split at least 128 slots long
  const int32_t hg = lla::kv_heads_per_group(c->d_head, c->dtype);
  const int64_t per_split = (int64_t)c->batch * ((c->heads + hg - 1) / hg);
  return fill_rounds(per_split, 256, std::max<int64_t>(1, c->max_ctx / 128));
}

lla::KvParams kv_params(const lla_kv_cache_t *c, int32_t layer, int32_t cache_loop,
                        const void *rope) {
  lla::KvParams p{};
  p.cache = c->data;
  p.B = c->batch;
  p.D = c->layers;
  p.L = c->loops;
  p.N = c->max_ctx;
  p.H = c->heads;
  p.d = c->d_head;
  p.layer = layer;
  p.cache_loop = cache_loop;
  p.rope_f32 = reinterpret_cast<const float *>(rope);
  return p;
}

// ---- SVD codec initialisation -----------------------------------------------
constexpr int32_t kSvdMaxBlock = 128;   // iterated block m (Jacobi in LDS, Cholesky in registers)
constexpr int32_t kSvdOversample = 16;
constexpr int32_t kSvdDefaultIters = 16;
constexpr int32_t kSvdSweeps = 10;

// The iterated block size m for rank r (0 if r is out of range).
int32_t svd_block(int32_t K, int32_t r) {
  if (r < 1 || r > K || r > kSvdMaxBlock) return 0;
  int32_t m = r + kSvdOversample;
  if (m > kSvdMaxBlock) m = kSvdMaxBlock;
  if (m > K) m = K;
  return m;
}

}  // namespace

extern "C" {

const char *lla_status_string(lla_status_t status) {
  // A C caller may pass any int: read the argument's bytes as an integer
  // rather than reading an enumerator that may be out of the type's range.
  int32_t s;
  static_assert(sizeof(s) == sizeof(status), "lla_status_t is 32-bit");
  std::memcpy(&s, &status, sizeof(s));
  switch (s) {
    case LLA_OK: return "LLA_OK";
    case LLA_E_NULL: return "LLA_E_NULL: a required pointer is NULL";
    case LLA_E_SHAPE: return "LLA_E_SHAPE: invalid or inconsistent sizes";
    case LLA_E_DTYPE: return "LLA_E_DTYPE: unknown element type";
    case LLA_E_RANGE: return "LLA_E_RANGE: index or value out of range";
    case LLA_E_WORKSPACE: return "LLA_E_WORKSPACE: workspace missing or too small";
    case LLA_E_UNSUPPORTED: return "LLA_E_UNSUPPORTED: no kernel for this shape";
    case LLA_E_VARIANT: return "LLA_E_VARIANT: store variant does not match the call";
    case LLA_E_HIP: return "LLA_E_HIP: HIP launch or runtime error";
    case LLA_E_OVERFLOW: return "LLA_E_OVERFLOW: size does not fit";
    case LLA_E_SCRATCH:
      return "LLA_E_SCRATCH: the call needs more than the static scratch "
             "(LLA_NOALLOC_SCRATCH_BYTES) of lla_decode_attn_noalloc";
  }
  return "LLA_E_UNKNOWN";
}

lla_status_t lla_store_check(const lla_store_t *s) {
  if (!s) return LLA_E_NULL;
  if (s->variant != LLA_PER_HEAD && s->variant != LLA_2D) return LLA_E_VARIANT;
  if (s->dtype != LLA_DT_F32 && s->dtype != LLA_DT_BF16) return LLA_E_DTYPE;
  if (s->batch <= 0 || s->layers <= 0 || s->max_ctx <= 0 || s->heads <= 0 || s->d_head <= 0 ||
      s->loops <= 0 || s->r_k <= 0 || s->r_v <= 0)
    return LLA_E_SHAPE;
  if (s->d_head % 2 != 0) return LLA_E_SHAPE;
  if (!(s->rope_base > 1.0f) || std::isinf(s->rope_base)) return LLA_E_RANGE;
  size_t bytes;
  const size_t n = store_elems(s);
  if (n == 0 || !mul_ok(n, elt_size(s->dtype), &bytes) || bytes > (size_t)INT64_MAX)
    return LLA_E_OVERFLOW;
  return LLA_OK;
}

size_t lla_store_bytes(const lla_store_t *s) {
  if (lla_store_check(s) != LLA_OK) return 0;
  return store_elems(s) * elt_size(s->dtype);
}

int64_t lla_store_offset(const lla_store_t *s, int32_t b, int32_t layer, int32_t pos,
                         int32_t head, int32_t comp) {
  if (lla_store_check(s) != LLA_OK) return -1;
  const int32_t Hs = store_heads(s), R = s->r_k + s->r_v;
  if (b < 0 || b >= s->batch || layer < 0 || layer >= s->layers || pos < 0 ||
      pos >= s->max_ctx || head < 0 || head >= Hs || comp < 0 || comp >= R)
    return -1;
  return (((((int64_t)b * s->layers + layer) * s->max_ctx + pos) * Hs + head) * R) + comp;
}

lla_status_t lla_compression_ratio(const lla_store_t *s, int64_t *num, int64_t *den) {
  const lla_status_t e = lla_store_check(s);
  if (e != LLA_OK) return e;
  if (!num || !den) return LLA_E_NULL;
  int64_t n = 2LL * s->loops * s->d_head * (s->variant == LLA_2D ? s->heads : 1);
  int64_t d = (int64_t)s->r_k + s->r_v;
  const int64_t g = std::gcd(n, d);
  *num = n / g;
  *den = d / g;
  return LLA_OK;
}

size_t lla_rope_table_bytes(const lla_store_t *s) {
  if (lla_store_check(s) != LLA_OK) return 0;
  return lla::rope_layout(s->max_ctx, s->d_head).total;
}

lla_status_t lla_rope_table_fill(const lla_store_t *s, void *host_table, size_t bytes) {
  const lla_status_t e = lla_store_check(s);
  if (e != LLA_OK) return e;
  return fill_rope_table(s->max_ctx, s->d_head, s->rope_base, host_table, bytes);
}

lla_status_t lla_encode_append(const lla_store_t *store, int32_t layer, const void *x_k,
                               const void *x_v, const float *mu_k, const float *mu_v,
                               const void *w_down_k, const void *w_down_v,
                               const int32_t *start_pos, int32_t n_new, hipStream_t stream) {
  return encode_impl(store, LLA_PER_HEAD, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v,
                     start_pos, n_new, stream);
}

lla_status_t lla2d_encode_append(const lla_store_t *store, int32_t layer, const void *x_k,
                                 const void *x_v, const float *mu_k, const float *mu_v,
                                 const void *w_down_k, const void *w_down_v,
                                 const int32_t *start_pos, int32_t n_new, hipStream_t stream) {
  return encode_impl(store, LLA_2D, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v, start_pos,
                     n_new, stream);
}

size_t lla_decode_workspace_bytes(const lla_store_t *s, int32_t n_splits) {
  if (lla_store_check(s) != LLA_OK || n_splits < 0) return 0;
  const int32_t S = n_splits ? n_splits : lla_decode_auto_splits(s);
  size_t n = (size_t)s->batch * s->heads;
  if (!mul_ok(n, (size_t)S, &n) || !mul_ok(n, (size_t)s->r_v + 2, &n) || !mul_ok(n, 4, &n))
    return 0;
  return n;
}

int32_t lla_decode_auto_splits(const lla_store_t *s) {
  if (lla_store_check(s) != LLA_OK) return 0;
  return auto_splits(s, use_mfma(s));
}

lla_status_t lla_decode_attn(const lla_store_t *store, int32_t layer, int32_t loop,
                             const float *q, const void *w_up_k_t, const void *w_up_v_t,
                             const float *mu_k_t, const float *mu_v_t, const int32_t *pos,
                             const void *rope_table, float softmax_scale, float *out,
                             void *workspace, size_t ws_bytes, int32_t n_splits,
                             hipStream_t stream) {
  return decode_impl(store, LLA_PER_HEAD, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t,
                     pos, rope_table, softmax_scale, out, workspace, ws_bytes, n_splits, stream);
}

lla_status_t lla2d_decode_attn(const lla_store_t *store, int32_t layer, int32_t loop,
                               const float *q, const void *w_up_k_t, const void *w_up_v_t,
                               const float *mu_k_t, const float *mu_v_t, const int32_t *pos,
                               const void *rope_table, float softmax_scale, float *out,
                               void *workspace, size_t ws_bytes, int32_t n_splits,
                               hipStream_t stream) {
  return decode_impl(store, LLA_2D, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos,
                     rope_table, softmax_scale, out, workspace, ws_bytes, n_splits, stream);
}

size_t lla_decode_inflight_workspace_bytes(const lla_store_t *s, int32_t n_q, int32_t n_splits) {
  if (n_q < 1 || lla_store_check(s) != LLA_OK) return 0;
  size_t n = lla_decode_workspace_bytes(s, n_splits ? n_splits : auto_splits(s, use_mfma(s), n_q));
  if (!mul_ok(n, (size_t)n_q, &n)) return 0;
  return n;
}

lla_status_t lla_decode_attn_inflight(const lla_store_t *store, int32_t layer, int32_t loop,
                                      int32_t n_q, const float *q, const float *k_new,
                                      const float *v_new, const void *w_up_k_t,
                                      const void *w_up_v_t, const float *mu_k_t,
                                      const float *mu_v_t, const int32_t *pos0,
                                      const void *rope_table, float softmax_scale, float *out,
                                      void *workspace, size_t ws_bytes, int32_t n_splits,
                                      hipStream_t stream) {
  if (!k_new || !v_new) return LLA_E_NULL;
  const int32_t variant = store ? store->variant : LLA_PER_HEAD;
  return decode_impl(store, variant, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos0,
                     rope_table, softmax_scale, out, workspace, ws_bytes, n_splits, stream, n_q,
                     k_new, v_new);
}

const char *lla_decode_path(const lla_store_t *s) {
  if (lla_store_check(s) != LLA_OK) return nullptr;
  return use_mfma(s) ? "mfma" : "valu";
}

lla_status_t lla_kv_cache_check(const lla_kv_cache_t *c) {
  if (!c) return LLA_E_NULL;
  if (c->dtype != LLA_DT_F32 && c->dtype != LLA_DT_BF16) return LLA_E_DTYPE;
  if (c->batch <= 0 || c->layers <= 0 || c->loops <= 0 || c->max_ctx <= 0 || c->heads <= 0 ||
      c->d_head <= 0 || c->d_head % 2 != 0)
    return LLA_E_SHAPE;
  if (!(c->rope_base > 1.0f) || std::isinf(c->rope_base)) return LLA_E_RANGE;
  size_t bytes;
  const size_t n = kv_elems(c);
  if (n == 0 || !mul_ok(n, elt_size(c->dtype), &bytes) || bytes > (size_t)INT64_MAX)
    return LLA_E_OVERFLOW;
  return LLA_OK;
}

size_t lla_kv_cache_bytes(const lla_kv_cache_t *c) {
  if (lla_kv_cache_check(c) != LLA_OK) return 0;
  return kv_elems(c) * elt_size(c->dtype);
}

size_t lla_kv_rope_table_bytes(const lla_kv_cache_t *c) {
  if (lla_kv_cache_check(c) != LLA_OK) return 0;
  return lla::rope_layout(c->max_ctx, c->d_head).total;
}

lla_status_t lla_kv_rope_table_fill(const lla_kv_cache_t *c, void *host_table, size_t bytes) {
  const lla_status_t e = lla_kv_cache_check(c);
  if (e != LLA_OK) return e;
  return fill_rope_table(c->max_ctx, c->d_head, c->rope_base, host_table, bytes);
}

lla_status_t lla_kv_fill_from_store(const lla_store_t *st, int32_t layer, const void *w_up_k_t,
                                    const void *w_up_v_t, const float *mu_k_t,
                                    const float *mu_v_t, int32_t slot0, int32_t n_slots,
                                    const void *rope_table, const lla_kv_cache_t *c,
                                    int32_t cache_loop, hipStream_t stream) {
  lla_status_t e = lla_store_check(st);
  if (e != LLA_OK) return e;
  if ((e = lla_kv_cache_check(c)) != LLA_OK) return e;
  if (st->dtype != c->dtype) return LLA_E_DTYPE;
  if (st->batch != c->batch || st->layers != c->layers || st->max_ctx != c->max_ctx ||
      st->heads != c->heads || st->d_head != c->d_head)
    return LLA_E_SHAPE;
  if (layer < 0 || layer >= st->layers || cache_loop < 0 || cache_loop >= c->loops)
    return LLA_E_RANGE;
  if (slot0 < 0 || n_slots < 0 || (int64_t)slot0 + n_slots > st->max_ctx) return LLA_E_RANGE;
  if (n_slots == 0) return LLA_OK;
  if (!st->data || !c->data || !w_up_k_t || !w_up_v_t || !mu_k_t || !mu_v_t || !rope_table)
    return LLA_E_NULL;
  lla::KvParams p = kv_params(c, layer, cache_loop, rope_table);
  p.store = st->data;
  p.Hs = store_heads(st);
  p.rk = st->r_k;
  p.rv = st->r_v;
  p.R = st->r_k + st->r_v;
  p.wk = w_up_k_t;
  p.wv = w_up_v_t;
  p.muk = mu_k_t;
  p.muv = mu_v_t;
  p.slot0 = slot0;
  p.n = n_slots;
  const bool mfma = st->dtype == LLA_DT_BF16 &&
                    lla::kv_fill_mfma_supported(st->d_head, st->r_k, st->r_v) &&
                    aligned16(st->data) && aligned16(c->data) && aligned16(w_up_k_t) &&
                    aligned16(w_up_v_t);
  return lla::launch_kv_fill(p, st->dtype, mfma, stream) == hipSuccess ? LLA_OK : LLA_E_HIP;
}

lla_status_t lla_kv_append(const lla_kv_cache_t *c, int32_t layer, int32_t cache_loop,
                           const float *k, const float *v, const int32_t *start_pos,
                           int32_t n_new, const void *rope_table, hipStream_t stream) {
  const lla_status_t e = lla_kv_cache_check(c);
  if (e != LLA_OK) return e;
  if (layer < 0 || layer >= c->layers || cache_loop < 0 || cache_loop >= c->loops)
    return LLA_E_RANGE;
  if (n_new < 0 || n_new > c->max_ctx) return LLA_E_RANGE;
  if (n_new == 0) return LLA_OK;
  if (!c->data || !k || !v || !start_pos || !rope_table) return LLA_E_NULL;
  lla::KvParams p = kv_params(c, layer, cache_loop, rope_table);
  p.k = k;
  p.v = v;
  p.start = start_pos;
  p.n = n_new;
  return lla::launch_kv_append(p, c->dtype, stream) == hipSuccess ? LLA_OK : LLA_E_HIP;
}

size_t lla_kv_decode_workspace_bytes(const lla_kv_cache_t *c, int32_t n_splits) {
  if (lla_kv_cache_check(c) != LLA_OK || n_splits < 0) return 0;
  if (!lla::kv_decode_supported(c->d_head, c->dtype)) return 0;
  const int32_t S = n_splits ? n_splits : kv_auto_splits(c);
  size_t n = (size_t)c->batch * c->heads;
  if (!mul_ok(n, (size_t)S, &n) || !mul_ok(n, (size_t)c->d_head + 2, &n) || !mul_ok(n, 4, &n))
    return 0;
  return n;
}

int32_t lla_kv_decode_auto_splits(const lla_kv_cache_t *c) {
  if (lla_kv_cache_check(c) != LLA_OK || !lla::kv_decode_supported(c->d_head, c->dtype))
    return 0;
  return kv_auto_splits(c);
}

lla_status_t lla_kv_decode_attn(const lla_kv_cache_t *c, int32_t layer, int32_t cache_loop,
                                const float *q, const int32_t *pos, const void *rope_table,
                                float softmax_scale, float *out, void *workspace,
                                size_t ws_bytes, int32_t n_splits, hipStream_t stream) {
  const lla_status_t e = lla_kv_cache_check(c);
  if (e != LLA_OK) return e;
  if (!c->data || !q || !pos || !rope_table || !out) return LLA_E_NULL;
  if (layer < 0 || layer >= c->layers || cache_loop < 0 || cache_loop >= c->loops)
    return LLA_E_RANGE;
  if (n_splits < 0 || n_splits > c->max_ctx) return LLA_E_RANGE;
  if (std::isnan(softmax_scale) || std::isinf(softmax_scale)) return LLA_E_RANGE;
  if (!lla::kv_decode_supported(c->d_head, c->dtype) || !aligned16(c->data))
    return LLA_E_UNSUPPORTED;
  const int32_t S = n_splits ? n_splits : kv_auto_splits(c);
  const int32_t hg = lla::kv_heads_per_group(c->d_head, c->dtype);
  if ((int64_t)c->batch * ((c->heads + hg - 1) / hg) * S > INT32_MAX) return LLA_E_OVERFLOW;
  if ((int64_t)c->batch * c->heads > INT32_MAX) return LLA_E_OVERFLOW;  // 32-bit (b, h) rows
  const size_t need = lla_kv_decode_workspace_bytes(c, S);
  if (!workspace) return LLA_E_WORKSPACE;
  if (need == 0 || ws_bytes < need) return LLA_E_WORKSPACE;
  lla::KvParams p = kv_params(c, layer, cache_loop, rope_table);
  p.q = q;
  p.pos = pos;
  const float sc =
      softmax_scale > 0.f ? softmax_scale : (float)(1.0 / std::sqrt((double)c->d_head));
  p.scale_log2 = (float)((double)sc * 1.4426950408889634);
  p.ws = reinterpret_cast<float *>(workspace);
  p.S = S;
  p.split_len = (c->max_ctx + S - 1) / S;
  p.out = out;
  return lla::launch_kv_decode(p, c->dtype, stream) == hipSuccess ? LLA_OK : LLA_E_HIP;
}

size_t lla_svd_init_workspace_bytes(int32_t groups, int32_t loops, int32_t width, int32_t r) {
  if (groups < 1 || groups > 65535 || loops < 1 || width < 1) return 0;
  const int64_t K = (int64_t)loops * width;
  if (K > 65536) return 0;
  const int32_t m = svd_block((int32_t)K, r);
  if (m == 0) return 0;
  return lla::svd_layout(groups, (int32_t)K, m, r).total;
}

lla_status_t lla_svd_init(int32_t dtype, int32_t groups, int32_t n_cal, int32_t loops,
                          int32_t width, int32_t r, const void *x, float *mu, void *w_down,
                          void *w_up, float *sigma, int32_t iters, void *workspace,
                          size_t ws_bytes, hipStream_t stream) {
  if (dtype != LLA_DT_F32 && dtype != LLA_DT_BF16) return LLA_E_DTYPE;
  if (groups < 1 || n_cal < 1 || loops < 1 || width < 1) return LLA_E_SHAPE;
  if (groups > 65535) return LLA_E_UNSUPPORTED;
  const int64_t K = (int64_t)loops * width;
  if (K > 65536) return LLA_E_UNSUPPORTED;
  if (r < 1 || r > K) return LLA_E_RANGE;
  if (r > kSvdMaxBlock) return LLA_E_UNSUPPORTED;
  if (iters < 0 || iters > 1000) return LLA_E_RANGE;
  if ((int64_t)n_cal * groups * K > ((int64_t)1 << 40)) return LLA_E_OVERFLOW;
  if (!x || !mu || !w_down || !w_up) return LLA_E_NULL;
  const size_t need = lla_svd_init_workspace_bytes(groups, loops, width, r);
  if (!workspace || need == 0 || ws_bytes < need) return LLA_E_WORKSPACE;
  lla::SvdParams p{};
  p.G = groups;
  p.N = n_cal;
  p.K = (int32_t)K;
  p.T = loops;
  p.width = width;
  p.r = r;
  p.m = svd_block((int32_t)K, r);
  p.iters = iters ? iters : kSvdDefaultIters;
  p.sweeps = kSvdSweeps;
  p.x = x;
  p.mu = mu;
  p.w_down = w_down;
  p.w_up = w_up;
  p.sigma = sigma;
  p.ws = workspace;
  return lla::launch_svd_init(p, dtype, stream) == hipSuccess ? LLA_OK : LLA_E_HIP;
}

}  // extern "C"
