/*
 * lla.h -- C ABI of the Looped Latent Attention (LLA) decode hot path,
 * built for AMD Instinct MI355X (gfx950).
 *
 * Method: "Looped Latent Attention: Cross-Loop KV Compression for Looped
 * Transformers" (arXiv 2607.15456), Section 3.  For every token, layer and
 * head the loop-indexed K (and V) vectors x = [x_1; ...; x_T] (Eq. 1) are
 * stored as one latent c = (x - mu) W_down (Eq. 2).  Decode-time attention
 * at loop t rebuilds x_hat_t = c W_up,t^T + mu_t (Eq. 3) only as it reads a
 * slot, applies RoPE after reconstruction at the slot's position (the
 * rotary phase is shared by all loops; "RoPE and reconstruction"), and
 * attends causally exactly like the uncompressed model.  LLA-2D ("LLA-2D
 * variant") keeps one latent per token and layer that decodes all H heads.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument named "device" is device memory owned by the
 *    caller; the library allocates no device memory, keeps no global
 *    mutable state and may be called from several host threads.  The one
 *    exception is lla_decode_attn_noalloc, which uses a static per-device
 *    scratch array instead of a workspace argument.
 *  - Launching calls are asynchronous on the given stream (0 = the null
 *    stream).  Nothing on the decode / encode path synchronises the host.
 *  - All arguments are validated on the host before any launch; an invalid
 *    call returns a non-zero lla_status_t and launches nothing.  A failed
 *    launch returns LLA_E_HIP.  No C++ exception crosses this boundary.
 *  - Store layout (element type = store->dtype):
 *        store[b][layer][slot][h'][k],  shape [B, D, N, H', r_k + r_v]
 *    row-major, H' = H (per-head) or 1 (LLA-2D).  Components k in [0, r_k)
 *    are the K latent, [r_k, r_k + r_v) the V latent.  Slot j holds the
 *    token at absolute position j.  Offsets are 64-bit (lla_store_offset).
 *  - RoPE: rotate-half pairs (i, i + d/2), theta_i = rope_base^(-2i/d).
 *  - Softmax scale: softmax_scale > 0 is used as given; <= 0 selects
 *    1/sqrt(d_head).
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLA_OK = 0,
  LLA_E_NULL = 1,        /* a required pointer is NULL                       */
  LLA_E_SHAPE = 2,       /* a size is non-positive or sizes are inconsistent */
  LLA_E_DTYPE = 3,       /* unknown element type                             */
  LLA_E_RANGE = 4,       /* layer / loop / n_new / scale out of range        */
  LLA_E_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
  LLA_E_UNSUPPORTED = 6, /* valid request that no kernel here implements    */
  LLA_E_VARIANT = 7,     /* per-head call on an LLA-2D store or vice versa   */
  LLA_E_HIP = 8,         /* a HIP runtime call or kernel launch failed       */
  LLA_E_OVERFLOW = 9,    /* a size does not fit (bytes in size_t / int64, or  */
                         /* batch x queries x heads in int32)                */
  LLA_E_SCRATCH = 10     /* lla_decode_attn_noalloc: the call needs more than */
                         /* LLA_NOALLOC_SCRATCH_BYTES of split partials      */
} lla_status_t;

typedef enum { LLA_DT_F32 = 0, LLA_DT_BF16 = 1 } lla_dtype_t;
typedef enum { LLA_PER_HEAD = 0, LLA_2D = 1 } lla_variant_t;

/* Descriptor of one latent store.  Plain data; the library never keeps it. */
typedef struct {
  int32_t variant;   /* lla_variant_t                                          */
  int32_t dtype;     /* lla_dtype_t of the store and of x, W_down, W_up        */
  int32_t batch;     /* B sequences                                            */
  int32_t layers;    /* D layers                                               */
  int32_t max_ctx;   /* N slots per (sequence, layer)                          */
  int32_t heads;     /* H attention heads (queries and K/V heads alike)        */
  int32_t d_head;    /* d, even                                                */
  int32_t loops;     /* T recurrence steps                                     */
  int32_t r_k;       /* K latent rank                                          */
  int32_t r_v;       /* V latent rank                                          */
  float rope_base;   /* RoPE base, e.g. 10000                                  */
  void *data;        /* device: the store, lla_store_bytes() bytes, caller-owned */
} lla_store_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *lla_status_string(lla_status_t status);

/* Checks a descriptor's fields (not its data pointer).  LLA_OK or the
 * first error found. */
lla_status_t lla_store_check(const lla_store_t *store);

/* Bytes of the latent store: B*D*N*H'*(r_k+r_v)*sizeof(dtype).
 * Returns 0 for an invalid descriptor or when the count overflows. */
size_t lla_store_bytes(const lla_store_t *store);

/* Element offset of store[b][layer][pos][head][comp] (64-bit).  head is
 * the stored head (must be 0 for LLA-2D).  Returns -1 when any index is
 * out of range or the descriptor is invalid.  Host-only, no device access. */
int64_t lla_store_offset(const lla_store_t *store, int32_t b, int32_t layer,
                         int32_t pos, int32_t head, int32_t comp);

/* Exact compression ratio of the store as a reduced fraction num/den
 * (paper Sec. 3 Eq. 4): per-head 2*T*d/(r_k+r_v); LLA-2D 2*T*H*d/(r_k+r_v). */
lla_status_t lla_compression_ratio(const lla_store_t *store, int64_t *num,
                                   int64_t *den);

/* Size of the RoPE table the decode calls read, for store's (N, d, base). */
size_t lla_rope_table_bytes(const lla_store_t *store);

/* Fills a HOST buffer of lla_rope_table_bytes() bytes with the RoPE table
 * (computed in double precision, rounded once); the caller copies it to
 * device memory and passes that copy to the decode calls.  The contents are
 * opaque: cos/sin of pos*theta_i for every slot, in the element orders the
 * decode kernels read.  Error if bytes is smaller than required. */
lla_status_t lla_rope_table_fill(const lla_store_t *store, void *host_table,
                                 size_t bytes);

/* ---------------------------------------------------------------------------
 * Append-time encoder (paper Sec. 3 Eq. 2): for every new token
 *     c = (x - mu) W_down
 * for the K and V axes separately, rounded to the store type (nearest,
 * ties even) and written to store[b][layer][start_pos[b] + j][h][...].
 * Call it once a token has finished all T loops (Eq. 2 needs the whole
 * T-loop stack).  n_new == 0 is a no-op.
 *
 * Per-head (lla_encode_append):
 *   x_k, x_v     device, store dtype, [B, n_new, H, T*d]  (x_1..x_T stacked, Eq. 1)
 *   mu_k, mu_v   device, float32,     [H, T*d]
 *   w_down_k     device, store dtype, [H, T*d, r_k]
 *   w_down_v     device, store dtype, [H, T*d, r_v]
 * LLA-2D (lla2d_encode_append): H' = 1 and the stack is [t][h][d]:
 *   x_k, x_v     [B, n_new, T*H*d];  mu_* [T*H*d];  w_down_* [T*H*d, r]
 *   start_pos    device, int32, [B]; slots outside [0, N) are not written.
 * ------------------------------------------------------------------------- */
lla_status_t lla_encode_append(const lla_store_t *store, int32_t layer,
                               const void *x_k, const void *x_v,
                               const float *mu_k, const float *mu_v,
                               const void *w_down_k, const void *w_down_v,
                               const int32_t *start_pos, int32_t n_new,
                               hipStream_t stream);
lla_status_t lla2d_encode_append(const lla_store_t *store, int32_t layer,
                                 const void *x_k, const void *x_v,
                                 const float *mu_k, const float *mu_v,
                                 const void *w_down_k, const void *w_down_v,
                                 const int32_t *start_pos, int32_t n_new,
                                 hipStream_t stream);

/* Workspace bytes a decode call needs for n_splits context splits
 * (0 = the automatic choice lla_decode_attn would make). */
size_t lla_decode_workspace_bytes(const lla_store_t *store, int32_t n_splits);

/* The split count lla_decode_attn uses when n_splits == 0. */
int32_t lla_decode_auto_splits(const lla_store_t *store);

/* ---------------------------------------------------------------------------
 * Decode-time attention at (layer, loop t) over the latent store
 * (paper Sec. 3 Eq. 3, "RoPE and reconstruction"): for every sequence b
 * and head h, the query at position pos[b] attends slots 0..pos[b]:
 *   k_j = RoPE(c_k,j W_up,k,t^T + mu_k,t, j),  v_j = c_v,j W_up,v,t^T + mu_v,t
 *   out[b][h] = sum_j softmax_j(scale * RoPE(q[b][h], pos[b]) . k_j) v_j
 * The current token's own K/V must already be in the store (slot pos[b]).
 *
 * Per-head (lla_decode_attn):
 *   q            device, float32, [B, H, d], before RoPE
 *   w_up_k_t     device, store dtype, [H, d, r_k]   (W_up,k,t of every head)
 *   w_up_v_t     device, store dtype, [H, d, r_v]
 *   mu_k_t       device, float32, [H, d]  (loop-t slice of mu_k)
 *   mu_v_t       device, float32, [H, d]
 * LLA-2D (lla2d_decode_attn): w_up_*_t [H*d, r] with rows [h][d];
 *   mu_*_t [H*d].
 *   pos          device, int32, [B]; values are clamped into [0, N-1].
 *   rope_table   device copy of lla_rope_table_fill()'s output.
 *   out          device, float32, [B, H, d].
 *   workspace    device, >= lla_decode_workspace_bytes(store, n_splits).
 *   loop         0 <= loop < T.  Validated; the RoPE phase does not depend
 *                on it -- W_up,t and mu_t carry the loop.
 * ------------------------------------------------------------------------- */
lla_status_t lla_decode_attn(const lla_store_t *store, int32_t layer,
                             int32_t loop, const float *q,
                             const void *w_up_k_t, const void *w_up_v_t,
                             const float *mu_k_t, const float *mu_v_t,
                             const int32_t *pos, const void *rope_table,
                             float softmax_scale, float *out, void *workspace,
                             size_t ws_bytes, int32_t n_splits,
                             hipStream_t stream);
lla_status_t lla2d_decode_attn(const lla_store_t *store, int32_t layer,
                               int32_t loop, const float *q,
                               const void *w_up_k_t, const void *w_up_v_t,
                               const float *mu_k_t, const float *mu_v_t,
                               const int32_t *pos, const void *rope_table,
                               float softmax_scale, float *out,
                               void *workspace, size_t ws_bytes,
                               int32_t n_splits, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Multi-query causal decode with the exact in-flight self-term.  In a looped
 * model the tokens of the current step run their T loops before their
 * latents can be encoded (Eq. 2 of the paper's Sec. 3 needs the whole T-loop
 * stack), so at loop t they must attend to their own fresh loop-t keys and
 * values in full precision.  For each sequence b the call handles n_q
 * consecutive new tokens at positions pos0[b] .. pos0[b] + n_q - 1; query i
 * attends
 *   - the store slots 0 .. pos0[b] - 1 (reconstructed exactly as in
 *     lla_decode_attn / lla2d_decode_attn, RoPE at each slot's position), and
 *   - the in-flight tokens m = 0 .. i (causal), key RoPE(k_new[b][m], pos0[b] + m),
 *     value v_new[b][m],
 * with the query rotated at pos0[b] + i.  Works on per-head and LLA-2D stores
 * (the store's variant selects the reconstruction).
 *   n_q          1 .. 32
 *   q, k_new, v_new  device, float32, [B, n_q, H, d] (pre-RoPE)
 *   pos0         device, int32, [B]; clamped into [0, N]; positions past N-1
 *                use the rotary phase of N-1
 *   out          device, float32, [B, n_q, H, d]
 *   workspace    >= lla_decode_inflight_workspace_bytes(store, n_q, n_splits)
 *   other arguments as lla_decode_attn.
 * ------------------------------------------------------------------------- */
size_t lla_decode_inflight_workspace_bytes(const lla_store_t *store, int32_t n_q,
                                           int32_t n_splits);
lla_status_t lla_decode_attn_inflight(const lla_store_t *store, int32_t layer, int32_t loop,
                                      int32_t n_q, const float *q, const float *k_new,
                                      const float *v_new, const void *w_up_k_t,
                                      const void *w_up_v_t, const float *mu_k_t,
                                      const float *mu_v_t, const int32_t *pos0,
                                      const void *rope_table, float softmax_scale, float *out,
                                      void *workspace, size_t ws_bytes, int32_t n_splits,
                                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * lla_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * lla_decode_attn, minus workspace / ws_bytes: the split partials go to a
 * static device array of LLA_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  The call allocates nothing
 * and calls no allocating routine.
 *  - The scratch belongs to the current device (hipGetDevice), which must be
 *    the device of `stream`; its address is looked up once per device, on
 *    that device's first call.
 *  - A call whose partials need more than LLA_NOALLOC_SCRATCH_BYTES
 *    (lla_decode_workspace_bytes(store, n_splits) with this call's split
 *    count) returns LLA_E_SCRATCH and launches nothing.
 *  - Every call on one GPU shares that GPU's scratch: calls that may overlap
 *    on one GPU (different streams, different host threads without ordering)
 *    race and must be serialised by the caller.  The kernels write every
 *    partial they read, so nothing in the scratch has to start at zero.
 * ------------------------------------------------------------------------- */
#define LLA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
lla_status_t lla_decode_attn_noalloc(const lla_store_t *store, int32_t layer, int32_t loop,
                                     const float *q, const void *w_up_k_t, const void *w_up_v_t,
                                     const float *mu_k_t, const float *mu_v_t,
                                     const int32_t *pos, const void *rope_table,
                                     float softmax_scale, float *out, int32_t n_splits,
                                     hipStream_t stream);

/* Name of the kernel family lla_decode_attn / lla2d_decode_attn would
 * launch for this store ("mfma" fast path or "valu" generic path), or NULL
 * for an invalid descriptor.  Host-only. */
const char *lla_decode_path(const lla_store_t *store);

/* ===========================================================================
 * Uncompressed K/V cache: the two comparison paths the paper sets against
 * the latent store.
 *  - The serving "fast path" (technical summary, "Serving Capacity"):
 *    reconstruct every loop's K/V from the latents once, cache them in full
 *    and decode with plain flash attention.  It keeps the reconstruction off
 *    the decode path but gives up the memory saving (cache loops L = T).
 *  - The final-loop-reuse control (paper Sec. 3, matched-axis baselines):
 *    cache only the last loop's K/V (L = 1) and let every loop's query
 *    attend to it; at T = 4 its footprint equals that of a 4x latent store.
 *
 * Cache layout (element type = cache->dtype):
 *     cache[b][layer][l][slot][h][0 = K | 1 = V][i],  shape [B, D, L, N, H, 2, d]
 * row-major.  Keys are stored after RoPE at their slot's position (the
 * same rotate-half convention as the latent path); values as they are.
 * The RoPE table of lla_kv_rope_table_fill() (or that of a latent store
 * with the same max_ctx, d_head and rope_base) serves every call.
 * ========================================================================= */
typedef struct {
  int32_t dtype;     /* lla_dtype_t of K and V                               */
  int32_t batch;     /* B sequences                                          */
  int32_t layers;    /* D layers                                             */
  int32_t loops;     /* L cached loops per layer (T: fast path; 1: control)  */
  int32_t max_ctx;   /* N slots                                              */
  int32_t heads;     /* H                                                    */
  int32_t d_head;    /* d, even                                              */
  float rope_base;   /* RoPE base                                            */
  void *data;        /* device: lla_kv_cache_bytes() bytes, caller-owned     */
} lla_kv_cache_t;

/* LLA_OK or the first error found in the descriptor (not its data). */
lla_status_t lla_kv_cache_check(const lla_kv_cache_t *cache);

/* B*D*L*N*H*2*d*sizeof(dtype); 0 for an invalid descriptor or on overflow. */
size_t lla_kv_cache_bytes(const lla_kv_cache_t *cache);

/* RoPE table for the cache's (N, d, base); same contract as
 * lla_rope_table_bytes / lla_rope_table_fill. */
size_t lla_kv_rope_table_bytes(const lla_kv_cache_t *cache);
lla_status_t lla_kv_rope_table_fill(const lla_kv_cache_t *cache, void *host_table, size_t bytes);

/* Reconstruct-to-cache (the fast path's fill): for every sequence b, head h
 * and slot j in [slot0, slot0 + n_slots) with j < N,
 *   cache[b][layer][cache_loop][j][h][K] = RoPE(c_k,j W_up,k,t^T + mu_k,t, j)
 *   cache[b][layer][cache_loop][j][h][V] = c_v,j W_up,v,t^T + mu_v,t
 * (paper Sec. 3 Eq. 3, "RoPE and reconstruction"), rounded once to the
 * cache type.  c is read from store[b][layer][j] (per-head: head h's latent;
 * LLA-2D: the token's one latent).  w_up_*_t and mu_*_t are laid out exactly
 * as for lla_decode_attn (per-head [H, d, r]; LLA-2D [H*d, r] -- the same
 * memory order).  The store and the cache must agree on dtype, batch, layers,
 * max_ctx, heads and d_head; 0 <= cache_loop < cache->loops.  n_slots == 0
 * is a no-op.  The caller names the loop t only through w_up_*_t and mu_*_t.
 * ------------------------------------------------------------------------- */
lla_status_t lla_kv_fill_from_store(const lla_store_t *store, int32_t layer,
                                    const void *w_up_k_t, const void *w_up_v_t,
                                    const float *mu_k_t, const float *mu_v_t,
                                    int32_t slot0, int32_t n_slots, const void *rope_table,
                                    const lla_kv_cache_t *cache, int32_t cache_loop,
                                    hipStream_t stream);

/* Append raw K/V (e.g. the final loop's, for the control): for j < n_new,
 *   cache[b][layer][cache_loop][start_pos[b] + j][h] = (RoPE(k[b][j][h], that slot), v[b][j][h])
 * rounded to the cache type; slots outside [0, N) are not written.
 *   k, v        device, float32, [B, n_new, H, d] (pre-RoPE)
 *   start_pos   device, int32, [B] */
lla_status_t lla_kv_append(const lla_kv_cache_t *cache, int32_t layer, int32_t cache_loop,
                           const float *k, const float *v, const int32_t *start_pos,
                           int32_t n_new, const void *rope_table, hipStream_t stream);

/* Flash-decode over the cache: for every sequence b and head h,
 *   out[b][h] = sum_{j <= pos[b]} softmax_j(scale * RoPE(q[b][h], pos[b]) . K_j) V_j
 * with K_j, V_j = cache[b][layer][cache_loop][j][h].  The fast path calls it
 * with cache_loop = t (the loop of q); the final-loop control with 0 for
 * every loop.  q [B, H, d] fp32 pre-RoPE; pos [B] clamped into [0, N-1];
 * out [B, H, d] fp32; softmax_scale as lla_decode_attn; workspace >=
 * lla_kv_decode_workspace_bytes(cache, n_splits) (n_splits 0 = automatic). */
size_t lla_kv_decode_workspace_bytes(const lla_kv_cache_t *cache, int32_t n_splits);
int32_t lla_kv_decode_auto_splits(const lla_kv_cache_t *cache);
lla_status_t lla_kv_decode_attn(const lla_kv_cache_t *cache, int32_t layer, int32_t cache_loop,
                                const float *q, const int32_t *pos, const void *rope_table,
                                float softmax_scale, float *out, void *workspace,
                                size_t ws_bytes, int32_t n_splits, hipStream_t stream);

/* ===========================================================================
 * SVD codec initialisation (paper Sec. 3, initialisation and conversion): for
 * each of G independent codecs (one per layer, head and axis), from n_cal
 * calibration rows of its stacked loop vector x = [x_1; ...; x_T] (Eq. 1):
 *   mu      = the mean row (the per-loop means, stacked)
 *   W_down  = the r leading right singular vectors of the centred matrix
 *             X - 1 mu^T (orthonormal columns, by decreasing singular value;
 *             each column's entry of largest magnitude is positive)
 *   W_up,t  = rows [t*width, (t+1)*width) of W_down, the loop-t slice.
 * Computed on the GPU: the Gram matrix of the centred rows, block subspace
 * iteration (r plus up to 16 extra vectors, CholeskyQR2 in fp64) and a
 * Rayleigh-Ritz step solved by cyclic Jacobi rotations in fp64.
 *   dtype      type of x, w_down and w_up (lla_dtype_t)
 *   groups     G, 1 .. 65535;  loops T, width (d per-head, H*d for LLA-2D)
 *   r          1 .. min(T*width, 128)
 *   x          device, [n_cal, G, T*width] (token-major, as the encoders take it)
 *   mu         device, float32, [G, T*width]
 *   w_down     device, [G, T*width, r]      (the encoders' W_down layout)
 *   w_up       device, [T, G, width, r]     (for loop t, the decode calls' W_up,t)
 *   sigma      device, float32, [G, r] singular values, or NULL
 *   iters      subspace iterations (0 = 16)
 *   workspace  device, >= lla_svd_init_workspace_bytes(); the call is
 *              asynchronous on the stream like every other launching call.
 * ------------------------------------------------------------------------- */
size_t lla_svd_init_workspace_bytes(int32_t groups, int32_t loops, int32_t width, int32_t r);
lla_status_t lla_svd_init(int32_t dtype, int32_t groups, int32_t n_cal, int32_t loops,
                          int32_t width, int32_t r, const void *x, float *mu, void *w_down,
                          void *w_up, float *sigma, int32_t iters, void *workspace,
                          size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
