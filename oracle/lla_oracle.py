"""Plain fp64 CPU oracle for Looped Latent Attention (LLA) decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (``looped_transformer_decode_amd``) never imports, links or executes it,
and this module imports nothing from the product path.  The two share no code:
only the seeded input generators in ``synth/`` feed both.

Sources (cited by section / equation, never by line):
  [paper]  "Looped Latent Attention: Cross-Loop KV Compression for Looped
           Transformers" (arXiv 2607.15456, HTML version).  Section 3 defines
           the teacher cache (Eq. 1), the cross-loop codec (Eqs. 2-3), the
           compression ratio (Eq. 4), "RoPE and reconstruction", the LLA-2D
           variant, and the SVD-initialisation convention.
  [summary] gist.science technical summary of the same paper ("Core
           Mechanism", "Key Contributions", "Serving Capacity").

What the oracle computes, in the paper's notation:
  x = [x_1; ...; x_T] in R^{T d}       one token / layer / head / axis (Eq. 1)
  c = (x - mu) W_down                  the stored latent (Eq. 2)
  x_hat_t = c W_up,t^T + mu_t          loop-t reconstruction (Eq. 3)
  rho = 2 T d / (r_k + r_v)            compression ratio (Eq. 4)
  RoPE is applied to the reconstructed key at the token's own position,
  with a phase that does not depend on the loop ("RoPE and reconstruction").
  Attention itself is ordinary causal softmax attention (Section 3 intro:
  only what the cache stores changes).

Readings where the pages are silent (each is a named choice, mirrored by the kernels):
  * RoPE pairing is rotate-half, pairs (i, i + d/2), theta_i = base^(-2i/d),
    applied over the full head width.  Parity unpinned by the pages: the
    pages name RoPE but print no convention.
  * The query arrives before RoPE and is rotated at its own position pos.
  * Softmax scale defaults to 1/sqrt(d_head).
  * A query at position pos attends store slots 0..pos; slot j holds the
    token at absolute position j.
  * LLA-2D stacks the loop/head axes as [t][h][d]; W_up,t rows are [h][d].
  * mu_t is the loop-t slice of mu (the same calibration mean Eq. 2 subtracts).

Everything here is float64 numpy; inputs given as bf16 / fp32 values are
taken at their exact value.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

ROPE_BASE = 10000.0


# --------------------------------------------------------------------------
# Sizes: Eq. (4) and the cache-size statements of Section 3
# --------------------------------------------------------------------------
def compression_ratio(T: int, d_head: int, r_k: int, r_v: int,
                      heads: int = 1, variant: str = "per_head") -> Fraction:
    """Exact compression ratio.

    Per-head LLA, [paper] Sec. 3 Eq. (4): the uncompressed cache holds
    2*T*H*d scalars per token and layer, the latent store (r_k + r_v)*H,
    so rho = 2*T*d / (r_k + r_v).  LLA-2D ([paper] Sec. 3, LLA-2D variant)
    keeps one latent of r_k + r_v scalars per token and layer for all H
    heads, so rho = 2*T*H*d / (r_k + r_v).
    """
    if variant == "per_head":
        return Fraction(2 * T * heads * d_head, (r_k + r_v) * heads)
    if variant == "2d":
        return Fraction(2 * T * heads * d_head, r_k + r_v)
    raise ValueError(variant)


def teacher_cache_scalars(T: int, layers: int, heads: int, d_head: int,
                          tokens: int) -> int:
    """Scalars in the uncompressed loop-indexed cache ([paper] Sec. 3,
    teacher cache): K and V for every loop, head and layer of every token."""
    return 2 * T * layers * heads * d_head * tokens


def latent_store_scalars(layers: int, tokens: int, store_heads: int,
                         r_k: int, r_v: int) -> int:
    """Scalars in the latent store: r_k + r_v per token, layer and stored
    head (H stored heads per-head, 1 for LLA-2D)."""
    return layers * tokens * store_heads * (r_k + r_v)


def store_offset(shape, b: int, layer: int, j: int, h: int, k: int) -> int:
    """Element offset of latent component k of (sequence b, layer, slot j,
    stored head h) in a row-major store of shape [B, D, N, H', r_k + r_v].
    Components [0, r_k) are the K latent, [r_k, r_k + r_v) the V latent."""
    B, D, N, Hs, R = (int(s) for s in shape)
    for v, n in ((b, B), (layer, D), (j, N), (h, Hs), (k, R)):
        if not 0 <= v < n:
            raise IndexError((v, n))
    return (((b * D + layer) * N + j) * Hs + h) * R + k


# --------------------------------------------------------------------------
# Rounding helper for comparing stored latents
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), directly
    from float64 (no intermediate float32 rounding).  Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                 # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # bf16 shares float32's exponent range
    q = np.ldexp(1.0, e - 8)           # spacing of 8-bit significands
    with np.errstate(invalid="ignore"):
        r = np.round(x / q) * q        # numpy rounds half to even
    return np.where(np.isfinite(x), r, x)


# --------------------------------------------------------------------------
# The codec: Eqs. (1)-(3)
# --------------------------------------------------------------------------
def stack_loops(per_loop: np.ndarray) -> np.ndarray:
    """Eq. (1): stack the T per-loop vectors of one token/layer/head/axis,
    per_loop[..., t, :] -> x[..., t*d:(t+1)*d]."""
    per_loop = np.asarray(per_loop, dtype=np.float64)
    return per_loop.reshape(per_loop.shape[:-2] + (-1,))


def encode(x: np.ndarray, mu: np.ndarray, W_down: np.ndarray) -> np.ndarray:
    """Eq. (2): c = (x - mu) W_down.

    x: [..., T*d] stacked loop vectors; mu: [T*d]; W_down: [T*d, r].
    Returns c: [..., r] in float64."""
    x = np.asarray(x, np.float64)
    mu = np.asarray(mu, np.float64)
    W_down = np.asarray(W_down, np.float64)
    return (x - mu) @ W_down


def loop_slice(v: np.ndarray, t: int, width: int) -> np.ndarray:
    """mu_t: the loop-t block of a stacked vector (rows t*width..)."""
    return np.asarray(v, np.float64)[..., t * width:(t + 1) * width]


def reconstruct(c: np.ndarray, W_up_t: np.ndarray, mu_t: np.ndarray) -> np.ndarray:
    """Eq. (3): x_hat_t = c W_up,t^T + mu_t, W_up,t in R^{d x r}."""
    c = np.asarray(c, np.float64)
    return c @ np.asarray(W_up_t, np.float64).T + np.asarray(mu_t, np.float64)


# --------------------------------------------------------------------------
# Rotary position embedding ([paper] Sec. 3, "RoPE and reconstruction")
# --------------------------------------------------------------------------
def rope_frequencies(d_head: int, base: float = ROPE_BASE) -> np.ndarray:
    """theta_i = base^(-2i/d), i = 0..d/2-1."""
    i = np.arange(d_head // 2, dtype=np.float64)
    return base ** (-2.0 * i / d_head)


def rope(x: np.ndarray, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate-half RoPE of x[..., d] at integer position(s) pos.

    Pair i is (x_i, x_{i+d/2}); it is rotated by the angle pos*theta_i:
      x_i'       = x_i cos - x_{i+d/2} sin
      x_{i+d/2}' = x_i sin + x_{i+d/2} cos
    pos broadcasts against x's leading dimensions."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    theta = rope_frequencies(d, base)
    ang = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# --------------------------------------------------------------------------
# Attention over the reconstructed cache
# --------------------------------------------------------------------------
def _softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max())
    return e / e.sum()


def decode_head(c_k: np.ndarray, c_v: np.ndarray, q: np.ndarray,
                W_up_k_t: np.ndarray, W_up_v_t: np.ndarray,
                mu_k_t: np.ndarray, mu_v_t: np.ndarray, pos: int,
                scale: float | None = None, base: float = ROPE_BASE,
                check_latent_v: bool = True) -> np.ndarray:
    """One head's decode-time attention at loop t over the latent store.

    c_k: [N, r_k], c_v: [N, r_v] latents of slots 0..N-1 of one (sequence,
    layer, head); q: [d] pre-RoPE query; W_up_*_t: [d, r]; mu_*_t: [d].

    Steps, in the paper's order: reconstruct the loop-t key of every slot
    j <= pos (Eq. 3), rotate it at position j (RoPE after reconstruction),
    rotate q at pos, take causal softmax attention, and reconstruct the
    loop-t values (Eq. 3) that the weights average.  Returns out: [d].
    """
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n = pos + 1
    k_hat = reconstruct(c_k[:n], W_up_k_t, mu_k_t)              # [n, d]
    k_rot = rope(k_hat, np.arange(n), base)                     # [n, d]
    q_rot = rope(q, pos, base)                                  # [d]
    p = _softmax(scale * (k_rot @ q_rot))                       # [n]
    v_hat = reconstruct(c_v[:n], W_up_v_t, mu_v_t)              # [n, d]
    out = p @ v_hat
    if check_latent_v:
        # The weights sum to one, so averaging reconstructed values equals
        # reconstructing the averaged latent: sum_j p_j (W c_j + mu) =
        # W (sum_j p_j c_j) + mu.  The GPU path relies on this identity.
        out_lat = reconstruct(p @ np.asarray(c_v[:n], np.float64),
                              W_up_v_t, mu_v_t)
        err = np.linalg.norm(out - out_lat)
        assert err <= 1e-11 * max(1.0, np.linalg.norm(out)), err
    return out


def decode(c_k: np.ndarray, c_v: np.ndarray, q: np.ndarray,
           W_up_k_t: np.ndarray, W_up_v_t: np.ndarray,
           mu_k_t: np.ndarray, mu_v_t: np.ndarray, pos: int,
           scale: float | None = None, base: float = ROPE_BASE) -> np.ndarray:
    """Per-head LLA decode for one (sequence, layer, loop t).

    c_k: [N, H, r_k], c_v: [N, H, r_v] (one [layer] slab of the store);
    q: [H, d]; W_up_*_t: [H, d, r]; mu_*_t: [H, d]; pos: query position.
    Returns out: [H, d]."""
    H = q.shape[0]
    return np.stack([
        decode_head(c_k[:, h], c_v[:, h], q[h], W_up_k_t[h], W_up_v_t[h],
                    mu_k_t[h], mu_v_t[h], pos, scale, base)
        for h in range(H)])


def decode_2d(c_k: np.ndarray, c_v: np.ndarray, q: np.ndarray,
              W_up_k_t: np.ndarray, W_up_v_t: np.ndarray,
              mu_k_t: np.ndarray, mu_v_t: np.ndarray, pos: int,
              scale: float | None = None, base: float = ROPE_BASE) -> np.ndarray:
    """LLA-2D decode for one (sequence, layer, loop t) ([paper] Sec. 3,
    LLA-2D variant): one latent per token and layer decodes all H heads.

    c_k: [N, r_k], c_v: [N, r_v]; q: [H, d]; W_up_*_t: [H*d, r] with rows
    ordered [h][d]; mu_*_t: [H*d].  Head h reconstructs rows h*d..h*d+d-1,
    then attends exactly as the per-head codec.  Returns out: [H, d]."""
    H, d = q.shape
    outs = []
    for h in range(H):
        rows = slice(h * d, (h + 1) * d)
        outs.append(decode_head(c_k, c_v, q[h], W_up_k_t[rows], W_up_v_t[rows],
                                mu_k_t[rows], mu_v_t[rows], pos, scale, base))
    return np.stack(outs)


# --------------------------------------------------------------------------
# Brute force: the explicitly materialised T-loop cache
# --------------------------------------------------------------------------
def materialise_loop_cache(c_k: np.ndarray, c_v: np.ndarray,
                           W_up_k: np.ndarray, W_up_v: np.ndarray,
                           mu_k: np.ndarray, mu_v: np.ndarray,
                           base: float = ROPE_BASE):
    """Rebuild the uncompressed cache of every loop for one head:
    K[t, j] = RoPE(c_k[j] W_up,k,t^T + mu_k,t, j) and V[t, j] likewise
    without RoPE.  W_up_*: [T, d, r]; mu_*: [T*d].  Returns (K, V) of
    shape [T, N, d]."""
    T, d = W_up_k.shape[0], W_up_k.shape[1]
    N = c_k.shape[0]
    K = np.stack([rope(reconstruct(c_k, W_up_k[t], loop_slice(mu_k, t, d)),
                       np.arange(N), base) for t in range(T)])
    V = np.stack([reconstruct(c_v, W_up_v[t], loop_slice(mu_v, t, d))
                  for t in range(T)])
    return K, V


# --------------------------------------------------------------------------
# Multi-query causal decode with the in-flight tokens
# --------------------------------------------------------------------------
def decode_inflight(c_k: np.ndarray, c_v: np.ndarray, q: np.ndarray, k_new: np.ndarray,
                    v_new: np.ndarray, W_up_k_t: np.ndarray, W_up_v_t: np.ndarray,
                    mu_k_t: np.ndarray, mu_v_t: np.ndarray, pos0: int,
                    variant: str = "per_head", scale: float | None = None,
                    base: float = ROPE_BASE) -> np.ndarray:
    """Decode at loop t for n_q new tokens of one sequence whose latents do
    not exist yet ([paper] Sec. 3 Eq. 2 needs the whole T-loop stack): new
    token i sits at position pos0 + i and attends, with ordinary causal
    softmax attention, the stored slots 0..pos0-1 (reconstructed by Eq. 3,
    RoPE at each slot's position) and the new tokens 0..i through their own
    loop-t keys and values k_new, v_new (RoPE at pos0 + m).

    c_k, c_v: [N, H', r] latents of the (sequence, layer) slab (H' = H
    per-head, 1 for LLA-2D); q, k_new, v_new: [n_q, H, d]; W_up_*_t, mu_*_t
    as decode / decode_2d.  Returns out: [n_q, H, d]."""
    q = np.asarray(q, np.float64)
    n_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n_q, H, d))
    for h in range(H):
        if variant == "2d":
            rows = slice(h * d, (h + 1) * d)
            ck, cv = c_k[:pos0, 0], c_v[:pos0, 0]
            Wk, Wv, mk, mv = W_up_k_t[rows], W_up_v_t[rows], mu_k_t[rows], mu_v_t[rows]
        else:
            ck, cv = c_k[:pos0, h], c_v[:pos0, h]
            Wk, Wv, mk, mv = W_up_k_t[h], W_up_v_t[h], mu_k_t[h], mu_v_t[h]
        K_store = rope(reconstruct(ck, Wk, mk), np.arange(pos0), base)      # [pos0, d]
        V_store = reconstruct(cv, Wv, mv)
        K_new = rope(np.asarray(k_new, np.float64)[:, h], pos0 + np.arange(n_q), base)
        V_new = np.asarray(v_new, np.float64)[:, h]
        for i in range(n_q):
            K = np.concatenate([K_store, K_new[:i + 1]])
            V = np.concatenate([V_store, V_new[:i + 1]])
            p = _softmax(scale * (K @ rope(q[i, h], pos0 + i, base)))
            out[i, h] = p @ V
    return out


# --------------------------------------------------------------------------
# Uncompressed K/V cache: the serving "fast path" and the final-loop control
# --------------------------------------------------------------------------
def fast_path_rows(c_k: np.ndarray, c_v: np.ndarray, W_up_k_t: np.ndarray,
                   W_up_v_t: np.ndarray, mu_k_t: np.ndarray, mu_v_t: np.ndarray,
                   positions, base: float = ROPE_BASE):
    """The rows the serving fast path caches ([summary] "Serving Capacity":
    reconstruct once, keep full K/V): for latents c_*: [n, r] of the slots at
    `positions`, the loop-t key reconstructed by Eq. 3 and then rotated at
    its slot ("RoPE and reconstruction"), and the loop-t value.
    Returns (K, V): [n, d] each."""
    K = rope(reconstruct(c_k, W_up_k_t, mu_k_t), positions, base)
    V = reconstruct(c_v, W_up_v_t, mu_v_t)
    return K, V


def cache_rows(k: np.ndarray, v: np.ndarray, positions, base: float = ROPE_BASE):
    """What an ordinary K/V cache stores for raw keys/values k, v: [n, d]
    at `positions`: the key rotated at its slot, the value unchanged."""
    return rope(k, positions, base), np.asarray(v, np.float64)


def decode_cache(K: np.ndarray, V: np.ndarray, q: np.ndarray, pos: int,
                 scale: float | None = None, base: float = ROPE_BASE) -> np.ndarray:
    """Ordinary causal softmax attention of one head's pre-RoPE query q: [d]
    at position pos over a cache whose keys K: [N, d] are already rotated
    (values V: [N, d]): softmax(scale * K[:pos+1] . RoPE(q, pos)) V[:pos+1]."""
    q = np.asarray(q, np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n = pos + 1
    p = _softmax(scale * (np.asarray(K, np.float64)[:n] @ rope(q, pos, base)))
    return p @ np.asarray(V, np.float64)[:n]


def final_loop_control(k_last: np.ndarray, v_last: np.ndarray, q_t: np.ndarray, pos: int,
                       scale: float | None = None, base: float = ROPE_BASE) -> np.ndarray:
    """The zero-parameter control of [paper] Sec. 3 (matched-axis baselines):
    only the final loop's keys and values k_last, v_last: [N, d] (pre-RoPE)
    are cached, and the query of every loop t attends to them.  q_t: [d]."""
    K, V = cache_rows(k_last, v_last, np.arange(np.asarray(k_last).shape[0]), base)
    return decode_cache(K, V, q_t, pos, scale, base)


# --------------------------------------------------------------------------
# SVD codec initialisation ([paper] Sec. 3, initialisation and conversion)
# --------------------------------------------------------------------------
def svd_init(x: np.ndarray, loops: int, width: int, r: int):
    """Initialise one codec from calibration rows x: [n_cal, T*width] of its
    stacked loop vectors (Eq. 1): centre by the per-loop mean (the column
    mean of the stacked rows), take W_down as the r leading right singular
    vectors of the centred matrix, and W_up,t as W_down's loop-t rows.
    Singular vectors are defined up to sign; each column is signed so that
    its entry of largest magnitude is positive (a named choice, mirrored by
    the kernels).  Returns (mu [K], W_down [K, r], [W_up,t [width, r]],
    sigma [r])."""
    X = np.asarray(x, np.float64)
    mu = X.mean(axis=0)
    # With fewer rows than r the centred matrix has fewer than r singular
    # values: the rest are zero and their vectors complete an orthonormal basis.
    full = r > min(X.shape)
    _, S, Vt = np.linalg.svd(X - mu, full_matrices=full)
    S = np.concatenate([S, np.zeros(max(0, r - S.shape[0]))])
    W = Vt[:r].T.copy()
    lead = np.argmax(np.abs(W), axis=0)
    W *= np.where(W[lead, np.arange(r)] < 0, -1.0, 1.0)
    W_up = [W[t * width:(t + 1) * width] for t in range(loops)]
    return mu, W, W_up, S[:r]


def codec_error(x: np.ndarray, mu: np.ndarray, W_down: np.ndarray, W_up: list) -> float:
    """Relative squared reconstruction error of rows x: [n, T*width] through
    the codec: encode by Eq. 2, rebuild every loop by Eq. 3, and compare with
    the centred energy: sum ||x - x_hat||^2 / sum ||x - mu||^2."""
    X = np.asarray(x, np.float64)
    c = encode(X, mu, W_down)
    width = np.asarray(W_up[0]).shape[0]
    X_hat = np.concatenate([reconstruct(c, W_up[t], loop_slice(mu, t, width))
                            for t in range(len(W_up))], axis=1)
    return float(((X - X_hat) ** 2).sum() / ((X - mu) ** 2).sum())
