"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin is written as a plain function so that ``test_oracle_mutants``
can re-run all of them against deliberately broken copies of the oracle
(planted on the CPU) and check that every plausible mistake is caught.

Sources: "Looped Latent Attention: Cross-Loop KV Compression for Looped
Transformers" (arXiv 2607.15456) -- Section 3 Eqs. (1)-(4), "RoPE and
reconstruction", "LLA-2D variant", SVD-initialisation convention; and the
gist.science technical summary of the same paper, "Serving Capacity".
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import lla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent helpers (library routines, complex arithmetic)
# --------------------------------------------------------------------------
def rope_complex(x, pos, base=10000.0):
    """RoPE as multiplication of z_i = x_i + i x_{i+d/2} by exp(i pos theta_i)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    theta = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def sdpa_last_query(q_rot, K_rot, V, scale):
    """Causal attention of one query over K/V rows via torch's library
    routine (float64, CPU)."""
    q = torch.from_numpy(np.ascontiguousarray(q_rot))[None, None, None, :]
    k = torch.from_numpy(np.ascontiguousarray(K_rot))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return out[0, 0, 0].numpy()


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# pins (raise AssertionError on failure)
# --------------------------------------------------------------------------
def pin_ratio_closed_form():
    """Eq. (4) equals the ratio of the two cache sizes the text counts."""
    for T, d, rk, rv, H in [(4, 128, 16, 32, 16), (4, 64, 8, 16, 2), (16, 128, 48, 80, 16),
                            (3, 10, 5, 7, 3), (32, 96, 13, 29, 1)]:
        D, N = 5, 7
        got = O.compression_ratio(T, d, rk, rv, H)
        assert got == Fraction(2 * T * d, rk + rv)
        sizes = Fraction(O.teacher_cache_scalars(T, D, H, d, N),
                         O.latent_store_scalars(D, N, H, rk, rv))
        assert got == sizes, (got, sizes)
        got2 = O.compression_ratio(T, d, rk, rv, H, "2d")
        assert got2 == Fraction(O.teacher_cache_scalars(T, D, H, d, N),
                                O.latent_store_scalars(D, N, 1, rk, rv))
        assert got2 == H * got


def pin_serving_capacity_example():
    """Printed worked example: 768 GiB -> 36 GiB at 21.3x, 1M context."""
    with open(os.path.join(GOLDEN, "serving_capacity.json")) as f:
        g = json.load(f)
    p, r = g["printed"], g["reading"]
    GiB = 2 ** 30
    assert p["loops_T"] * p["layers_D"] == p["cache_layers_T_times_D"]
    full = O.teacher_cache_scalars(p["loops_T"], p["layers_D"], r["heads"], r["d_head"],
                                   p["context_tokens"]) * r["bytes_per_scalar"]
    assert full == p["uncompressed_GiB"] * GiB
    # the loop-indexed cache equals a T*D-layer single-pass cache
    assert full == O.teacher_cache_scalars(1, p["cache_layers_T_times_D"], r["heads"],
                                           r["d_head"], p["context_tokens"]) * 2
    rho = O.compression_ratio(p["loops_T"], r["d_head"], r["r_k_plus_r_v"], 0, r["heads"])
    assert f"{float(rho):.1f}" == p["compression_label"]
    comp = O.latent_store_scalars(p["layers_D"], p["context_tokens"], r["heads"],
                                  r["r_k_plus_r_v"], 0) * r["bytes_per_scalar"]
    assert comp == p["compressed_GiB"] * GiB
    assert Fraction(full, comp) == rho


def pin_store_offset():
    rng = np.random.default_rng(5)
    shape = (3, 4, 5, 6, 7)
    seen = set()
    for idx in np.ndindex(*shape):
        o = O.store_offset(shape, *idx)
        assert o == np.ravel_multi_index(idx, shape)
        seen.add(o)
    assert seen == set(range(int(np.prod(shape))))
    big = (768, 24, 4096, 16, 48)
    for _ in range(50):
        idx = tuple(int(rng.integers(0, s)) for s in big)
        assert O.store_offset(big, *idx) == int(np.ravel_multi_index(idx, big))
    last = O.store_offset(big, *(s - 1 for s in big))
    assert last == int(np.prod(big, dtype=np.int64)) - 1 > 2 ** 31


def pin_exact_reconstruction():
    """r = T*d with orthonormal W_down and W_up,t = its loop-t slice (the
    SVD-initialisation convention) reconstructs every loop exactly."""
    rng = np.random.default_rng(1)
    for T, d in [(4, 8), (3, 6)]:
        Q, _ = np.linalg.qr(rng.standard_normal((T * d, T * d)))
        per_loop = rng.standard_normal((5, T, d))
        x = O.stack_loops(per_loop)
        mu = rng.standard_normal(T * d)
        c = O.encode(x, mu, Q)
        for t in range(T):
            xt = O.reconstruct(c, Q[t * d:(t + 1) * d, :], O.loop_slice(mu, t, d))
            assert np.abs(xt - per_loop[:, t]).max() < 1e-12
    # T = 1, square codec: a transposed up-projection would not invert
    Q, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    x, mu = rng.standard_normal((4, 6)), rng.standard_normal(6)
    assert np.abs(O.reconstruct(O.encode(x, mu, Q), Q, mu) - x).max() < 1e-12


def _teacher_setup(rng, T, H, d, N):
    """A teacher cache (per token, loop, head: K and V vectors) and an
    exact codec for it (r = T*d, orthonormal)."""
    K = rng.standard_normal((N, T, H, d))
    V = rng.standard_normal((N, T, H, d))
    codec = {}
    for axis in "kv":
        Q = np.stack([np.linalg.qr(rng.standard_normal((T * d, T * d)))[0] for _ in range(H)])
        mu = rng.standard_normal((H, T * d)) * 0.3
        codec[axis] = (Q, mu)
    return K, V, codec


def pin_decode_equals_teacher_attention():
    """End to end: encode the teacher's loop-indexed cache with an exact
    codec, decode at every loop and position, and compare with ordinary
    RoPE causal attention (complex-number RoPE, torch's attention routine)
    over the teacher's own loop-t K/V."""
    rng = np.random.default_rng(2)
    T, H, d, N = 3, 2, 8, 12
    K, V, codec = _teacher_setup(rng, T, H, d, N)
    c = {}
    for axis, X in (("k", K), ("v", V)):
        Q, mu = codec[axis]
        c[axis] = np.stack([O.encode(O.stack_loops(X[:, :, h]), mu[h], Q[h])
                            for h in range(H)], axis=1)           # [N, H, T*d]
    q = rng.standard_normal((H, d))
    scale = 1 / np.sqrt(d)
    for t in range(T):
        Wk = codec["k"][0][:, t * d:(t + 1) * d, :]
        Wv = codec["v"][0][:, t * d:(t + 1) * d, :]
        mk = codec["k"][1][:, t * d:(t + 1) * d]
        mv = codec["v"][1][:, t * d:(t + 1) * d]
        for pos in range(N):
            out = O.decode(c["k"], c["v"], q, Wk, Wv, mk, mv, pos)
            for h in range(H):
                Kt = rope_complex(K[:pos + 1, t, h], np.arange(pos + 1))
                ref = sdpa_last_query(rope_complex(q[h], pos), Kt, V[:pos + 1, t, h], scale)
                assert rel(out[h], ref) < 1e-12, (t, pos, h, rel(out[h], ref))


def pin_decode_equals_materialised_cache():
    """Low-rank codec: decoding the latent store equals library attention
    over the explicitly materialised T-loop cache, for every loop and
    query position."""
    rng = np.random.default_rng(3)
    T, d, rk, rv, N = 4, 16, 5, 7, 20
    ck, cv = rng.standard_normal((N, rk)), rng.standard_normal((N, rv))
    Wk, Wv = rng.standard_normal((T, d, rk)), rng.standard_normal((T, d, rv))
    mk, mv = rng.standard_normal(T * d), rng.standard_normal(T * d)
    q = rng.standard_normal(d)
    Kc, Vc = O.materialise_loop_cache(ck, cv, Wk, Wv, mk, mv)
    for t in range(T):
        # the materialised cache agrees with the definition of Eq. (3) + RoPE
        Kdef = rope_complex(ck @ Wk[t].T + mk[t * d:(t + 1) * d], np.arange(N))
        assert np.abs(Kc[t] - Kdef).max() < 1e-12
        for pos in range(N):
            out = O.decode_head(ck, cv, q, Wk[t], Wv[t], O.loop_slice(mk, t, d),
                                O.loop_slice(mv, t, d), pos)
            ref = sdpa_last_query(rope_complex(q, pos), Kc[t, :pos + 1], Vc[t, :pos + 1],
                                  1 / np.sqrt(d))
            assert rel(out, ref) < 1e-12


def pin_special_cases():
    rng = np.random.default_rng(4)
    d, rk, rv, N = 8, 3, 4, 10
    ck, cv = rng.standard_normal((N, rk)), rng.standard_normal((N, rv))
    Wk, Wv = rng.standard_normal((d, rk)), rng.standard_normal((d, rv))
    mk, mv = rng.standard_normal(d), rng.standard_normal(d)
    q = rng.standard_normal(d)
    # a query at position 0 sees one slot: the output is that slot's value
    out0 = O.decode_head(ck, cv, q, Wk, Wv, mk, mv, 0)
    assert np.abs(out0 - (Wv @ cv[0] + mv)).max() < 1e-13
    # all latents zero: every value reconstructs to mu_v,t
    outz = O.decode_head(0 * ck, 0 * cv, q, Wk, Wv, mk, mv, N - 1)
    assert np.abs(outz - mv).max() < 1e-14
    # T = 1, r = d, W = I, mu = 0: plain RoPE attention over the latents
    ckd, cvd = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    eye, zero = np.eye(d), np.zeros(d)
    for pos in (0, 3, N - 1):
        out = O.decode_head(ckd, cvd, q, eye, eye, zero, zero, pos, scale=0.7)
        ref = sdpa_last_query(rope_complex(q, pos),
                              rope_complex(ckd[:pos + 1], np.arange(pos + 1)),
                              cvd[:pos + 1], 0.7)
        assert rel(out, ref) < 1e-12
    # only slots 0..pos are read: garbage beyond pos changes nothing
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[6:] = 1e6
    cv2[6:] = -1e6
    assert np.array_equal(O.decode_head(ck, cv, q, Wk, Wv, mk, mv, 5),
                          O.decode_head(ck2, cv2, q, Wk, Wv, mk, mv, 5))


def pin_rope():
    rng = np.random.default_rng(6)
    d = 16
    x = rng.standard_normal((7, d))
    pos = rng.integers(0, 5000, 7)
    assert np.abs(O.rope(x, 0) - x).max() == 0
    assert np.abs(O.rope(x, pos) - rope_complex(x, pos)).max() < 1e-12
    assert np.allclose(np.linalg.norm(O.rope(x, pos), axis=-1), np.linalg.norm(x, axis=-1),
                       rtol=1e-14)
    # scores depend on positions only through their difference
    qv, kv = rng.standard_normal(d), rng.standard_normal(d)
    a = O.rope(qv, 40) @ O.rope(kv, 17)
    b = O.rope(qv, 40 + 1234) @ O.rope(kv, 17 + 1234)
    assert abs(a - b) < 1e-11
    # theta_0 = 1 and theta_{d/2-1} = base^{-(d-2)/d}
    th = O.rope_frequencies(d)
    assert th[0] == 1.0 and abs(th[-1] - 10000.0 ** (-(d - 2) / d)) < 1e-16


def pin_2d_reduces_to_per_head():
    """LLA-2D with block-diagonal up-projections over concatenated per-head
    latents is per-head LLA; its ratio is H times larger at equal r."""
    rng = np.random.default_rng(7)
    H, d, rk, rv, N = 3, 8, 2, 3, 9
    ck, cv = rng.standard_normal((N, H, rk)), rng.standard_normal((N, H, rv))
    Wk, Wv = rng.standard_normal((H, d, rk)), rng.standard_normal((H, d, rv))
    mk, mv = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    q = rng.standard_normal((H, d))
    Wk2 = np.zeros((H * d, H * rk))
    Wv2 = np.zeros((H * d, H * rv))
    for h in range(H):
        Wk2[h * d:(h + 1) * d, h * rk:(h + 1) * rk] = Wk[h]
        Wv2[h * d:(h + 1) * d, h * rv:(h + 1) * rv] = Wv[h]
    for pos in (0, 4, N - 1):
        a = O.decode(ck, cv, q, Wk, Wv, mk, mv, pos)
        b = O.decode_2d(ck.reshape(N, -1), cv.reshape(N, -1), q, Wk2, Wv2,
                        mk.reshape(-1), mv.reshape(-1), pos)
        assert np.abs(a - b).max() < 1e-12
    # LLA-2D encode over the [t][h][d] stack with a block-diagonal W_down
    T = 2
    xs = rng.standard_normal((5, T, H, d))
    mu = rng.standard_normal((T, H, d))
    Wd = rng.standard_normal((H, T * d, rk))
    Wd2 = np.zeros((T * H * d, H * rk))
    for h in range(H):
        for t in range(T):
            Wd2[t * H * d + h * d: t * H * d + (h + 1) * d, h * rk:(h + 1) * rk] = \
                Wd[h, t * d:(t + 1) * d]
    c2 = O.encode(xs.reshape(5, -1), mu.reshape(-1), Wd2)
    c1 = np.concatenate([O.encode(xs[:, :, h].reshape(5, -1), mu[:, h].reshape(-1), Wd[h])
                         for h in range(H)], axis=1)
    assert np.abs(c1 - c2).max() < 1e-12


def pin_inflight():
    """Multi-query decode with in-flight tokens.
    (a) A new token whose loop-t key/value are exactly the reconstruction of
        a latent gives the store-only decode of that latent placed at slot
        pos0 (the same attention, assembled from two independent paths).
    (b) pos0 = 0, one new token: it attends only itself, out = v_new.
    (c) Causality: query i ignores the new tokens after it.
    (d) All queries against library attention (torch, fp64) over the
        explicitly concatenated [materialised store; new] keys with a causal
        mask, complex-number RoPE."""
    rng = np.random.default_rng(12)
    H, d, rk, rv, N, n_q = 2, 8, 3, 5, 30, 4
    ck, cv = rng.standard_normal((N, H, rk)), rng.standard_normal((N, H, rv))
    Wk, Wv = rng.standard_normal((H, d, rk)), rng.standard_normal((H, d, rv))
    mk, mv = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    q = rng.standard_normal((n_q, H, d))
    kn, vn = rng.standard_normal((n_q, H, d)), rng.standard_normal((n_q, H, d))
    pos0 = 17
    # (a)
    k1 = np.stack([O.reconstruct(ck[pos0, h], Wk[h], mk[h]) for h in range(H)])
    v1 = np.stack([O.reconstruct(cv[pos0, h], Wv[h], mv[h]) for h in range(H)])
    got = O.decode_inflight(ck, cv, q[:1], k1[None], v1[None], Wk, Wv, mk, mv, pos0)[0]
    ref = O.decode(ck, cv, q[0], Wk, Wv, mk, mv, pos0)
    assert rel(got, ref) < 1e-12, rel(got, ref)
    # (b)
    got = O.decode_inflight(ck, cv, q[:1], kn[:1], vn[:1], Wk, Wv, mk, mv, 0)[0]
    assert np.abs(got - vn[0]).max() < 1e-12
    # (c)
    a = O.decode_inflight(ck, cv, q, kn, vn, Wk, Wv, mk, mv, pos0)
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[2:], vn2[2:] = rng.standard_normal((2, H, d)), rng.standard_normal((2, H, d))
    b = O.decode_inflight(ck, cv, q, kn2, vn2, Wk, Wv, mk, mv, pos0)
    assert np.array_equal(a[:2], b[:2]) and not np.allclose(a[2:], b[2:])
    # (d)
    for h in range(H):
        Ks = rope_complex(ck[:pos0, h] @ Wk[h].T + mk[h], np.arange(pos0))
        Vs = cv[:pos0, h] @ Wv[h].T + mv[h]
        K = np.concatenate([Ks, rope_complex(kn[:, h], pos0 + np.arange(n_q))])
        V = np.concatenate([Vs, vn[:, h]])
        Q = rope_complex(q[:, h], pos0 + np.arange(n_q))
        mask = np.arange(pos0 + n_q)[None, :] <= (pos0 + np.arange(n_q))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], attn_mask=torch.from_numpy(mask)[None, None],
            scale=1 / np.sqrt(d))[0, 0].numpy()
        assert rel(a[:, h], ref) < 1e-12, (h, rel(a[:, h], ref))
    # (e) LLA-2D with concatenated per-head latents and a block-diagonal W_up
    #     is per-head LLA, in-flight tokens included
    c2k = ck.reshape(N, 1, H * rk)
    c2v = cv.reshape(N, 1, H * rv)
    W2k = np.zeros((H * d, H * rk))
    W2v = np.zeros((H * d, H * rv))
    for h in range(H):
        W2k[h * d:(h + 1) * d, h * rk:(h + 1) * rk] = Wk[h]
        W2v[h * d:(h + 1) * d, h * rv:(h + 1) * rv] = Wv[h]
    g = O.decode_inflight(c2k, c2v, q, kn, vn, W2k, W2v, mk.reshape(-1), mv.reshape(-1), pos0,
                          variant="2d")
    assert rel(g, a) < 1e-12


def pin_bf16_round():
    one = 1.0
    cases = {one: one, one + 2 ** -8: one, one + 3 * 2 ** -8: one + 2 ** -6,
             one + 2 ** -8 + 2 ** -30: one + 2 ** -7, -(one + 2 ** -8 + 2 ** -30): -(one + 2 ** -7),
             2 ** -130: 2 ** -130, 2 ** -133 * 1.5: 2 ** -132}
    for x, want in cases.items():
        assert O.bf16_round(np.array([x]))[0] == want, x
    x32 = np.random.default_rng(8).standard_normal(4096).astype(np.float32) * 3
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x32.astype(np.float64)), want)


def pin_kv_cache():
    """The uncompressed-cache paths: the serving fast path ([summary]
    "Serving Capacity") and the final-loop control ([paper] Sec. 3,
    matched-axis baselines).
    (a) decode_cache over cache_rows equals torch's library attention (fp64)
        over keys rotated by complex multiplication, at every position.
    (b) fast_path_rows equals c W^T + mu rotated by complex multiplication at
        the slot, and decoding over them equals the LLA oracle (reconstruct on
        read) at every position: the two serving paths compute one thing.
    (c) Special cases: at pos = 0 the output is V[0]; with all keys equal it
        is the mean of V[:pos+1].
    (d) With an exact codec (r = T*d, square orthonormal W_down, W_up,t its
        loop-t rows) LLA at the final loop equals the control; at loop 0 the
        control still attends final-loop keys and differs."""
    rng = np.random.default_rng(21)
    d, N, rk, rv = 8, 19, 3, 5
    k, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    q = rng.standard_normal(d)
    K, V = O.cache_rows(k, v, np.arange(N))
    for pos in (0, 1, 7, N - 1):
        got = O.decode_cache(K, V, q, pos)
        ref = sdpa_last_query(rope_complex(q, pos), rope_complex(k[:pos + 1], np.arange(pos + 1)),
                              v[:pos + 1], 1 / np.sqrt(d))
        assert rel(got, ref) < 1e-12, (pos, rel(got, ref))
    # (b)
    ck, cv = rng.standard_normal((N, rk)), rng.standard_normal((N, rv))
    Wk, Wv = rng.standard_normal((d, rk)), rng.standard_normal((d, rv))
    mk, mv = rng.standard_normal(d), rng.standard_normal(d)
    Kf, Vf = O.fast_path_rows(ck, cv, Wk, Wv, mk, mv, np.arange(N))
    assert rel(Kf, rope_complex(ck @ Wk.T + mk, np.arange(N))) < 1e-12
    assert rel(Vf, cv @ Wv.T + mv) < 1e-12
    for pos in (0, 5, N - 1):
        got = O.decode_cache(Kf, Vf, q, pos)
        ref = O.decode_head(ck, cv, q, Wk, Wv, mk, mv, pos)
        assert rel(got, ref) < 1e-12, (pos, rel(got, ref))
    # rows for a slot range starting past 0 are those rows of the full fill
    K3, V3 = O.fast_path_rows(ck[4:9], cv[4:9], Wk, Wv, mk, mv, np.arange(4, 9))
    assert rel(K3, Kf[4:9]) < 1e-14 and rel(V3, Vf[4:9]) < 1e-14
    # (c)
    assert np.abs(O.decode_cache(K, V, q, 0) - v[0]).max() < 1e-12
    Keq = np.tile(rng.standard_normal(d), (N, 1))
    assert np.abs(O.decode_cache(Keq, V, q, 9) - v[:10].mean(0)).max() < 1e-12
    # (d)
    T, dd, n = 3, 4, 11
    xk = rng.standard_normal((n, T, dd))
    xv = rng.standard_normal((n, T, dd))
    muk, muv = rng.standard_normal(T * dd), rng.standard_normal(T * dd)
    Qk, _ = np.linalg.qr(rng.standard_normal((T * dd, T * dd)))
    Qv, _ = np.linalg.qr(rng.standard_normal((T * dd, T * dd)))
    c_k = O.encode(O.stack_loops(xk), muk, Qk)
    c_v = O.encode(O.stack_loops(xv), muv, Qv)
    qq = rng.standard_normal(dd)
    pos = n - 1
    for t in (T - 1, 0):
        lla = O.decode_head(c_k, c_v, qq, Qk[t * dd:(t + 1) * dd], Qv[t * dd:(t + 1) * dd],
                            O.loop_slice(muk, t, dd), O.loop_slice(muv, t, dd), pos)
        ctl = O.final_loop_control(xk[:, T - 1], xv[:, T - 1], qq, pos)
        if t == T - 1:
            assert rel(ctl, lla) < 1e-10, rel(ctl, lla)
        else:
            assert rel(ctl, lla) > 1e-3


def pin_svd_init():
    """SVD codec initialisation ([paper] Sec. 3, initialisation and
    conversion), pinned by what the mathematics fixes:
    (a) mu's loop-t slice is the mean of the loop-t vectors;
    (b) Eckart-Young: the codec's error on its calibration rows is the
        discarded energy, and no other rank-r orthonormal basis (random ones,
        small rotations of the optimum) does better;
    (c) rows of exact rank r (after centring) are rebuilt exactly;
    (d) rank one: x_n = mu0 + a_n u gives W_down = u, sigma = ||a - mean(a)||;
    (e) a constant offset moves mu only; W_down and sigma are unchanged;
    (f) W_down is orthonormal, sigma non-increasing, W_up,t its loop-t rows."""
    rng = np.random.default_rng(31)
    T, width, n, r = 3, 4, 60, 3
    K = T * width
    x = rng.standard_normal((n, 2)) @ rng.standard_normal((2, K)) * 3 \
        + 0.3 * rng.standard_normal((n, K)) + rng.standard_normal(K)
    mu, W, W_up, sig = O.svd_init(x, T, width, r)
    # (a)
    for t in range(T):
        assert np.abs(mu[t * width:(t + 1) * width] - x[:, t * width:(t + 1) * width].mean(0)).max() < 1e-12
    # (b)
    Xc = x - x.mean(0)
    tot = (Xc ** 2).sum()
    err = O.codec_error(x, mu, W, W_up)
    assert abs(err * tot - (tot - (sig ** 2).sum())) < 1e-9 * tot
    for _ in range(20):
        Qr, _ = np.linalg.qr(rng.standard_normal((K, r)))
        assert O.codec_error(x, mu, Qr, [Qr[t * width:(t + 1) * width] for t in range(T)]) >= err - 1e-12
        A = rng.standard_normal((K, K)) * 1e-3
        Rot = np.linalg.qr(np.eye(K) + A - A.T)[0]
        Wp = Rot @ W
        assert O.codec_error(x, mu, Wp, [Wp[t * width:(t + 1) * width] for t in range(T)]) >= err - 1e-12
    # (c)
    xe = rng.standard_normal((n, r)) @ rng.standard_normal((r, K)) + 5.0
    m2, W2, U2, _ = O.svd_init(xe, T, width, r)
    assert O.codec_error(xe, m2, W2, U2) < 1e-20
    # (d)
    u = rng.standard_normal(K)
    u /= np.linalg.norm(u)
    a = rng.standard_normal(n) * 2 + 1
    x1 = 0.7 + a[:, None] * u[None, :]
    _, W1, _, s1 = O.svd_init(x1, T, width, 1)
    uu = u * (1 if u[np.argmax(np.abs(u))] > 0 else -1)
    assert np.abs(W1[:, 0] - uu).max() < 1e-10
    assert abs(s1[0] - np.linalg.norm(a - a.mean())) < 1e-9
    # (e)
    off = rng.standard_normal(K) * 10
    mu3, W3, _, s3 = O.svd_init(x + off, T, width, r)
    assert np.abs(mu3 - mu - off).max() < 1e-10
    assert np.abs(W3 - W).max() < 1e-8 and np.abs(s3 - sig).max() < 1e-8
    # (c') fewer rows than r: exact, orthonormal, the missing singular values zero
    xf = rng.standard_normal((5, K))
    mf, Wf, Uf, sf = O.svd_init(xf, T, width, 8)
    assert O.codec_error(xf, mf, Wf, Uf) < 1e-20
    assert np.abs(Wf.T @ Wf - np.eye(8)).max() < 1e-12 and np.abs(sf[4:]).max() < 1e-12
    # (f)
    assert np.abs(W.T @ W - np.eye(r)).max() < 1e-12
    assert np.all(np.diff(sig) <= 0)
    for t in range(T):
        assert np.array_equal(W_up[t], W[t * width:(t + 1) * width])


PINS = [pin_ratio_closed_form, pin_serving_capacity_example, pin_store_offset,
        pin_exact_reconstruction, pin_decode_equals_teacher_attention,
        pin_decode_equals_materialised_cache, pin_special_cases, pin_rope,
        pin_2d_reduces_to_per_head, pin_bf16_round, pin_inflight, pin_kv_cache,
        pin_svd_init]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_latent_v_identity():
    """Averaging reconstructed values equals reconstructing the averaged
    latent (the weights sum to one): the oracle asserts it on every call;
    check it directly with non-normalised weights failing it."""
    rng = np.random.default_rng(9)
    W, mu = rng.standard_normal((8, 3)), rng.standard_normal(8)
    c = rng.standard_normal((6, 3))
    p = rng.random(6)
    p /= p.sum()
    lhs = p @ (c @ W.T + mu)
    assert np.abs(lhs - ((p @ c) @ W.T + mu)).max() < 1e-13
    assert np.abs((2 * p) @ (c @ W.T + mu) - ((2 * p @ c) @ W.T + mu)).max() > 1e-3
