"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins of ``test_oracle.py`` catch every one of them.

A pin suite that still passes on a broken oracle would not be evidence of
anything; each mutant below is one small, realistic slip (a dropped term, a
wrong sign, an off-by-one, a transposed operand, a swapped axis)."""
import numpy as np
import pytest

from oracle import lla_oracle as O
from tests import test_oracle as P


def _decode_head_variant(mask_extra=0, scale_pow=-0.5, rotate_q=True, key_shift=0,
                         v_uses_k=False, no_max=False):
    def decode_head(c_k, c_v, q, W_up_k_t, W_up_v_t, mu_k_t, mu_v_t, pos,
                    scale=None, base=O.ROPE_BASE, check_latent_v=True):
        d = q.shape[-1]
        if scale is None:
            scale = float(d) ** scale_pow
        n = max(pos + 1 + mask_extra, 1)
        k_hat = O.reconstruct(c_k[:n], W_up_k_t, mu_k_t)
        k_rot = O.rope(k_hat, np.arange(n) + key_shift, base)
        q_rot = O.rope(q, pos, base) if rotate_q else np.asarray(q, np.float64)
        s = scale * (k_rot @ q_rot)
        e = np.exp(s) if no_max else np.exp(s - s.max())
        p = e / e.sum()
        if v_uses_k:
            return p @ O.reconstruct(c_k[:n], W_up_k_t, mu_k_t)
        return p @ O.reconstruct(c_v[:n], W_up_v_t, mu_v_t)
    return decode_head


def _rope_variant(sign=1.0, interleaved=False, freq_div=1.0):
    def rope(x, pos, base=O.ROPE_BASE):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        theta = base ** (-2.0 * np.arange(d // 2) / d / freq_div)
        ang = sign * np.asarray(pos, np.float64)[..., None] * theta
        c, s = np.cos(ang), np.sin(ang)
        if interleaved:
            a, b = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2], out[..., 1::2] = a * c - b * s, a * s + b * c
            return out
        a, b = x[..., : d // 2], x[..., d // 2:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    return rope


def _decode_2d_interleaved_heads(c_k, c_v, q, W_up_k_t, W_up_v_t, mu_k_t, mu_v_t, pos,
                                 scale=None, base=O.ROPE_BASE):
    H, d = q.shape
    return np.stack([O.decode_head(c_k, c_v, q[h], W_up_k_t[h::H], W_up_v_t[h::H],
                                   mu_k_t[h::H], mu_v_t[h::H], pos, scale, base)
                     for h in range(H)])


def _inflight_variant(new_pos_shift=0, causal=True, q_at_pos0=False, store_extra=0,
                      new_values_are_keys=False):
    """decode_inflight with one planted slip."""
    def decode_inflight(c_k, c_v, q, k_new, v_new, W_up_k_t, W_up_v_t, mu_k_t, mu_v_t, pos0,
                        variant="per_head", scale=None, base=O.ROPE_BASE):
        q = np.asarray(q, np.float64)
        n_q, H, d = q.shape
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        out = np.zeros((n_q, H, d))
        ns = pos0 + store_extra
        for h in range(H):
            if variant == "2d":
                rows = slice(h * d, (h + 1) * d)
                ck, cv = c_k[:ns, 0], c_v[:ns, 0]
                Wk, Wv, mk, mv = W_up_k_t[rows], W_up_v_t[rows], mu_k_t[rows], mu_v_t[rows]
            else:
                ck, cv = c_k[:ns, h], c_v[:ns, h]
                Wk, Wv, mk, mv = W_up_k_t[h], W_up_v_t[h], mu_k_t[h], mu_v_t[h]
            Ks = O.rope(O.reconstruct(ck, Wk, mk), np.arange(ns), base)
            Vs = O.reconstruct(cv, Wv, mv)
            Kn = O.rope(np.asarray(k_new, np.float64)[:, h],
                        pos0 + np.arange(n_q) + new_pos_shift, base)
            Vn = (np.asarray(k_new if new_values_are_keys else v_new, np.float64))[:, h]
            for i in range(n_q):
                m = i + 1 if causal else n_q
                K, V = np.concatenate([Ks, Kn[:m]]), np.concatenate([Vs, Vn[:m]])
                s = scale * (K @ O.rope(q[i, h], pos0 if q_at_pos0 else pos0 + i, base))
                e = np.exp(s - s.max())
                out[i, h] = (e / e.sum()) @ V
        return out
    return decode_inflight


def _decode_cache_variant(rotate_q=True, extra=0):
    def decode_cache(K, V, q, pos, scale=None, base=O.ROPE_BASE):
        q = np.asarray(q, np.float64)
        d = q.shape[-1]
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        n = pos + 1 + extra
        s = scale * (np.asarray(K)[:n] @ (O.rope(q, pos, base) if rotate_q else q))
        e = np.exp(s - s.max())
        return (e / e.sum()) @ np.asarray(V)[:n]
    return decode_cache


def _fast_path_variant(rotate_before_mu=False, rotate_values=False):
    def fast_path_rows(c_k, c_v, W_up_k_t, W_up_v_t, mu_k_t, mu_v_t, positions,
                       base=O.ROPE_BASE):
        if rotate_before_mu:
            K = O.rope(np.asarray(c_k) @ np.asarray(W_up_k_t).T, positions, base) + mu_k_t
        else:
            K = O.rope(O.reconstruct(c_k, W_up_k_t, mu_k_t), positions, base)
        V = O.reconstruct(c_v, W_up_v_t, mu_v_t)
        return K, (O.rope(V, positions, base) if rotate_values else V)
    return fast_path_rows


def _svd_variant(centre=True, smallest=False, slice_shift=0, row_mean=False):
    def svd_init(x, loops, width, r):
        X = np.asarray(x, np.float64)
        mu = X.mean(axis=1, keepdims=True).repeat(X.shape[1], 1).mean(0) if row_mean else X.mean(0)
        _, S, Vt = np.linalg.svd(X - mu if centre else X, full_matrices=False)
        W = (Vt[-r:] if smallest else Vt[:r]).T.copy()
        K = W.shape[0]
        W_up = [W[((t + slice_shift) % loops) * width:((t + slice_shift) % loops + 1) * width]
                for t in range(loops)]
        return mu, W, W_up, (S[-r:] if smallest else S[:r])
    return svd_init


MUTANTS = {
    "svd_uncentred": ("svd_init", _svd_variant(centre=False)),
    "svd_smallest_vectors": ("svd_init", _svd_variant(smallest=True)),
    "svd_up_slices_shifted": ("svd_init", _svd_variant(slice_shift=1)),
    "svd_mean_over_features": ("svd_init", _svd_variant(row_mean=True)),
    "cache_keys_not_rotated": ("cache_rows", lambda k, v, positions, base=O.ROPE_BASE:
                               (np.asarray(k, np.float64), np.asarray(v, np.float64))),
    "cache_values_rotated": ("cache_rows", lambda k, v, positions, base=O.ROPE_BASE:
                             (O.rope(k, positions, base), O.rope(v, positions, base))),
    "decode_cache_query_not_rotated": ("decode_cache", _decode_cache_variant(rotate_q=False)),
    "decode_cache_one_slot_long": ("decode_cache", _decode_cache_variant(extra=1)),
    "fast_path_rotates_before_mu": ("fast_path_rows", _fast_path_variant(rotate_before_mu=True)),
    "fast_path_rotates_values": ("fast_path_rows", _fast_path_variant(rotate_values=True)),
    "control_keys_at_slot_zero": ("final_loop_control",
                                  lambda k_last, v_last, q_t, pos, scale=None, base=O.ROPE_BASE:
                                  O.decode_cache(O.rope(k_last, 0, base), v_last, q_t, pos,
                                                 scale, base)),
    "inflight_keys_rotated_one_early": ("decode_inflight", _inflight_variant(new_pos_shift=-1)),
    "inflight_not_causal": ("decode_inflight", _inflight_variant(causal=False)),
    "inflight_queries_at_pos0": ("decode_inflight", _inflight_variant(q_at_pos0=True)),
    "inflight_store_one_slot_long": ("decode_inflight", _inflight_variant(store_extra=1)),
    "inflight_values_are_keys": ("decode_inflight", _inflight_variant(new_values_are_keys=True)),
    "reconstruct_drops_mu": ("reconstruct", lambda c, W, mu: np.asarray(c) @ np.asarray(W).T),
    "encode_uncentred": ("encode", lambda x, mu, W: np.asarray(x) @ np.asarray(W)),
    "encode_adds_mu": ("encode", lambda x, mu, W: (np.asarray(x) + mu) @ np.asarray(W)),
    "rope_negative_angle": ("rope", _rope_variant(sign=-1.0)),
    "rope_interleaved_pairs": ("rope", _rope_variant(interleaved=True)),
    "rope_wrong_frequencies": ("rope", _rope_variant(freq_div=2.0)),
    "mask_one_slot_short": ("decode_head", _decode_head_variant(mask_extra=-1)),
    "mask_one_slot_long": ("decode_head", _decode_head_variant(mask_extra=1)),
    "scale_sqrt_d": ("decode_head", _decode_head_variant(scale_pow=0.5)),
    "query_not_rotated": ("decode_head", _decode_head_variant(rotate_q=False)),
    "keys_rotated_one_late": ("decode_head", _decode_head_variant(key_shift=1)),
    "values_from_key_codec": ("decode_head", _decode_head_variant(v_uses_k=True)),
    "loop_slice_reversed": ("loop_slice",
                            lambda v, t, width: np.asarray(v, np.float64)[
                                ..., (np.shape(v)[-1] // width - 1 - t) * width:
                                (np.shape(v)[-1] // width - t) * width]),
    "ratio_missing_factor_two": ("compression_ratio",
                                 lambda T, d, rk, rv, heads=1, variant="per_head":
                                 P.Fraction(T * d * (heads if variant == "2d" else 1), rk + rv)),
    "teacher_cache_one_axis": ("teacher_cache_scalars",
                               lambda T, L, H, d, n: T * L * H * d * n),
    "offset_slot_head_swapped": ("store_offset",
                                 lambda shape, b, l, j, h, k:
                                 (((b * shape[1] + l) * shape[3] + h) * shape[2] + j) * shape[4] + k),
    "2d_heads_interleaved": ("decode_2d", _decode_2d_interleaved_heads),
    "bf16_truncates": ("bf16_round",
                       lambda x: np.sign(x) * np.ldexp(np.floor(np.ldexp(np.abs(x), 8 - np.frexp(x)[1])),
                                                      np.frexp(x)[1] - 8)),
}


def _pins_fail():
    failed = []
    for pin in P.PINS:
        try:
            pin()
        except Exception:  # an assertion or a crash both reveal the mutant
            failed.append(pin.__name__)
    return failed


def test_unmutated_oracle_passes_all_pins():
    assert _pins_fail() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = _pins_fail()
    assert failed, f"mutant {name} passed every pin"
