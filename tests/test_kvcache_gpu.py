"""GPU parity of the uncompressed-cache paths against the fp64 oracle:
reconstruct-to-cache (the serving fast path's fill), raw append (the
final-loop control's), and flash-decode over the cache.

Bar: decode outputs per row (relative L2) 1e-5 for float32 caches and 2e-2
for bfloat16 caches (float32 accumulation); cache rows the fill or append
writes within one bf16 rounding (plus the float32 accumulation bound) of
the oracle's exact value, every other row of the cache untouched."""
import sys

import numpy as np
import pytest
import torch

import looped_transformer_decode_amd as L
from oracle import lla_oracle as O
from synth import gen
from synth.device import fill_hash_normal
from synth.workloads import WORKLOADS, Codec
from tests.gpu_cases import (TOL, DecodeInputs, from_device, host_store, new_store, row_rel_l2,
                             to_device)

pytestmark = pytest.mark.gpu
SENTINEL = 7.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def new_cache(dtype, B, D, Lp, N, H, d, device, fill=SENTINEL):
    c = L.KvCache(dtype, batch=B, layers=D, loops=Lp, max_ctx=N, heads=H, d_head=d,
                  device=device)
    c.tensor.fill_(fill)
    return c


def rows_close(got, ref, dtype):
    """Elementwise: within one bf16 ulp of the exact value plus a float32
    accumulation allowance (bf16); 1e-5 relative per row (float32)."""
    if dtype == "f32":
        return row_rel_l2(got, ref).max() <= TOL["f32"]
    scale = np.linalg.norm(ref, axis=-1, keepdims=True) / np.sqrt(ref.shape[-1])
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    return bool((np.abs(got - ref) <= ulp + 1e-5 * scale).all())


# ------------------------------------------------------- reconstruct-to-cache
FILL_CASES = [
    ("tiny_fp32", dict(B=2, D=2, N=150), 3, 140),                      # fp32, generic kernel
    ("bf16_b32_ctx4k", dict(B=2, D=2, N=300, H=3), 5, 290),            # MFMA, 4 k-steps
    ("extreme_batch_b768_ctx4k", dict(B=3, D=2, N=260), 0, 260),       # MFMA, 2 k-steps
    ("long_recurrence_t16_ctx8k", dict(B=2, D=2, N=200), 37, 1),       # one slot
    ("lla2d_b256_ctx4k", dict(B=2, D=2, N=170, H=4), 31, 139),         # LLA-2D store
    ("bf16_b32_ctx4k", dict(B=2, D=2, N=100, H=2, d=64), 10, 90),      # d = 64 (2 waves)
    ("bf16_b32_ctx4k", dict(B=1, D=2, N=70, H=2, d=256, r_k=16, r_v=32), 0, 70),  # d = 256
    ("bf16_b32_ctx4k", dict(B=2, D=1, N=90, H=2, r_k=8, r_v=24), 20, 50),  # ranks off 16
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=1), 0, 1),            # a single slot
    ("bf16_b32_ctx4k", dict(B=2, D=1, N=90, H=2, r_k=32, r_v=160), 7, 80),  # 10 k-steps (widest instance)
]


@pytest.mark.parametrize("tmpl,kw,slot0,n", FILL_CASES,
                         ids=[f"{c[0]}-{i}" for i, c in enumerate(FILL_CASES)])
def test_fill_from_store(device, tmpl, kw, slot0, n):
    w = WORKLOADS[tmpl].scaled(**kw)
    layer, t, cl = w.D - 1, w.T - 1, 1
    say(f"[kv fill] {w.name} {w.variant} {w.dtype} B={w.B} N={w.N} H={w.H} d={w.d} "
        f"rk={w.r_k} rv={w.r_v} slots [{slot0}, {slot0 + n})")
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), layer, t, device)
    cache = new_cache(w.dtype, w.B, w.D, 2, w.N, w.H, w.d, device)
    L.lla_kv_fill_from_store(store, layer, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv, slot0, n,
                             rope, cache, cl)
    torch.cuda.synchronize()
    got = from_device(cache.tensor)                                  # [B, D, 2, N, H, 2, d]
    pos = np.arange(slot0, slot0 + n)
    for b in range(w.B):
        lat = vals[b, layer, slot0:slot0 + n]                        # [n, H', R]
        for h in range(w.H):
            if w.variant == "2d":
                rows = slice(h * w.d, (h + 1) * w.d)
                ck, cv = lat[:, 0, :w.r_k], lat[:, 0, w.r_k:]
                Wk, Wv, mk, mv = inp.wk[0][rows], inp.wv[0][rows], inp.mk[0][rows], inp.mv[0][rows]
            else:
                ck, cv = lat[:, h, :w.r_k], lat[:, h, w.r_k:]
                Wk, Wv, mk, mv = inp.wk[h], inp.wv[h], inp.mk[h], inp.mv[h]
            K, V = O.fast_path_rows(ck, cv, Wk, Wv, mk, mv, pos)
            assert rows_close(got[b, layer, cl, slot0:slot0 + n, h, 0], K, w.dtype), (b, h, "K")
            assert rows_close(got[b, layer, cl, slot0:slot0 + n, h, 1], V, w.dtype), (b, h, "V")
    # nothing else written
    mask = np.ones(got.shape, bool)
    mask[:, layer, cl, slot0:slot0 + n] = False
    assert (got[mask] == SENTINEL).all()


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append(device, dtype, d):
    B, D, N, H, n_new = 4, 2, 50, 3, 5
    rng = np.random.default_rng(3)
    k = rng.standard_normal((B, n_new, H, d)).astype(np.float32)
    v = rng.standard_normal((B, n_new, H, d)).astype(np.float32)
    start = np.array([0, 47, -2, 60], np.int32)       # ragged, past the end, before 0
    say(f"[kv append] {dtype} d={d} start={start.tolist()}")
    cache = new_cache(dtype, B, D, 1, N, H, d, device)
    rope = L.lla_kv_rope_table_fill(cache).to(device)
    L.lla_kv_append(cache, 1, 0, torch.from_numpy(k).to(device), torch.from_numpy(v).to(device),
                    torch.from_numpy(start).to(device), rope)
    torch.cuda.synchronize()
    got = from_device(cache.tensor)                   # [B, D, 1, N, H, 2, d]
    written = np.zeros(got.shape, bool)
    for b in range(B):
        for j in range(n_new):
            p = int(start[b]) + j
            if not 0 <= p < N:
                continue
            written[b, 1, 0, p] = True
            K, V = O.cache_rows(k[b, j], v[b, j], np.full(H, p))
            assert rows_close(got[b, 1, 0, p, :, 0], K, dtype), (b, j)
            Vw = V if dtype == "f32" else O.bf16_round(V)
            assert np.array_equal(got[b, 1, 0, p, :, 1], Vw), (b, j)   # values: one rounding
    assert (got[~written] == SENTINEL).all()


# ----------------------------------------------------------- flash-decode
DECODE_CASES = [
    # dtype, B, D, L, N, H, d, splits
    ("f32", 2, 1, 1, 128, 2, 64, 0),
    ("f32", 3, 2, 3, 300, 5, 128, 4),
    ("bf16", 4, 2, 4, 700, 16, 128, 0),
    ("bf16", 3, 2, 2, 333, 3, 128, 5),          # heads fewer than one group covers
    ("bf16", 2, 1, 1, 257, 20, 64, 1),
    ("bf16", 2, 1, 1, 200, 4, 256, 3),
    ("bf16", 2, 1, 1, 96, 2, 32, 96),           # one split per slot
    ("bf16", 3, 1, 1, 1, 16, 128, 0),           # a single slot
]


@pytest.mark.parametrize("dtype,B,D,Lp,N,H,d,S", DECODE_CASES,
                         ids=[f"{c[0]}-d{c[6]}-H{c[5]}-S{c[7]}" for c in DECODE_CASES])
def test_decode(device, dtype, B, D, Lp, N, H, d, S):
    rng = np.random.default_rng(B * 1000 + N)
    layer, cl = D - 1, Lp - 1
    exact = gen.as_storage(rng.standard_normal((B, N, H, 2, d)), dtype)[1]
    pos = np.minimum(np.array([N - 1, 0, 1, N // 2][:B], np.int32), N - 1)
    # slots past each query hold values that would dominate any unmasked score
    for b in range(B):
        exact[b, pos[b] + 1:] = 24.0
    say(f"[kv decode] {dtype} B={B} N={N} H={H} d={d} splits={S} pos={pos.tolist()}")
    cache = new_cache(dtype, B, D, Lp, N, H, d, device, fill=-3.0)
    cache.tensor[:, layer, cl] = to_device(exact, dtype, device)
    rope = L.lla_kv_rope_table_fill(cache).to(device)
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    out = torch.empty((B, H, d), dtype=torch.float32, device=device)
    L.lla_kv_decode_attn(cache, layer, cl, torch.from_numpy(q).to(device),
                         torch.from_numpy(pos).to(device), rope, out,
                         L.kv_workspace(cache, S), n_splits=S)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = np.stack([np.stack([O.decode_cache(exact[b, :, h, 0], exact[b, :, h, 1], q[b, h],
                                             int(pos[b])) for h in range(H)])
                    for b in range(B)])
    err = row_rel_l2(got, ref).max()
    say(f"  max row rel L2 {err:.3e}")
    assert err <= TOL[dtype]


def test_decode_scale_and_pos_clamp(device):
    B, N, H, d = 2, 64, 2, 128
    rng = np.random.default_rng(5)
    exact = gen.as_storage(rng.standard_normal((B, N, H, 2, d)), "bf16")[1]
    cache = new_cache("bf16", B, 1, 1, N, H, d, device)
    cache.tensor[:, 0, 0] = to_device(exact, "bf16", device)
    rope = L.lla_kv_rope_table_fill(cache).to(device)
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    out = torch.empty((B, H, d), dtype=torch.float32, device=device)
    pos = np.array([-5, 1000], np.int32)              # clamped to 0 and N-1
    L.lla_kv_decode_attn(cache, 0, 0, torch.from_numpy(q).to(device),
                         torch.from_numpy(pos).to(device), rope, out, L.kv_workspace(cache),
                         softmax_scale=0.3)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for b, p in enumerate([0, N - 1]):
        ref = np.stack([O.decode_cache(exact[b, :, h, 0], exact[b, :, h, 1], q[b, h], p, 0.3)
                        for h in range(H)])
        assert row_rel_l2(got[b], ref).max() <= TOL["bf16"]


# --------------------------------------------- the two serving paths, end to end
@pytest.mark.parametrize("tmpl,kw", [
    ("extreme_batch_b768_ctx4k", dict(B=3, D=2, N=400)),
    ("lla2d_b256_ctx4k", dict(B=2, D=2, N=200)),
    ("tiny_fp32", dict(B=2, N=128)),
], ids=["per_head", "lla2d", "fp32"])
def test_fast_path_matches_lla(device, tmpl, kw):
    """Fill every loop's cache from the latent store, then flash-decode:
    the outputs are those of LLA decode (the oracle's), loop by loop."""
    w = WORKLOADS[tmpl].scaled(**kw)
    layer = w.D - 1
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    codec = Codec(w)
    cache = new_cache(w.dtype, w.B, w.D, w.T, w.N, w.H, w.d, device)
    pos = np.array([w.N - 1, 17, 0][:w.B], np.int32)
    d_pos = torch.from_numpy(pos).to(device)
    ws = L.kv_workspace(cache)
    for t in range(w.T):
        say(f"[fast path] {w.name} loop {t}")
        inp = DecodeInputs(w, codec, layer, t, device)
        L.lla_kv_fill_from_store(store, layer, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv, 0, w.N,
                                 rope, cache, t)
        out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=device)
        L.lla_kv_decode_attn(cache, layer, t, inp.d_q, d_pos, rope, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = np.stack([inp.oracle(vals[b, layer, :, :, :w.r_k], vals[b, layer, :, :, w.r_k:], b,
                                   pos[b]) for b in range(w.B)])
        err = row_rel_l2(got, ref).max()
        say(f"  max row rel L2 vs LLA oracle {err:.3e}")
        assert err <= TOL[w.dtype]


def test_final_loop_control(device):
    """Cache the final loop's K/V only (raw append of every slot), then let
    the query of every loop attend them."""
    B, N, H, d, T = 3, 160, 4, 128, 4
    rng = np.random.default_rng(11)
    k_last = rng.standard_normal((B, N, H, d)).astype(np.float32)
    v_last = rng.standard_normal((B, N, H, d)).astype(np.float32)
    cache = new_cache("bf16", B, 1, 1, N, H, d, device)
    rope = L.lla_kv_rope_table_fill(cache).to(device)
    L.lla_kv_append(cache, 0, 0, torch.from_numpy(k_last).to(device),
                    torch.from_numpy(v_last).to(device),
                    torch.zeros(B, dtype=torch.int32, device=device), rope)
    stored = from_device(cache.tensor)[:, 0, 0]                        # [B, N, H, 2, d]
    pos = np.array([N - 1, 63, 5], np.int32)
    for t in range(T):
        say(f"[final-loop control] loop {t}")
        q = rng.standard_normal((B, H, d)).astype(np.float32)
        out = torch.empty((B, H, d), dtype=torch.float32, device=device)
        L.lla_kv_decode_attn(cache, 0, 0, torch.from_numpy(q).to(device),
                             torch.from_numpy(pos).to(device), rope, out, L.kv_workspace(cache))
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for b in range(B):
            ref = np.stack([O.final_loop_control(k_last[b, :, h], v_last[b, :, h], q[b, h],
                                                 int(pos[b])) for h in range(H)])
            assert row_rel_l2(got[b], ref).max() <= TOL["bf16"]
            # and exactly the flash-decode of what the cache holds
            ref2 = np.stack([O.decode_cache(stored[b, :, h, 0], stored[b, :, h, 1], q[b, h],
                                            int(pos[b])) for h in range(H)])
            assert row_rel_l2(got[b], ref2).max() <= 1e-5


# ------------------------------------------------------------- full size
def test_decode_full_size_sampled(device):
    """The bench's fast-path call shape (32 sequences, 4096 slots, 16 heads,
    d = 128, bf16, automatic splits) on a device-filled cache; sampled
    sequences against the oracle."""
    B, N, H, d = 32, 4096, 16, 128
    key = gen.stream_key(77, 1)
    cache = L.KvCache("bf16", batch=B, layers=1, loops=1, max_ctx=N, heads=H, d_head=d,
                      device=device)
    fill_hash_normal(cache.tensor, key)
    rope = L.lla_kv_rope_table_fill(cache).to(device)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    pos = rng.integers(0, N, B).astype(np.int32)
    pos[:3] = [N - 1, 0, 2047]
    say(f"[kv decode full] B={B} N={N} splits={L.lla_kv_decode_auto_splits(cache)}")
    out = torch.empty((B, H, d), dtype=torch.float32, device=device)
    L.lla_kv_decode_attn(cache, 0, 0, torch.from_numpy(q).to(device),
                         torch.from_numpy(pos).to(device), rope, out, L.kv_workspace(cache))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    per_seq = N * H * 2 * d
    for b in [0, 1, 2, 17, 31]:
        slab = gen.hash_normal(key, b * per_seq, per_seq).reshape(N, H, 2, d)
        ref = np.stack([O.decode_cache(slab[:, h, 0], slab[:, h, 1], q[b, h], int(pos[b]))
                        for h in range(H)])
        err = row_rel_l2(got[b], ref).max()
        say(f"  b={b} pos={pos[b]}: {err:.3e}")
        assert err <= TOL["bf16"]
