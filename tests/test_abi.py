"""The C ABI on the CPU: the library loads, exports every entry point that
include/lla.h declares, and its host-only logic (sizes, offsets, exact
ratio, RoPE table, argument validation) is right.  No call here reaches a
kernel launch: every launching call is given arguments that fail host-side
validation first."""
import ctypes
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import looped_transformer_decode_amd as L
from oracle import lla_oracle as O
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lla2?d?_\w+)\s*\(", text)))


def store_for(w, data=None):
    return L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                         d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(L.lla.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_sizes_match_oracle(name):
    w = WORKLOADS[name]
    s = store_for(w)
    assert L.lla_store_bytes(s) == w.store_bytes
    elems = O.latent_store_scalars(w.D, w.N, w.store_heads, w.r_k, w.r_v) * w.B
    assert L.lla_store_bytes(s) == elems * w.elt_bytes
    rho = O.compression_ratio(w.T, w.d, w.r_k, w.r_v, w.H, w.variant)
    assert L.lla_compression_ratio(s) == rho
    assert Fraction(O.teacher_cache_scalars(w.T, w.D, w.H, w.d, w.N) * w.B, elems) == rho


def test_extreme_batch_store_is_116_gb():
    w = WORKLOADS["extreme_batch_b768_ctx4k"]
    assert L.lla_store_bytes(store_for(w)) == 115_964_116_992
    assert L.lla_compression_ratio(store_for(w)) == Fraction(64, 3)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_offsets_match_oracle(name):
    w = WORKLOADS[name]
    s = store_for(w)
    rng = np.random.default_rng(0)
    for _ in range(200):
        idx = tuple(int(rng.integers(0, n)) for n in w.store_shape)
        assert L.lla_store_offset(s, *idx) == O.store_offset(w.store_shape, *idx)
    last = tuple(n - 1 for n in w.store_shape)
    assert L.lla_store_offset(s, *last) == math.prod(w.store_shape) - 1
    for bad in [(-1, 0, 0, 0, 0), (w.B, 0, 0, 0, 0), (0, w.D, 0, 0, 0), (0, 0, w.N, 0, 0),
                (0, 0, 0, w.store_heads, 0), (0, 0, 0, 0, w.R)]:
        assert L.lla_store_offset(s, *bad) == -1


def test_invalid_descriptors():
    base = dict(batch=2, layers=2, max_ctx=64, heads=4, d_head=16, loops=4, r_k=4, r_v=8)
    for k in base:
        bad = dict(base, **{k: 0})
        with pytest.raises(L.LlaError) as e:
            L.lla_store_check(L.LatentStore("per_head", "f32", **bad))
        assert e.value.status == 2
        assert L.lla_store_bytes(L.LatentStore("per_head", "f32", **bad)) == 0
    with pytest.raises(L.LlaError) as e:
        L.lla_store_check(L.LatentStore("per_head", "f32", **dict(base, d_head=15)))
    assert e.value.status == 2
    with pytest.raises(L.LlaError) as e:
        L.lla_store_check(L.LatentStore("per_head", 7, **base))
    assert e.value.status == 3
    with pytest.raises(L.LlaError) as e:
        L.lla_store_check(L.LatentStore(5, "f32", **base))
    assert e.value.status == 7
    with pytest.raises(L.LlaError) as e:
        L.lla_store_check(L.LatentStore("per_head", "f32", rope_base=1.0, **base))
    assert e.value.status == 4
    huge = dict(base, batch=2 ** 31 - 1, layers=2 ** 31 - 1, max_ctx=2 ** 31 - 1)
    with pytest.raises(L.LlaError) as e:
        L.lla_store_check(L.LatentStore("per_head", "f32", **huge))
    assert e.value.status == 9
    assert L.lla_store_bytes(L.LatentStore("per_head", "f32", **huge)) == 0


def test_status_strings():
    for i, name in enumerate(L.lla.STATUS):
        assert L.status_string(i).startswith(name)
    assert L.status_string(99) == "LLA_E_UNKNOWN"


def test_workspace_and_splits():
    w = WORKLOADS["extreme_batch_b768_ctx4k"]
    s = store_for(w)
    assert L.lla_decode_path(s) == "mfma"
    S = L.lla_decode_auto_splits(s)
    assert 1 <= S <= w.N // 256
    assert L.lla_decode_workspace_bytes(s, 0) == w.B * w.H * S * (w.r_v + 2) * 4
    assert L.lla_decode_workspace_bytes(s, 7) == w.B * w.H * 7 * (w.r_v + 2) * 4
    assert L.lla_decode_workspace_bytes(s, -1) == 0
    t = WORKLOADS["tiny_fp32"]
    assert L.lla_decode_path(store_for(t)) == "valu"
    s2 = store_for(WORKLOADS["lla2d_b256_ctx4k"])
    assert L.lla_decode_path(s2) == "mfma"
    assert L.lla_decode_auto_splits(s2) == 1      # B = 256: one workgroup per CU
    assert L.lla_decode_path(store_for(WORKLOADS["lla2d_b256_ctx4k"].scaled(H=4))) == "valu"


@pytest.mark.parametrize("d,N", [(64, 128), (128, 100)])
def test_rope_table(d, N):
    s = L.LatentStore("per_head", "bf16", batch=1, layers=1, max_ctx=N, heads=1, d_head=d,
                      loops=1, r_k=16, r_v=32)
    host = L.lla_rope_table_fill(s).numpy()
    assert host.size == L.lla_rope_table_bytes(s)
    f32 = host[:N * d * 4].view(np.float32).reshape(N, d // 2, 2)
    theta = O.rope_frequencies(d)
    ang = np.arange(N)[:, None] * theta[None, :]
    np.testing.assert_allclose(f32[..., 0], np.cos(ang), rtol=0, atol=1.2e-7)
    np.testing.assert_allclose(f32[..., 1], np.sin(ang), rtol=0, atol=1.2e-7)
    off = (N * d * 4 + 255) // 256 * 256
    tiles = (N + 31) // 32
    bf = host[off:off + tiles * 32 * d * 2].view(np.uint16).reshape(tiles, d // 16, 64, 8)
    vals = (bf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    t, st, lane, e = np.meshgrid(np.arange(tiles), np.arange(d // 16), np.arange(64),
                                 np.arange(8), indexing="ij")
    j = 32 * t + lane % 32
    i = 16 * st + 8 * (lane // 32) + e
    ii = np.where(i < d // 2, i, i - d // 2)
    want = np.where(i < d // 2, np.cos(j * theta[ii]), np.sin(j * theta[ii]))
    assert np.array_equal(vals, O.bf16_round(want))


def _args_for(w, device_like=1):
    """Fake non-null pointers: every call below fails validation before a
    launch, so they are never dereferenced."""
    return device_like


@pytest.mark.parametrize("fn", ["decode", "decode2d", "encode", "encode2d"])
def test_launching_calls_validate_first(fn):
    lib = L.lib()
    ph = L.LatentStore("per_head", "bf16", batch=2, layers=3, max_ctx=64, heads=16, d_head=128,
                       loops=4, r_k=16, r_v=32)
    d2 = L.LatentStore("2d", "bf16", batch=2, layers=3, max_ctx=64, heads=16, d_head=128,
                       loops=4, r_k=64, r_v=128)
    P = 4096  # stands for a device pointer; never dereferenced
    if fn.startswith("decode"):
        f = lib.lla_decode_attn if fn == "decode" else lib.lla2d_decode_attn
        good, other = (ph, d2) if fn == "decode" else (d2, ph)

        def call(store, layer=0, loop=0, ptrs=(P,) * 7, out=P, ws=P, ws_bytes=1 << 30,
                 n_splits=0, scale=0.0, data=True):
            dsc = store.desc()
            if data:
                dsc.data = P
            return f(ctypes.byref(dsc), layer, loop, *ptrs, scale, out, ws, ws_bytes,
                     n_splits, None)
        assert call(other) == 7
        assert call(good, data=False) == 1
        assert call(good, layer=3) == 4
        assert call(good, layer=-1) == 4
        assert call(good, loop=4) == 4
        assert call(good, ptrs=(None,) + (P,) * 6) == 1
        assert call(good, ptrs=(P,) * 6 + (None,)) == 1
        assert call(good, out=None) == 1
        assert call(good, ws=None) == 5
        assert call(good, ws_bytes=16) == 5
        assert call(good, n_splits=-1) == 4
        assert call(good, n_splits=65) == 4
        assert call(good, scale=float("nan")) == 4
        assert call(good, scale=float("inf")) == 4
        assert f(None, 0, 0, *(P,) * 7, 0.0, P, P, 1 << 30, 0, None) == 1
        # batch x heads beyond the kernels' 32-bit (query, head) rows
        wide = L.LatentStore("per_head" if fn == "decode" else "2d", "bf16", batch=1 << 17,
                             layers=1, max_ctx=1, heads=1 << 15, d_head=2, loops=1, r_k=2, r_v=2)
        assert call(wide) == 9
    else:
        f = lib.lla_encode_append if fn == "encode" else lib.lla2d_encode_append
        good, other = (ph, d2) if fn == "encode" else (d2, ph)

        def call(store, layer=0, ptrs=(P,) * 7, n_new=1, data=True):
            dsc = store.desc()
            if data:
                dsc.data = P
            return f(ctypes.byref(dsc), layer, *ptrs, n_new, None)
        assert call(other) == 7
        assert call(good, layer=3) == 4
        assert call(good, n_new=-1) == 4
        assert call(good, n_new=65) == 4
        assert call(good, n_new=0) == 0          # empty append: a no-op
        assert call(good, data=False) == 1
        assert call(good, ptrs=(P,) * 6 + (None,)) == 1
        assert call(good, ptrs=(None,) + (P,) * 6) == 1


# ------------------------------------------------------ uncompressed K/V cache
def kv_for(w, loops=None):
    return L.KvCache(w.dtype, batch=w.B, layers=w.D, loops=w.T if loops is None else loops,
                     max_ctx=w.N, heads=w.H, d_head=w.d)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_kv_cache_sizes(name):
    """The fast path's cache is the teacher cache (all T loops, K and V);
    the final-loop control's is 1/T of it, so at T = 4 it matches a 4x
    latent store."""
    w = WORKLOADS[name]
    full = L.lla_kv_cache_bytes(kv_for(w))
    assert full == O.teacher_cache_scalars(w.T, w.D, w.H, w.d, w.N) * w.B * w.elt_bytes
    assert L.lla_kv_cache_bytes(kv_for(w, 1)) * w.T == full
    assert Fraction(full, L.lla_store_bytes(store_for(w))) == L.lla_compression_ratio(
        store_for(w))


def test_kv_cache_extreme_batch_does_not_fit_one_gpu():
    w = WORKLOADS["extreme_batch_b768_ctx4k"]
    assert L.lla_kv_cache_bytes(kv_for(w)) == 2_473_901_162_496     # 2.47 TB > 288 GB
    assert L.lla_kv_cache_bytes(kv_for(WORKLOADS["bf16_b32_ctx4k"])) == 103_079_215_104


def test_kv_cache_invalid_descriptors():
    base = dict(batch=2, layers=2, loops=4, max_ctx=64, heads=4, d_head=16)
    for k in base:
        with pytest.raises(L.LlaError) as e:
            L.lla_kv_cache_check(L.KvCache("f32", **dict(base, **{k: 0})))
        assert e.value.status == 2
    with pytest.raises(L.LlaError) as e:
        L.lla_kv_cache_check(L.KvCache("f32", **dict(base, d_head=15)))
    assert e.value.status == 2
    with pytest.raises(L.LlaError) as e:
        L.lla_kv_cache_check(L.KvCache(9, **base))
    assert e.value.status == 3
    with pytest.raises(L.LlaError) as e:
        L.lla_kv_cache_check(L.KvCache("f32", rope_base=0.5, **base))
    assert e.value.status == 4
    huge = dict(base, batch=2 ** 31 - 1, layers=2 ** 31 - 1, max_ctx=2 ** 31 - 1)
    assert L.lla_kv_cache_bytes(L.KvCache("f32", **huge)) == 0


def test_kv_rope_table_is_the_store_table():
    s = L.LatentStore("per_head", "bf16", batch=1, layers=1, max_ctx=100, heads=1, d_head=128,
                      loops=1, r_k=16, r_v=32)
    c = L.KvCache("bf16", batch=1, layers=1, loops=1, max_ctx=100, heads=1, d_head=128)
    assert np.array_equal(L.lla_kv_rope_table_fill(c).numpy(), L.lla_rope_table_fill(s).numpy())


def test_kv_decode_splits_and_workspace():
    c = kv_for(WORKLOADS["bf16_b32_ctx4k"])
    S = L.lla_kv_decode_auto_splits(c)
    assert 1 <= S <= 4096 // 128
    assert L.lla_kv_decode_workspace_bytes(c, 0) == 32 * 16 * S * (128 + 2) * 4
    assert L.lla_kv_decode_workspace_bytes(c, 3) == 32 * 16 * 3 * 130 * 4
    odd = L.KvCache("bf16", batch=1, layers=1, loops=1, max_ctx=64, heads=2, d_head=40)
    assert L.lla_kv_decode_auto_splits(odd) == 0          # no kernel for d = 40
    assert L.lla_kv_decode_workspace_bytes(odd, 1) == 0


def test_kv_calls_validate_first():
    lib = L.lib()
    P = 4096  # stands for a device pointer; never dereferenced
    c = L.KvCache("bf16", batch=2, layers=3, loops=4, max_ctx=64, heads=16, d_head=128)
    s = L.LatentStore("per_head", "bf16", batch=2, layers=3, max_ctx=64, heads=16, d_head=128,
                      loops=4, r_k=16, r_v=32)

    def dec(cache=c, layer=0, cl=0, q=P, pos=P, rope=P, out=P, ws=P, ws_bytes=1 << 30,
            n_splits=0, scale=0.0, data=True):
        d = cache.desc()
        if data:
            d.data = P
        return lib.lla_kv_decode_attn(ctypes.byref(d), layer, cl, q, pos, rope, scale, out, ws,
                                      ws_bytes, n_splits, None)
    assert dec(data=False) == 1
    assert dec(q=None) == 1 and dec(pos=None) == 1 and dec(rope=None) == 1 and dec(out=None) == 1
    assert dec(layer=3) == 4 and dec(cl=4) == 4 and dec(cl=-1) == 4
    assert dec(n_splits=-1) == 4 and dec(n_splits=65) == 4
    assert dec(scale=float("nan")) == 4
    assert dec(ws=None) == 5 and dec(ws_bytes=8) == 5
    odd = L.KvCache("bf16", batch=2, layers=3, loops=4, max_ctx=64, heads=16, d_head=40)
    assert dec(cache=odd) == 6
    assert lib.lla_kv_decode_attn(None, 0, 0, P, P, P, 0.0, P, P, 1 << 30, 0, None) == 1
    wide = L.KvCache("bf16", batch=1 << 17, layers=1, loops=1, max_ctx=1, heads=1 << 15,
                     d_head=128)
    assert dec(cache=wide, n_splits=1) == 9   # 32-bit (b, h) rows

    def fill(store=s, cache=c, layer=0, slot0=0, n=8, cl=0, ptrs=(P,) * 4, rope=P, data=True):
        sd, cd = store.desc(), cache.desc()
        if data:
            sd.data, cd.data = P, P
        return lib.lla_kv_fill_from_store(ctypes.byref(sd), layer, *ptrs, slot0, n, rope,
                                          ctypes.byref(cd), cl, None)
    assert fill(layer=3) == 4 and fill(cl=4) == 4
    assert fill(slot0=-1) == 4 and fill(slot0=60, n=5) == 4 and fill(n=-1) == 4
    assert fill(n=0) == 0                                   # empty range: a no-op
    assert fill(data=False) == 1 and fill(ptrs=(P, P, P, None)) == 1 and fill(rope=None) == 1
    assert fill(cache=L.KvCache("f32", batch=2, layers=3, loops=4, max_ctx=64, heads=16,
                                d_head=128)) == 3
    assert fill(cache=L.KvCache("bf16", batch=2, layers=3, loops=4, max_ctx=32, heads=16,
                                d_head=128)) == 2

    def app(cache=c, layer=0, cl=0, k=P, v=P, start=P, n=1, rope=P, data=True):
        d = cache.desc()
        if data:
            d.data = P
        return lib.lla_kv_append(ctypes.byref(d), layer, cl, k, v, start, n, rope, None)
    assert app(layer=-1) == 4 and app(cl=4) == 4 and app(n=-1) == 4 and app(n=65) == 4
    assert app(n=0) == 0
    assert app(data=False) == 1 and app(k=None) == 1 and app(start=None) == 1


# --------------------------------------------------------- SVD initialisation
def test_svd_init_sizes_and_validation():
    lib = L.lib()
    P = 4096  # stands for a device pointer; never dereferenced
    assert L.lla_svd_init_workspace_bytes(16, 16, 128, 48) > 16 * 2048 * 2048 * 4
    assert L.lla_svd_init_workspace_bytes(0, 4, 128, 8) == 0
    assert L.lla_svd_init_workspace_bytes(1, 4, 8, 33) == 0       # r > K
    assert L.lla_svd_init_workspace_bytes(1, 4, 128, 129) == 0    # r above the block limit

    def call(dtype=1, G=2, n=100, T=4, width=32, r=8, x=P, mu=P, wd=P, wu=P, iters=0,
             ws=P, ws_bytes=1 << 40):
        return lib.lla_svd_init(dtype, G, n, T, width, r, x, mu, wd, wu, None, iters, ws,
                                ws_bytes, None)
    assert call(dtype=4) == 3
    assert call(G=0) == 2 and call(n=0) == 2 and call(T=0) == 2 and call(width=0) == 2
    assert call(r=0) == 4 and call(r=129, width=64) == 6 and call(r=200) == 4
    assert call(iters=-1) == 4
    assert call(x=None) == 1 and call(mu=None) == 1 and call(wd=None) == 1 and call(wu=None) == 1
    assert call(ws=None) == 5 and call(ws_bytes=1024) == 5
    assert call(G=70000) == 6
