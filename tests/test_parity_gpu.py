"""GPU parity: the HIP decode / encode path, called through the C ABI, against
the fp64 oracle on identical seeded inputs.

Bar (per output row out[b, h, :], relative L2): 1e-5 for float32 stores,
2e-2 for bfloat16 stores with float32 accumulation.  Encoded latents: every
value within half a bf16 ulp plus the float32 accumulation bound of the
oracle's exact value (two results are correct near a rounding tie), nearly
all bit-identical, and every slot outside the append bit-identical."""
import sys

import numpy as np
import pytest
import torch

import looped_transformer_decode_amd as L
from oracle import lla_oracle as O
from synth import gen
from synth.workloads import WORKLOADS, Codec
from tests.gpu_cases import (TOL, DecodeInputs, attn_rel_l2, device_slab, fill_store_on_device,
                             from_device, full_precision_slab, host_store, mu_rows, new_store,
                             put_slab, row_rel_l2, to_device)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, **kw):
    return WORKLOADS[name].scaled(**kw)


def decode_case(w, layer, t, pos, device, n_splits=0, tid=1, scale=0.0):
    """Host-generated store; returns (gpu [B,H,d], oracle [B,H,d], store path).
    Also checks the error of the softmax-dependent part, (out - mu_v,t),
    against the same bound."""
    say(f"[decode] {w.name} {w.variant} {w.dtype} B={w.B} N={w.N} H={w.H} rk={w.r_k} "
        f"rv={w.r_v} layer={layer} t={t} splits={n_splits}")
    vals = host_store(w, tid)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), layer, t, device)
    got = inp.run(store, pos, rope, n_splits=n_splits, scale=scale)
    ref = np.stack([inp.oracle(vals[b, layer, :, :, :w.r_k], vals[b, layer, :, :, w.r_k:], b,
                               pos[b], None if scale == 0.0 else scale)
                    for b in range(w.B)])
    check_attn_part(got, ref, mu_rows(inp, w), w.dtype)
    return got, ref, L.lla_decode_path(store)


def check_attn_part(got, ref, mu_v, dtype):
    """Print and bound the relative L2 of (out - mu_v,t) per row."""
    a = attn_rel_l2(got, ref, mu_v).max()
    say(f"  (out - mu_v,t) max row rel L2 {a:.3e}")
    assert a <= TOL[dtype], a


# ----------------------------------------------------------------- float32
def test_tiny_fp32_every_loop(device):
    w = WORKLOADS["tiny_fp32"]
    for t in range(w.T):
        got, ref, path = decode_case(w, 0, t, np.array([w.N - 1]), device)
        err = row_rel_l2(got, ref).max()
        say(f"  loop {t}: max row rel L2 {err:.3e} ({path})")
        assert err <= TOL["f32"]


def test_tiny_fp32_causal_sweep(device):
    """Every query position 0..N-1: the store holds the same latents for
    each of N sequences, and sequence b queries at position b."""
    w0 = WORKLOADS["tiny_fp32"]
    w = w0.scaled(B=w0.N)
    one = host_store(w0)
    vals = np.repeat(one, w.B, axis=0)
    store = new_store(w, device, tensor=to_device(vals, "f32", device))
    rope = L.rope_table(store, device)
    codec = Codec(w0)
    inp = DecodeInputs(w0, codec, 0, 1, device)
    inp.d_q = to_device(np.repeat(inp.q, w.B, axis=0), "f32", device)
    inp.w = w
    pos = np.arange(w.N)
    got = inp.run(store, pos, rope)
    ref = np.stack([O.decode(one[0, 0, :, :, :w.r_k], one[0, 0, :, :, w.r_k:], inp.q[0], inp.wk,
                             inp.wv, inp.mk, inp.mv, int(p)) for p in pos])
    err = row_rel_l2(got, ref)
    say(f"  causal sweep max {err.max():.3e}")
    assert err.max() <= TOL["f32"]
    # position 0 attends only slot 0: its output is that slot's value
    v0 = one[0, 0, 0, :, w.r_k:]
    assert np.abs(got[0] - (np.einsum("hdr,hr->hd", inp.wv, v0) + inp.mv)).max() < 1e-5


def test_fp32_encode_then_decode_exact_codec(device):
    """End to end on the GPU: an exact codec (r = T*d, orthonormal W_down,
    W_up,t = its loop-t slice) encodes a teacher cache; decoding it equals
    textbook RoPE attention over the teacher's own loop-t K/V."""
    T, d, H, N, B = 2, 64, 2, 96, 2
    r = T * d
    w = WORKLOADS["tiny_fp32"].scaled(T=T, d=d, H=H, N=N, B=B, r_k=r, r_v=r)
    rng = np.random.default_rng(11)
    K = rng.standard_normal((B, N, T, H, d)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((B, N, T, H, d)).astype(np.float32).astype(np.float64)
    Q = {a: np.stack([np.linalg.qr(rng.standard_normal((r, r)))[0] for _ in range(H)])
         .astype(np.float32).astype(np.float64) for a in "kv"}
    mu = {a: (rng.standard_normal((H, r)) * 0.2).astype(np.float32).astype(np.float64)
          for a in "kv"}
    store = new_store(w, device)
    store.tensor.fill_(float("nan"))
    xk = to_device(K.transpose(0, 1, 3, 2, 4).reshape(B, N, H, r), "f32", device)
    xv = to_device(V.transpose(0, 1, 3, 2, 4).reshape(B, N, H, r), "f32", device)
    start = torch.zeros(B, dtype=torch.int32, device=device)
    L.lla_encode_append(store, 0, xk, xv, to_device(mu["k"], "f32", device),
                        to_device(mu["v"], "f32", device), to_device(Q["k"], "f32", device),
                        to_device(Q["v"], "f32", device), start)
    torch.cuda.synchronize()
    lat = from_device(store.tensor)
    for b in range(B):
        for h in range(H):
            for a, X, off in (("k", K, 0), ("v", V, r)):
                want = O.encode(O.stack_loops(X[b, :, :, h]), mu[a][h], Q[a][h])
                np.testing.assert_allclose(lat[b, 0, :, h, off:off + r], want, rtol=0,
                                           atol=2e-5 * (1 + np.abs(want).max()))
    rope = L.rope_table(store, device)
    pos = np.array([N - 1, 37])
    q = rng.standard_normal((B, H, d)).astype(np.float32).astype(np.float64)
    for t in range(T):
        sl = slice(t * d, (t + 1) * d)
        out = torch.empty((B, H, d), device=device)
        L.lla_decode_attn(store, 0, t, to_device(q, "f32", device),
                          to_device(Q["k"][:, sl, :], "f32", device),
                          to_device(Q["v"][:, sl, :], "f32", device),
                          to_device(mu["k"][:, sl], "f32", device),
                          to_device(mu["v"][:, sl], "f32", device),
                          torch.from_numpy(pos.astype(np.int32)).to(device), rope, out,
                          L.workspace(store))
        got = out.cpu().numpy().astype(np.float64)
        for b in range(B):
            p = pos[b]
            for h in range(H):
                Kt = O.rope(K[b, :p + 1, t, h], np.arange(p + 1))
                s = Kt @ O.rope(q[b, h], p) / np.sqrt(d)
                e = np.exp(s - s.max())
                ref = (e / e.sum()) @ V[b, :p + 1, t, h]
                err = np.linalg.norm(got[b, h] - ref) / np.linalg.norm(ref)
                assert err <= TOL["f32"], (t, b, h, err)


# ----------------------------------------------------------------- bf16, small
BF16_SHAPES = [
    # (workload template, overrides): several tiles and a ragged tail
    ("extreme_batch_b768_ctx4k", dict(B=3, D=2, N=300)),
    ("lla2d_b256_ctx4k", dict(B=3, D=2, N=1100)),                 # several splits of 256+
    ("bf16_b32_ctx4k", dict(B=3, D=2, N=200, H=8)),
    ("long_recurrence_t16_ctx8k", dict(B=2, D=2, N=260, H=8)),
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=160, d=64)),   # generic (VALU) bf16 path
    ("lla2d_b256_ctx4k", dict(B=2, D=2, N=170)),
    # two head groups per sequence on the fast path (16, 8 and 8 heads per workgroup)
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=130, H=32)),
    ("bf16_b32_ctx4k", dict(B=2, D=1, N=100, H=16)),
    ("long_recurrence_t16_ctx8k", dict(B=2, D=1, N=90, H=16)),
]


@pytest.mark.parametrize("tmpl,kw", BF16_SHAPES,
                         ids=[f"{t}-{'-'.join(f'{k}{v}' for k, v in kw.items())}"
                              for t, kw in BF16_SHAPES])
def test_bf16_small_vs_oracle(device, tmpl, kw):
    w = small(tmpl, **kw)
    pos = np.array([w.N - 1, 0, 117][:w.B])
    # 11 splits: the merges read partials in batches of 8, so this takes two
    # batches, the later splits of the short sequences empty
    for n_splits in (1, 3, 11, 0):
        got, ref, path = decode_case(w, w.D - 1, w.T - 1, pos, device, n_splits=n_splits)
        err = row_rel_l2(got, ref)
        say(f"  path={path} splits={n_splits} max row rel L2 {err.max():.3e}")
        assert err.max() <= TOL["bf16"]
        assert np.isfinite(got).all()


def test_mfma_path_is_selected_for_paper_shapes():
    for name in ("bf16_b32_ctx4k", "extreme_batch_b768_ctx4k", "long_recurrence_t16_ctx8k",
                 "lla2d_b256_ctx4k"):
        w = WORKLOADS[name]
        s = L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                          d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v)
        assert L.lla_decode_path(s) == "mfma", name


def test_loop_index_does_not_change_rope(device):
    """The rotary phase is shared by all loops: with the same W_up,t and
    mu_t, the loop argument must not change a single bit of the output."""
    w = small("extreme_batch_b768_ctx4k", B=2, D=1, N=96)
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), 0, 0, device)
    pos = np.array([95, 50])
    outs = [inp.run(store, pos, rope, loop=t) for t in range(w.T)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_positions_are_clamped(device):
    w = small("extreme_batch_b768_ctx4k", B=2, D=1, N=64)
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), 0, 1, device)
    a = inp.run(store, np.array([63, 0]), rope)
    b = inp.run(store, np.array([10_000, -7]), rope)
    assert np.array_equal(a, b)


def test_explicit_softmax_scale(device):
    w = small("extreme_batch_b768_ctx4k", B=2, D=1, N=128)
    got, ref, _ = decode_case(w, 0, 2, np.array([127, 64]), device, scale=0.05)
    assert row_rel_l2(got, ref).max() <= TOL["bf16"]


@pytest.mark.parametrize("tmpl", ["extreme_batch_b768_ctx4k", "lla2d_b256_ctx4k"])
def test_garbage_beyond_pos_is_ignored(device, tmpl):
    """Slots after pos hold NaN: nothing of them may leak into the output."""
    w = small(tmpl, B=2, D=1, N=200)
    vals = host_store(w)
    dev_vals = to_device(vals, w.dtype, device)
    dev_vals[:, :, 150:] = float("nan")
    store = new_store(w, device, tensor=dev_vals)
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), 0, 0, device)
    pos = np.array([149, 31])
    got = inp.run(store, pos, rope)
    ref = np.stack([inp.oracle(vals[b, 0, :, :, :w.r_k], vals[b, 0, :, :, w.r_k:], b, pos[b])
                    for b in range(w.B)])
    assert np.isfinite(got).all()
    assert row_rel_l2(got, ref).max() <= TOL["bf16"]


# ----------------------------------------------------------------- in-flight
INFLIGHT_SHAPES = [
    ("long_recurrence_t16_ctx8k", dict(B=2, D=2, N=300, H=8), 16),   # fast path, n_q = 16
    ("extreme_batch_b768_ctx4k", dict(B=3, D=1, N=200), 4),
    ("bf16_b32_ctx4k", dict(B=2, D=1, N=260, H=6), 7),                # heads not a multiple of 4
    ("tiny_fp32", dict(B=3, N=128), 3),                              # generic fp32 path
    ("lla2d_b256_ctx4k", dict(B=2, D=1, N=170), 4),                  # LLA-2D fast path
    ("tiny_fp32", dict(B=2, N=128, d=96), 5),                        # d not dividing the block
    ("bf16_b32_ctx4k", dict(B=2, D=1, N=200, H=2), 32),              # most queries: 4 groups of 8
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=150), 20),         # single-query fast path per query
]


def inflight_case(w, n_q, pos0, device, n_splits=0, layer=None):
    """Returns (gpu [B, n_q, H, d], oracle [B, n_q, H, d])."""
    layer = w.D - 1 if layer is None else layer
    t = w.T - 1
    say(f"[inflight] {w.name} {w.variant} {w.dtype} B={w.B} N={w.N} H={w.H} n_q={n_q} "
        f"pos0={list(pos0)} splits={n_splits}")
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), layer, t, device)
    rng = np.random.default_rng(w.seed + 77)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    q = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    kn = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    vn = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    out = torch.empty((w.B, n_q, w.H, w.d), dtype=torch.float32, device=device)
    ws = L.workspace(store, n_splits, n_q=n_q)
    L.lla_decode_attn_inflight(store, layer, t, to_device(q, "f32", device),
                               to_device(kn, "f32", device), to_device(vn, "f32", device),
                               inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv,
                               torch.from_numpy(np.asarray(pos0, np.int32)).to(device), rope, out,
                               ws, n_splits=n_splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    is2d = w.variant == "2d"
    ref = np.stack([O.decode_inflight(vals[b, layer, :, :, :w.r_k], vals[b, layer, :, :, w.r_k:],
                                      q[b], kn[b], vn[b], inp.wk.reshape(-1, w.r_k) if is2d
                                      else inp.wk, inp.wv.reshape(-1, w.r_v) if is2d else inp.wv,
                                      inp.mk.reshape(-1) if is2d else inp.mk,
                                      inp.mv.reshape(-1) if is2d else inp.mv, int(pos0[b]),
                                      variant=w.variant) for b in range(w.B)])
    check_attn_part(got, ref, mu_rows(inp, w), w.dtype)
    return got, ref


@pytest.mark.parametrize("tmpl,kw,n_q", INFLIGHT_SHAPES,
                         ids=[f"{t}-nq{n}" for t, _, n in INFLIGHT_SHAPES])
def test_inflight_vs_oracle(device, tmpl, kw, n_q):
    w = small(tmpl, **kw)
    pos0 = np.array([w.N - n_q, 0, 57][:w.B])
    for n_splits in (1, 3, 11, 0):
        got, ref = inflight_case(w, n_q, pos0, device, n_splits=n_splits)
        err = row_rel_l2(got, ref)
        say(f"  splits={n_splits} max row rel L2 {err.max():.3e}")
        assert err.max() <= TOL[w.dtype]
        assert np.isfinite(got).all()


def test_inflight_single_query_matches_decode(device):
    """One in-flight token whose key/value are the exact reconstruction of
    the latent at slot pos0 = the store-only decode at pos0 (same kernels'
    store part, different assembly)."""
    w = small("extreme_batch_b768_ctx4k", B=2, D=1, N=160)
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), 0, 1, device)
    pos = np.array([159, 40])
    want = inp.run(store, pos, rope)
    ck = vals[np.arange(w.B), 0, pos][:, :, :w.r_k]                 # [B, H, r_k]
    cv = vals[np.arange(w.B), 0, pos][:, :, w.r_k:]
    kn = np.einsum("hdr,bhr->bhd", inp.wk, ck) + inp.mk[None]
    vn = np.einsum("hdr,bhr->bhd", inp.wv, cv) + inp.mv[None]
    out = torch.empty((w.B, 1, w.H, w.d), dtype=torch.float32, device=device)
    L.lla_decode_attn_inflight(store, 0, 1, inp.d_q[:, None].contiguous(),
                               to_device(kn[:, None], "f32", device),
                               to_device(vn[:, None], "f32", device), inp.d_wk, inp.d_wv,
                               inp.d_mk, inp.d_mv,
                               torch.from_numpy(pos.astype(np.int32)).to(device), rope, out,
                               L.workspace(store, n_q=1))
    torch.cuda.synchronize()
    got = out.cpu().numpy()[:, 0].astype(np.float64)
    assert row_rel_l2(got, want).max() <= TOL["bf16"]


def test_inflight_full_size_sampled(device):
    """Long-recurrence shape at full size (B=64, N=8192, T=16) with the
    step's 16 appended tokens in flight, launched as the benchmark launches
    it; sampled sequences against the oracle on slabs regenerated on the host."""
    w = WORKLOADS["long_recurrence_t16_ctx8k"]
    n_q = w.n_new
    say(f"[inflight full] {w.name}: n_q={n_q}")
    torch.cuda.empty_cache()
    store = new_store(w, device)
    fill_store_on_device(w, store)
    rope = L.rope_table(store, device)
    layer, t = w.D - 1, w.T - 1
    # the sampled sequences get full-precision N(0, 1) latents from the host
    samples = sorted({0, 1, w.B - 1})
    slabs = {b: full_precision_slab(w, b, layer) for b in samples}
    for b in samples:
        put_slab(store, w, b, layer, slabs[b])
    inp = DecodeInputs(w, Codec(w), layer, t, device)
    rng = np.random.default_rng(w.seed + 78)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    q = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    kn = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    vn = f32(rng.standard_normal((w.B, n_q, w.H, w.d)))
    pos0 = np.full(w.B, w.N - n_q)
    pos0[1::3] = rng.integers(0, w.N - n_q, size=len(pos0[1::3]))
    out = torch.empty((w.B, n_q, w.H, w.d), dtype=torch.float32, device=device)
    L.lla_decode_attn_inflight(store, layer, t, to_device(q, "f32", device),
                               to_device(kn, "f32", device), to_device(vn, "f32", device),
                               inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv,
                               torch.from_numpy(pos0.astype(np.int32)).to(device), rope, out,
                               L.workspace(store, n_q=n_q))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    worst = worst_attn = 0.0
    for b in samples:
        ck, cv = slabs[b][..., :w.r_k], slabs[b][..., w.r_k:]
        ref = O.decode_inflight(ck, cv, q[b], kn[b], vn[b], inp.wk, inp.wv, inp.mk, inp.mv,
                                int(pos0[b]))
        err = row_rel_l2(got[b], ref).max()
        ea = attn_rel_l2(got[b], ref, mu_rows(inp, w)).max()
        worst, worst_attn = max(worst, err), max(worst_attn, ea)
        say(f"  b={b} pos0={pos0[b]} max row rel L2 {err:.3e}; (out - mu_v,t) {ea:.3e}")
    assert worst <= TOL["bf16"] and worst_attn <= TOL["bf16"]
    del store
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- encode
ENCODE_SHAPES = [
    ("extreme_batch_b768_ctx4k", dict(B=5, D=2, N=64)),
    ("long_recurrence_t16_ctx8k", dict(B=3, D=2, N=64, H=4)),
    ("lla2d_b256_ctx4k", dict(B=3, D=2, N=32, H=4)),
    ("tiny_fp32", dict(B=3, N=64)),
    # enough rows for two 16-row tiles per wave and several row blocks
    ("extreme_batch_b768_ctx4k", dict(B=260, D=2, N=16)),
    ("bf16_b32_ctx4k", dict(B=70, D=2, N=16, H=4, T=1)),
    # enough row blocks for the LDS-ring form: K = 2048 (32 chunks), and
    # K = 128 (two chunks, fewer than the ring holds); ragged last blocks
    ("long_recurrence_t16_ctx8k", dict(B=104, D=2, N=24)),
    ("bf16_b32_ctx4k", dict(B=78, D=2, N=16, T=1)),
    # 33 row blocks x 2 heads x 2 axes = 132 workgroups, not a multiple of the
    # eight XCDs: the plain workgroup numbering
    ("extreme_batch_b768_ctx4k", dict(B=821, D=2, N=8, H=2)),
]


def check_latents(got, want, dtype, K):
    """Stored latents vs the oracle's exact value (rounded once by the GPU).
    Returns the number of values that differ from the oracle's own rounding
    (a float32 accumulation near a bf16 rounding tie may round the other
    way; both results are correct)."""
    if dtype == "f32":
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * (1 + np.abs(want).max()))
        return 0
    _, e = np.frexp(want)
    half_ulp = np.ldexp(1.0, np.maximum(e, -125) - 9)
    acc_bound = 4 * K * 2.0 ** -24 * (1 + np.abs(want))
    assert (np.abs(got - want) <= half_ulp + acc_bound).all()
    return int(np.sum(got != O.bf16_round(want)))


@pytest.mark.parametrize("tmpl,kw", ENCODE_SHAPES,
                         ids=[f"{t}-{'-'.join(f'{k}{v}' for k, v in kw.items())}"
                              for t, kw in ENCODE_SHAPES])
def test_encode_vs_oracle(device, tmpl, kw):
    w = small(tmpl, **kw)
    n_new = 5
    say(f"[encode] {w.name} {w.variant} {w.dtype} B={w.B} N={w.N} H={w.H} T={w.T}")
    codec = Codec(w)
    layer = w.D - 1
    start = np.array([0, w.N - n_new, w.N - 2, 17, 40][:w.B], dtype=np.int32)  # one overflows
    if w.B > 5:
        start = np.resize(start % max(1, w.N - n_new + 1), w.B).astype(np.int32)
        start[2] = w.N - 2
    sentinel = from_device(to_device(np.full(1, 3.0), w.dtype, device))[0]
    store = new_store(w, device)
    store.tensor.fill_(sentinel)
    x = {a: codec.x(a, layer, w.B * n_new) for a in "kv"}      # [rows, codec_rows, K]
    mu = {a: codec.mu(a, layer) for a in "kv"}
    wd = {a: codec.w_down(a, layer) for a in "kv"}
    K = w.T * w.width
    if w.variant == "2d":
        args = [to_device(x[a].reshape(w.B, n_new, K), w.dtype, device) for a in "kv"]
        args += [to_device(mu[a][0], "f32", device) for a in "kv"]
        args += [to_device(wd[a][0], w.dtype, device) for a in "kv"]
        fn = L.lla2d_encode_append
    else:
        args = [to_device(x[a].reshape(w.B, n_new, w.H, K), w.dtype, device) for a in "kv"]
        args += [to_device(mu[a], "f32", device) for a in "kv"]
        args += [to_device(wd[a], w.dtype, device) for a in "kv"]
        fn = L.lla_encode_append
    fn(store, layer, *args, torch.from_numpy(start).to(device))
    torch.cuda.synchronize()
    got = from_device(store.tensor)
    written = np.zeros(w.store_shape[:3], bool)
    want = {a: np.stack([O.encode(x[a][:, h], mu[a][h], wd[a][h]) for h in range(w.store_heads)],
                        axis=1) for a in "kv"}                 # [rows, H', r]
    flips, total = 0, 0
    for b in range(w.B):
        for j in range(n_new):
            slot = start[b] + j
            if not 0 <= slot < w.N:
                continue
            written[b, layer, slot] = True
            row = b * n_new + j
            for a, off, r in (("k", 0, w.r_k), ("v", w.r_k, w.r_v)):
                flips += check_latents(got[b, layer, slot, :, off:off + r], want[a][row], w.dtype,
                                       K)
                total += r * w.store_heads
    say(f"  {total} latents, {flips} rounded the other way at a tie")
    assert flips <= 0.02 * total
    assert (got[~written] == sentinel).all()


@pytest.mark.parametrize("name", ["extreme_batch_b768_ctx4k", "long_recurrence_t16_ctx8k",
                                  "lla2d_b256_ctx4k", "bf16_b32_ctx4k"])
def test_encode_full_size(device, name):
    """The append of one benchmark step at full size (all sequences, all
    heads, the step's n_new tokens) into a full-size store, as the benchmark
    launches it: every written latent against the oracle, and the slots on
    either side of each append untouched."""
    w = WORKLOADS[name]
    n_new = w.n_new
    say(f"[encode full] {name}: B={w.B} n_new={n_new} H'={w.store_heads} K={w.T * w.width}")
    torch.cuda.empty_cache()
    codec = Codec(w)
    layer = 1
    K = w.T * w.width
    rng = np.random.default_rng(w.seed + 5)
    start = rng.integers(1, w.N - n_new, size=w.B).astype(np.int32)
    start[0] = w.N - n_new - 1
    start[-1] = 1
    sentinel = from_device(to_device(np.full(1, 3.0), w.dtype, device))[0]
    store = new_store(w, device)
    store.tensor[:, layer].fill_(sentinel)
    x = {a: codec.x(a, layer, w.B * n_new) for a in "kv"}
    mu = {a: codec.mu(a, layer) for a in "kv"}
    wd = {a: codec.w_down(a, layer) for a in "kv"}
    if w.variant == "2d":
        args = [to_device(x[a].reshape(w.B, n_new, K), w.dtype, device) for a in "kv"]
        args += [to_device(mu[a][0], "f32", device) for a in "kv"]
        args += [to_device(wd[a][0], w.dtype, device) for a in "kv"]
        fn = L.lla2d_encode_append
    else:
        args = [to_device(x[a].reshape(w.B, n_new, w.H, K), w.dtype, device) for a in "kv"]
        args += [to_device(mu[a], "f32", device) for a in "kv"]
        args += [to_device(wd[a], w.dtype, device) for a in "kv"]
        fn = L.lla_encode_append
    fn(store, layer, *args, torch.from_numpy(start).to(device))
    torch.cuda.synchronize()
    b_idx = torch.arange(w.B, device=device).repeat_interleave(n_new)
    s_idx = (torch.from_numpy(start).to(device).long().repeat_interleave(n_new)
             + torch.arange(n_new, device=device).repeat(w.B))
    got = from_device(store.tensor[b_idx, layer, s_idx])            # [rows, H', R]
    b_all = torch.arange(w.B, device=device)
    st = torch.from_numpy(start).to(device).long()
    before = from_device(store.tensor[b_all, layer, st - 1])
    after = from_device(store.tensor[b_all, layer, st + n_new])
    assert (before == sentinel).all() and (after == sentinel).all()
    flips, total = 0, 0
    for a, off, r in (("k", 0, w.r_k), ("v", w.r_k, w.r_v)):
        for h in range(w.store_heads):
            want = O.encode(x[a][:, h], mu[a][h], wd[a][h])           # [rows, r]
            flips += check_latents(got[:, h, off:off + r], want, w.dtype, K)
            total += want.size
    say(f"  {total} latents, {flips} rounded the other way at a tie")
    assert flips <= 0.02 * total
    del store
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- full size
FULL = ["bf16_b32_ctx4k", "extreme_batch_b768_ctx4k", "lla2d_b256_ctx4k",
        "long_recurrence_t16_ctx8k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(device, name):
    """The full configuration, launched as the benchmark launches it
    (automatic split count), the store filled on the device with the
    counter-based generator; sampled sequences are checked against the
    oracle on slabs regenerated on the host."""
    w = WORKLOADS[name]
    say(f"[full] {name}: store {w.store_bytes / 1e9:.1f} GB")
    torch.cuda.empty_cache()
    store = new_store(w, device)
    fill_store_on_device(w, store)
    rope = L.rope_table(store, device)
    layer, t = w.D - 1, w.T - 1
    inp = DecodeInputs(w, Codec(w), layer, t, device)
    rng = np.random.default_rng(w.seed)
    pos = np.full(w.B, w.N - 1)
    pos[1::3] = rng.integers(0, w.N, size=len(pos[1::3]))
    samples = sorted({0, 1, w.B - 1, int(rng.integers(0, w.B))})
    # half of the sampled sequences hold full-precision N(0, 1) latents from
    # the host (full mantissas and tails), the rest the device filler's values
    host = {b: full_precision_slab(w, b, layer) for b in samples[::2]}
    for b, v in host.items():
        put_slab(store, w, b, layer, v)
    got = inp.run(store, pos, rope)
    worst = worst_attn = 0.0
    for b in samples:
        if b in host:
            ck, cv = host[b][..., :w.r_k], host[b][..., w.r_k:]
        else:
            ck, cv = device_slab(w, b, layer)
        ref = inp.oracle(ck, cv, b, pos[b])
        err = row_rel_l2(got[b], ref).max()
        ea = attn_rel_l2(got[b], ref, mu_rows(inp, w)).max()
        worst, worst_attn = max(worst, err), max(worst_attn, ea)
        say(f"  b={b} pos={pos[b]} ({'host N(0,1)' if b in host else 'device filler'}) "
            f"max row rel L2 {err:.3e}; (out - mu_v,t) {ea:.3e}")
    assert worst <= TOL["bf16"] and worst_attn <= TOL["bf16"]
    assert np.isfinite(got).all()
    del store
    torch.cuda.empty_cache()


def test_device_fill_matches_host_generator(device):
    from synth.device import fill_hash_normal
    key = gen.stream_key(7, 3)
    t16 = torch.empty(100_003, dtype=torch.bfloat16, device=device)
    fill_hash_normal(t16, key, first=2 ** 33)
    want = gen.hash_normal(key, 2 ** 33, t16.numel())
    assert np.array_equal(from_device(t16), want)
    t32 = torch.empty(4097, dtype=torch.float32, device=device)
    fill_hash_normal(t32, key, first=5, scale=0.1)
    want32 = (gen.hash_normal(key, 5, 4097).astype(np.float32) * np.float32(0.1))
    assert np.array_equal(t32.cpu().numpy(), want32)


# ------------------------------------------------------------ degenerate sizes
@pytest.mark.parametrize("tmpl,kw", [
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=1)),     # one slot: out = v_hat_0
    ("extreme_batch_b768_ctx4k", dict(B=1, D=1, N=33)),    # one full tile + one slot
    ("long_recurrence_t16_ctx8k", dict(B=1, D=1, N=1)),
    ("lla2d_b256_ctx4k", dict(B=1, D=1, N=1)),
    ("lla2d_b256_ctx4k", dict(B=2, D=1, N=33)),
    ("tiny_fp32", dict(B=1, N=1)),
], ids=["per_head_N1", "per_head_N33", "long_rec_N1", "lla2d_N1", "lla2d_N33", "fp32_N1"])
def test_smallest_stores(device, tmpl, kw):
    """Stores of one slot (the query attends only itself) and of one tile plus
    one slot, at every query position, on the paths the shapes select."""
    w = small(tmpl, **kw)
    for p0 in sorted({0, w.N - 1, w.N // 2}):
        got, ref, path = decode_case(w, w.D - 1, w.T - 1, np.full(w.B, p0), device)
        err = row_rel_l2(got, ref).max()
        say(f"  pos {p0} ({path}): max row rel L2 {err:.3e}")
        assert err <= TOL[w.dtype]


@pytest.mark.parametrize("tmpl,kw,n_q,pos0", [
    ("long_recurrence_t16_ctx8k", dict(B=2, D=1, N=20, H=4), 16, [4, 0]),
    ("extreme_batch_b768_ctx4k", dict(B=2, D=1, N=16), 16, [0, 0]),
    ("lla2d_b256_ctx4k", dict(B=1, D=1, N=18), 16, [2]),
], ids=["store_of_four", "empty_store", "lla2d_store_of_two"])
def test_inflight_short_stores(device, tmpl, kw, n_q, pos0):
    """In-flight tokens that fill the context up to its last slot, over
    stores of a few slots or none."""
    w = small(tmpl, **kw)
    got, ref = inflight_case(w, n_q, np.array(pos0), device)
    err = row_rel_l2(got, ref)
    say(f"  max row rel L2 {err.max():.3e}")
    assert err.max() <= TOL[w.dtype]
