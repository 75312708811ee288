"""GPU: the decode and encode calls captured in a HIP graph (as the benchmark
replays its step) give, on every replay, exactly what the same calls give
when launched eagerly.  Replays are interleaved with eager work and
synchronisations."""
import numpy as np
import pytest
import torch

import looped_transformer_decode_amd as L
from synth.workloads import WORKLOADS, Codec
from tests.gpu_cases import DecodeInputs, host_store, new_store, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tmpl,kw", [
    ("extreme_batch_b768_ctx4k", dict(B=3, D=2, N=300)),
    ("lla2d_b256_ctx4k", dict(B=2, D=2, N=170)),
    ("bf16_b32_ctx4k", dict(B=3, D=2, N=700, H=8)),      # several splits + merge
    # 400 appended rows: enough row blocks for the LDS-ring encode
    ("extreme_batch_b768_ctx4k", dict(B=400, D=2, N=16)),
], ids=["per_head", "lla2d", "per_head_split", "per_head_streamed_encode"])
def test_graph_replay_matches_eager(device, tmpl, kw):
    w = WORKLOADS[tmpl].scaled(**kw)
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    codec = Codec(w)
    inp = DecodeInputs(w, codec, 1, w.T - 1, device)
    is2d = w.variant == "2d"
    decode = L.lla2d_decode_attn if is2d else L.lla_decode_attn
    encode = L.lla2d_encode_append if is2d else L.lla_encode_append
    K = w.T * w.width
    x = {a: codec.x(a, 0, w.B) for a in "kv"}
    if is2d:
        xs = [to_device(x[a].reshape(w.B, 1, K), w.dtype, device) for a in "kv"]
        mus = [to_device(codec.mu(a, 0)[0], "f32", device) for a in "kv"]
        wds = [to_device(codec.w_down(a, 0)[0], w.dtype, device) for a in "kv"]
    else:
        xs = [to_device(x[a].reshape(w.B, 1, w.H, K), w.dtype, device) for a in "kv"]
        mus = [to_device(codec.mu(a, 0), "f32", device) for a in "kv"]
        wds = [to_device(codec.w_down(a, 0), w.dtype, device) for a in "kv"]
    pos = torch.tensor(np.resize([w.N - 1, min(41, w.N - 1), min(200, w.N - 1)], w.B),
                       dtype=torch.int32, device=device)
    start = torch.full((w.B,), w.N - 1, dtype=torch.int32, device=device)
    out = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=device)
    ws = L.workspace(store)

    def step():
        decode(store, 1, w.T - 1, inp.d_q, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv, pos, rope,
               out, ws)
        encode(store, 0, *xs, *mus, *wds, start)

    store0 = store.tensor.clone()
    step()
    torch.cuda.synchronize()
    want_out = out.clone()
    want_store = store.tensor.clone()

    store.tensor.copy_(store0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other_q = torch.randn_like(inp.d_q)
    for rep in range(3):
        out.zero_()
        store.tensor.copy_(store0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {rep}: decode output differs"
        assert torch.equal(store.tensor, want_store), f"replay {rep}: encoded store differs"
        # eager work between replays, on the same buffers
        decode(store, 1, 0, other_q, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv, pos, rope, out, ws)
        torch.cuda.synchronize()
        assert np.isfinite(out.cpu().numpy()).all()


def test_graph_replay_inflight_and_kv(device):
    """The in-flight multi-query call and the uncompressed-cache calls (fill,
    append, flash-decode), as the benchmark replays them, give on every
    replay what eager launches give."""
    w = WORKLOADS["long_recurrence_t16_ctx8k"].scaled(B=2, D=1, N=300, H=8)
    vals = host_store(w)
    store = new_store(w, device, tensor=to_device(vals, w.dtype, device))
    rope = L.rope_table(store, device)
    inp = DecodeInputs(w, Codec(w), 0, w.T - 1, device)
    nq = 16
    g = torch.Generator(device="cpu").manual_seed(5)
    q = torch.randn((w.B, nq, w.H, w.d), generator=g).to(device)
    kn = torch.randn((w.B, nq, w.H, w.d), generator=g).to(device)
    vn = torch.randn((w.B, nq, w.H, w.d), generator=g).to(device)
    pos0 = torch.tensor([w.N - nq, 100], dtype=torch.int32, device=device)
    out_if = torch.empty((w.B, nq, w.H, w.d), dtype=torch.float32, device=device)
    ws_if = L.workspace(store, n_q=nq)
    cache = L.KvCache(w.dtype, batch=w.B, layers=1, loops=2, max_ctx=w.N, heads=w.H,
                      d_head=w.d, device=device)
    cache.tensor.zero_()
    kq = torch.randn((w.B, w.H, w.d), generator=g).to(device)
    pos = torch.tensor([w.N - 1, 57], dtype=torch.int32, device=device)
    start = torch.tensor([w.N - 1, 57], dtype=torch.int32, device=device)
    k1 = torch.randn((w.B, 1, w.H, w.d), generator=g).to(device)
    v1 = torch.randn((w.B, 1, w.H, w.d), generator=g).to(device)
    out_kv = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=device)
    ws_kv = L.kv_workspace(cache)

    def step():
        L.lla_decode_attn_inflight(store, 0, w.T - 1, q, kn, vn, inp.d_wk, inp.d_wv, inp.d_mk,
                                   inp.d_mv, pos0, rope, out_if, ws_if)
        L.lla_kv_fill_from_store(store, 0, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv, 0, w.N, rope,
                                 cache, 0)
        L.lla_kv_append(cache, 0, 1, k1, v1, start, rope)
        L.lla_kv_decode_attn(cache, 0, 0, kq, pos, rope, out_kv, ws_kv)

    step()
    torch.cuda.synchronize()
    want = (out_if.clone(), out_kv.clone(), cache.tensor.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        out_if.zero_()
        out_kv.zero_()
        cache.tensor.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_if, want[0]), f"replay {rep}: in-flight output differs"
        assert torch.equal(out_kv, want[1]), f"replay {rep}: flash-decode output differs"
        assert torch.equal(cache.tensor, want[2]), f"replay {rep}: cache differs"
        L.lla_kv_decode_attn(cache, 0, 0, torch.randn_like(kq), pos, rope, out_kv, ws_kv)
        torch.cuda.synchronize()
