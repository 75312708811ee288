"""lla_decode_attn_noalloc: the allocation-free variant of lla_decode_attn
(split partials in the library's static per-device scratch).

GPU: through the C ABI, its output equals lla_decode_attn's on the same
inputs and split count, on two calls in a row (the second with a smaller
batch, context and split count), for the matrix-core bf16 path and the
generic float32 path, and both stay within the bf16 / fp32 tolerance of the
oracle on sampled rows.  CPU: the host-side rejections (oversized calls,
missing pointers) return before any device access."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import looped_transformer_decode_amd as L
from synth.workloads import WORKLOADS, Codec
from tests.gpu_cases import TOL, DecodeInputs, host_store, new_store, row_rel_l2, to_device

LLA_E_NULL, LLA_E_VARIANT, LLA_E_SCRATCH = 1, 7, 10


def _both(w, n_splits, dev):
    vals = host_store(w)
    store = new_store(w, dev, tensor=to_device(vals, w.dtype, dev))
    rope = L.rope_table(store, dev)
    inp = DecodeInputs(w, Codec(w), w.D - 1, w.T - 1, dev)
    rng = np.random.default_rng(w.B * 1000 + w.N)
    pos = rng.integers(0, w.N, size=w.B)
    pos[0] = w.N - 1
    d_pos = torch.from_numpy(pos.astype(np.int32)).to(dev)
    out_ws = torch.full((w.B, w.H, w.d), float("nan"), device=dev)
    out_na = torch.full((w.B, w.H, w.d), float("nan"), device=dev)
    ws = L.workspace(store, n_splits)
    L.lla_decode_attn(store, inp.layer, inp.t, inp.d_q, inp.d_wk, inp.d_wv, inp.d_mk, inp.d_mv,
                      d_pos, rope, out_ws, ws, n_splits=n_splits)
    L.lla_decode_attn_noalloc(store, inp.layer, inp.t, inp.d_q, inp.d_wk, inp.d_wv, inp.d_mk,
                              inp.d_mv, d_pos, rope, out_na, n_splits=n_splits)
    torch.cuda.synchronize()
    a = out_ws.cpu().numpy().astype(np.float64)
    b = out_na.cpu().numpy().astype(np.float64)
    ref = np.stack([inp.oracle(vals[i, inp.layer, :, :, :w.r_k], vals[i, inp.layer, :, :, w.r_k:],
                               i, pos[i]) for i in (0, w.B - 1)])
    return a, b, ref


@pytest.mark.gpu
@pytest.mark.parametrize("base,first,second", [
    # (per-head bf16 matrix-core path) a larger call, then a smaller one
    ("bf16_b32_ctx4k", dict(B=6, D=2, N=1000, S=4), dict(B=3, D=1, N=300, S=2)),
    ("extreme_batch_b768_ctx4k", dict(B=5, D=1, N=777, S=3), dict(B=2, D=1, N=129, S=0)),
    # generic float32 path
    ("tiny_fp32", dict(B=4, D=1, N=128, S=3), dict(B=1, D=1, N=64, S=2)),
])
def test_noalloc_matches_workspace_call(device, base, first, second):
    for cfg in (first, second):
        cfg = dict(cfg)
        S = cfg.pop("S")
        w = WORKLOADS[base].scaled(**cfg)
        a, b, ref = _both(w, S, device)
        print(f"noalloc {base} {cfg} S={S}: equal={np.array_equal(a, b)}", flush=True)
        assert np.all(np.isfinite(b))
        assert np.array_equal(a, b), "same kernels and split count: identical output"
        err = row_rel_l2(b[[0, w.B - 1]], ref).max()
        assert err <= TOL[w.dtype], err


def _desc(w, data=1):
    d = L.StoreDesc(0 if w.variant == "per_head" else 1, 1 if w.dtype == "bf16" else 0, w.B,
                    w.D, w.N, w.H, w.d, w.T, w.r_k, w.r_v, 10000.0, data)
    return d


def _call(d, n_splits=0, null_q=False):
    fake = ctypes.c_void_p(256)  # never dereferenced: the call is rejected on the host
    q = None if null_q else fake
    return L.lib().lla_decode_attn_noalloc(ctypes.byref(d), 0, 0, q, fake, fake, fake, fake,
                                           fake, fake, 0.0, fake, n_splits, None)


def test_noalloc_rejects_on_host():
    w = WORKLOADS["extreme_batch_b768_ctx4k"]
    # B = 768 at 16 splits: 768*16*16*34*4 B = 26.7 MB of partials > 8 MiB
    assert _call(_desc(w), n_splits=16) == LLA_E_SCRATCH
    assert "scratch" in L.status_string(LLA_E_SCRATCH)
    big = w.scaled(B=8192)
    assert _call(_desc(big), n_splits=1) == LLA_E_SCRATCH
    assert _call(_desc(w), null_q=True) == LLA_E_NULL
    assert _call(_desc(WORKLOADS["lla2d_b256_ctx4k"])) == LLA_E_VARIANT
    # the largest call that fits is exactly LLA_NOALLOC_SCRATCH_BYTES or less
    s = L.LatentStore("per_head", "bf16", batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                      d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v)
    assert L.lla_decode_workspace_bytes(s, 2) <= L.NOALLOC_SCRATCH_BYTES
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "lla.h")).read()
    m = re.search(r"#define LLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES
