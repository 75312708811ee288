"""Helpers for the GPU parity tests: build seeded inputs once, hand the
exact same values to the HIP path (through the C ABI binding) and to the
fp64 oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch

import looped_transformer_decode_amd as L
from oracle import lla_oracle as O
from synth import gen
from synth.workloads import Codec, Workload, store_key, store_slab

TOL = {"f32": 1e-5, "bf16": 2e-2}


def to_device(exact: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload float64 values that are exact in `dtype` (f32 / bf16)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(exact, dtype=np.float32)).to(device)
    bits = gen.f32_to_bf16_bits(np.asarray(exact, dtype=np.float32))
    assert np.array_equal(gen.bf16_bits_to_f64(bits), exact), "value not exact in bf16"
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def from_device(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return gen.bf16_bits_to_f64(bits)
    return t.float().cpu().numpy().astype(np.float64)


def row_rel_l2(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error of every output row out[b, h, :]."""
    num = np.linalg.norm(gpu - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)
    return num / den


def attn_rel_l2(gpu: np.ndarray, ref: np.ndarray, mu_v: np.ndarray) -> np.ndarray:
    """Per-row error relative to the softmax-dependent part of the output:
    ||out - out_ref|| / ||out_ref - mu_v,t||, i.e. the relative L2 of
    (out - mu_v,t).  Over long contexts ||mu_v,t|| can exceed the attention
    part several times, and the plain row metric then understates the error
    of the part the kernels compute.  mu_v: broadcastable to the rows [.., H, d]."""
    num = np.linalg.norm(gpu - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref - mu_v, axis=-1), 1e-300)
    return num / den


def mu_rows(inp, w) -> np.ndarray:
    """mu_v,t of a DecodeInputs as [H, d] (LLA-2D's [H*d] split by head)."""
    return np.asarray(inp.mv).reshape(w.H, w.d)


def full_precision_slab(w: Workload, b: int, layer: int) -> np.ndarray:
    """Host N(0, 1) latents of one (sequence, layer) slab rounded to the
    store type: full mantissas and tails, unlike the device filler's
    multiples of 1/32.  [N, H', R] float64 exact values."""
    v = gen.normal(w.seed, 50_000 + b * 1000 + layer, (w.N, w.store_heads, w.R))
    return gen.as_storage(v, w.dtype)[1]


def put_slab(store: L.LatentStore, w: Workload, b: int, layer: int, vals: np.ndarray):
    """Overwrite store[b, layer] on the device with exact values vals."""
    store.tensor[b, layer].copy_(to_device(vals, w.dtype, store.tensor.device))


def new_store(w: Workload, device, tensor=None) -> L.LatentStore:
    return L.LatentStore(w.variant, w.dtype, batch=w.B, layers=w.D, max_ctx=w.N, heads=w.H,
                         d_head=w.d, loops=w.T, r_k=w.r_k, r_v=w.r_v, tensor=tensor,
                         device=device if tensor is None else None)


class DecodeInputs:
    """Device-side codec tensors of one (layer, loop) call plus the exact
    host values the oracle consumes."""

    def __init__(self, w: Workload, codec: Codec, layer: int, t: int, device, batch=None):
        self.w, self.layer, self.t = w, layer, t
        B = w.B if batch is None else batch
        self.q = codec.q(layer, t, B)                                # [B, H, d]
        self.wk = codec.w_up("k", layer, t)                          # [rows, width, r_k]
        self.wv = codec.w_up("v", layer, t)
        self.mk = O.loop_slice(codec.mu("k", layer), t, w.width)     # [rows, width]
        self.mv = O.loop_slice(codec.mu("v", layer), t, w.width)
        if w.variant == "2d":
            shp_k, shp_v, shp_mu = (w.H * w.d, w.r_k), (w.H * w.d, w.r_v), (w.H * w.d,)
        else:
            shp_k, shp_v, shp_mu = (w.H, w.d, w.r_k), (w.H, w.d, w.r_v), (w.H, w.d)
        self.d_q = to_device(self.q, "f32", device)
        self.d_wk = to_device(self.wk.reshape(shp_k), w.dtype, device)
        self.d_wv = to_device(self.wv.reshape(shp_v), w.dtype, device)
        self.d_mk = to_device(self.mk.reshape(shp_mu), "f32", device)
        self.d_mv = to_device(self.mv.reshape(shp_mu), "f32", device)

    def run(self, store: L.LatentStore, pos: np.ndarray, rope, n_splits=0, loop=None,
            scale=0.0) -> np.ndarray:
        dev = store.tensor.device
        d_pos = torch.from_numpy(np.asarray(pos, np.int32)).to(dev)
        out = torch.empty((store.batch, self.w.H, self.w.d), dtype=torch.float32, device=dev)
        ws = L.workspace(store, n_splits)
        fn = L.lla2d_decode_attn if self.w.variant == "2d" else L.lla_decode_attn
        fn(store, self.layer, self.t if loop is None else loop, self.d_q, self.d_wk, self.d_wv,
           self.d_mk, self.d_mv, d_pos, rope, out, ws, softmax_scale=scale, n_splits=n_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    def oracle(self, slab_k: np.ndarray, slab_v: np.ndarray, b: int, pos: int,
               scale=None) -> np.ndarray:
        """slab_*: [N, H', r] exact latents of (b, layer)."""
        w = self.w
        p = min(max(int(pos), 0), w.N - 1)
        if w.variant == "2d":
            return O.decode_2d(slab_k[:, 0], slab_v[:, 0], self.q[b], self.wk[0], self.wv[0],
                               self.mk[0], self.mv[0], p, scale)
        return O.decode(slab_k, slab_v, self.q[b], self.wk, self.wv, self.mk, self.mv, p, scale)


def host_store(w: Workload, tensor_id: int = 1) -> np.ndarray:
    """Small stores: numpy-generated N(0,1) latents, exact in w.dtype."""
    v = gen.normal(w.seed, 900 + tensor_id, w.store_shape)
    return gen.as_storage(v, w.dtype)[1]


def fill_store_on_device(w: Workload, store: L.LatentStore):
    from synth.device import fill_hash_normal
    fill_hash_normal(store.tensor, store_key(w))


def device_slab(w: Workload, b: int, layer: int):
    """Host regeneration of the device-filled slab (b, layer): (c_k, c_v)."""
    s = store_slab(w, b, layer)
    return s[..., :w.r_k], s[..., w.r_k:]
