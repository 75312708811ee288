"""The synthetic workloads: shapes and value recipes (no method arithmetic).

Geometry follows the paper's Ouro-1.4B setting where the pages fix it
(T = 4 loops over D = 24 layers, H*d_head = 2048), ranks follow the
compression ratios the pages quote.  Values are seeded and synthetic:
latents and queries ~ N(0, 1); means mu ~ N(0, 0.1^2) (float32);
W_up,t ~ N(0, 1/r); W_down has orthonormal columns (QR of a seeded
Gaussian).  The long-recurrence workload instead initialises
W_up,t as the loop-t slice of W_down and draws appended activations from a
rank-8 trajectory across loops plus N(0, 0.05^2) noise.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import gen


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str          # "per_head" or "2d"
    dtype: str            # storage / codec-matrix type: "f32" or "bf16"
    D: int                # layers
    H: int                # heads
    d: int                # d_head
    T: int                # loops
    r_k: int
    r_v: int
    B: int                # sequences
    N: int                # context slots
    seed: int
    n_new: int = 1        # tokens appended per step and sequence
    w_up_from_w_down: bool = False
    trajectory_inputs: bool = False

    @property
    def store_heads(self) -> int:
        return 1 if self.variant == "2d" else self.H

    @property
    def R(self) -> int:
        return self.r_k + self.r_v

    @property
    def store_shape(self):
        return (self.B, self.D, self.N, self.store_heads, self.R)

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def store_bytes(self) -> int:
        return int(np.prod(self.store_shape)) * self.elt_bytes

    @property
    def width(self) -> int:
        """Width of one loop's vector in the stacked x: d (per-head) or H*d."""
        return self.H * self.d if self.variant == "2d" else self.d

    @property
    def codec_rows(self) -> int:
        """Number of independent codecs per layer and axis."""
        return self.store_heads

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", "per_head", "f32", D=1, H=2, d=64, T=4, r_k=8,
                 r_v=16, B=1, N=128, seed=0),
        Workload("bf16_b32_ctx4k", "per_head", "bf16", D=24, H=16, d=128, T=4,
                 r_k=32, r_v=64, B=32, N=4096, seed=1),
        Workload("extreme_batch_b768_ctx4k", "per_head", "bf16", D=24, H=16,
                 d=128, T=4, r_k=16, r_v=32, B=768, N=4096, seed=2),
        Workload("lla2d_b256_ctx4k", "2d", "bf16", D=24, H=16, d=128, T=4,
                 r_k=64, r_v=128, B=256, N=4096, seed=3),
        Workload("long_recurrence_t16_ctx8k", "per_head", "bf16", D=8, H=16,
                 d=128, T=16, r_k=48, r_v=80, B=64, N=8192, seed=4, n_new=16,
                 w_up_from_w_down=True, trajectory_inputs=True),
    ]
}

# tensor ids inside one workload's seed space
TID_STORE = 1
TID_Q = 2
TID_MU_K, TID_MU_V = 3, 4
TID_WUP_K, TID_WUP_V = 5, 6
TID_WDOWN_K, TID_WDOWN_V = 7, 8
TID_X_K, TID_X_V = 9, 10
TID_POS = 11


class Codec:
    """Host-side codec matrices of one workload, generated lazily per layer.

    All values are returned as (payload, exact float64) pairs by the
    ``*_payload`` helpers; the plain accessors return exact float64."""

    def __init__(self, w: Workload):
        self.w = w
        self._cache = {}

    def _get(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    def mu(self, axis: str, layer: int) -> np.ndarray:
        """[codec_rows, T*width] float32-exact calibration mean."""
        w = self.w
        tid = (TID_MU_K if axis == "k" else TID_MU_V) * 1000 + layer
        return self._get(("mu", axis, layer), lambda: gen.as_storage(
            gen.normal(w.seed, tid, (w.codec_rows, w.T * w.width), 0.1), "f32")[1])

    def w_down(self, axis: str, layer: int) -> np.ndarray:
        """[codec_rows, T*width, r] orthonormal columns, storage-exact."""
        w = self.w
        r = w.r_k if axis == "k" else w.r_v
        base = (TID_WDOWN_K if axis == "k" else TID_WDOWN_V) * 1000 + layer

        def make():
            m = np.stack([gen.orthonormal_columns(w.seed, base * 64 + h, w.T * w.width, r)
                          for h in range(w.codec_rows)])
            return gen.as_storage(m, w.dtype)[1]
        return self._get(("wd", axis, layer), make)

    def w_up(self, axis: str, layer: int, t: int) -> np.ndarray:
        """[codec_rows, width, r] loop-t up-projection, storage-exact.
        Per-head rows are [h][d, r]; LLA-2D is one [H*d, r] matrix."""
        w = self.w
        r = w.r_k if axis == "k" else w.r_v

        def make():
            if w.w_up_from_w_down:
                wd = self.w_down(axis, layer)
                return wd[:, t * w.width:(t + 1) * w.width, :].copy()
            tid = ((TID_WUP_K if axis == "k" else TID_WUP_V) * 1000 + layer) * 64 + t
            return gen.as_storage(gen.normal(w.seed, tid, (w.codec_rows, w.width, r),
                                             1.0 / np.sqrt(r)), w.dtype)[1]
        return self._get(("wu", axis, layer, t), make)

    def q(self, layer: int, t: int, batch: int | None = None) -> np.ndarray:
        """[B, H, d] float32-exact pre-RoPE queries of call (layer, t)."""
        w = self.w
        B = w.B if batch is None else batch
        tid = (TID_Q * 1000 + layer) * 64 + t
        return gen.as_storage(gen.normal(w.seed, tid, (B, w.H, w.d)), "f32")[1]

    def x(self, axis: str, layer: int, rows: int, step: int = 0) -> np.ndarray:
        """[rows, codec_rows, T*width] appended activations (storage-exact)."""
        w = self.w
        tid = ((TID_X_K if axis == "k" else TID_X_V) * 1000 + layer) * 4096 + step
        if w.trajectory_inputs:
            v = np.stack([gen.low_rank_trajectory(w.seed, tid * 64 + h, rows, w.T * w.width)
                          for h in range(w.codec_rows)], axis=1)
        else:
            v = gen.normal(w.seed, tid, (rows, w.codec_rows, w.T * w.width))
        return gen.as_storage(v, w.dtype)[1]


def store_key(w: Workload) -> int:
    return gen.stream_key(w.seed, TID_STORE)


def store_slab(w: Workload, b: int, layer: int, n_slots: int | None = None) -> np.ndarray:
    """Host regeneration of store[b, layer, :n_slots] from the counter-based
    generator: [n_slots, H', R] float64 values (exact in bf16 and f32)."""
    n = w.N if n_slots is None else n_slots
    per_slot = w.store_heads * w.R
    first = (b * w.D + layer) * w.N * per_slot
    v = gen.hash_normal(store_key(w), first, n * per_slot)
    return v.reshape(n, w.store_heads, w.R)
