"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds input generation only: random numbers, rounding of those
numbers to the storage type, and the workload shapes.  It contains none of
the attention / codec arithmetic, and imports neither ``oracle`` nor the
product package.

Two generators:

* ``normal(seed, tensor_id, shape)`` -- numpy PCG64 seeded with
  SeedSequence([seed, tensor_id]); used for every tensor small enough to
  build on the host (queries, codec matrices, means, small stores).

* ``hash_normal(key, first, count)`` -- a counter-based generator for the
  multi-GB latent stores, which are filled on the device.  Element i of a
  stream is SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom
  Number Generators", OOPSLA 2014; mixing constants of Vigna's reference
  splitmix64.c) evaluated at counter i, and the 64-bit output is turned
  into an approximately standard normal value by the Irwin-Hall sum of
  twelve 5-bit uniform fields:  v = (sum_{f=0..11} bits[5f:5f+5] - 186)/32.
  v is a multiple of 1/32 with |v| <= 5.8125, exactly representable in
  bfloat16 and float32, with variance 1023/1024.  The device kernel in
  ``synth/fill.hip`` implements the same definition; any slab of a device
  store can therefore be regenerated on the host, independently of the GPU.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


# --------------------------------------------------------------------------
# float32 / bfloat16 storage helpers (rounding of generated inputs)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (nearest, ties even)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_storage(x64: np.ndarray, dtype: str):
    """Round generated float64 values to the storage type.

    Returns (payload, exact_value_f64): payload is what is uploaded (uint16
    bit patterns for bf16, float32 for f32) and exact_value_f64 is its exact
    value, which is what the oracle consumes."""
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# numpy PCG64 generator
# --------------------------------------------------------------------------
def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def normal(seed: int, tensor_id: int, shape, std: float = 1.0) -> np.ndarray:
    return rng(seed, tensor_id).standard_normal(shape) * std


def orthonormal_columns(seed: int, tensor_id: int, n: int, r: int) -> np.ndarray:
    """n x r matrix with orthonormal columns: Q of the QR factorisation of a
    seeded Gaussian (sign-fixed so that diag(R) > 0)."""
    a = normal(seed, tensor_id, (n, r))
    q, rr = np.linalg.qr(a)
    return q * np.sign(np.diag(rr))[None, :]


def low_rank_trajectory(seed: int, tensor_id: int, rows: int, width: int,
                        rank: int = 8, noise: float = 0.05) -> np.ndarray:
    """rows x width samples x = z M + eps with z ~ N(0, I_rank) per row,
    M ~ N(0, 1/rank) fixed, eps ~ N(0, noise^2): stacked per-loop vectors
    that span `rank` directions plus noise."""
    g = rng(seed, tensor_id)
    M = g.standard_normal((rank, width)) / np.sqrt(rank)
    z = g.standard_normal((rows, rank))
    return z @ M + noise * g.standard_normal((rows, width))


# --------------------------------------------------------------------------
# counter-based generator (matches synth/fill.hip bit for bit)
# --------------------------------------------------------------------------
def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> int:
    """64-bit key of one stream: SplitMix64 output for the counter
    (seed << 32 | tensor_id)."""
    with np.errstate(over="ignore"):
        z = np.array([((seed & 0xFFFFFFFF) << 32) | (tensor_id & 0xFFFFFFFF)],
                     dtype=np.uint64) + GOLDEN_GAMMA
        return int(_mix64(z)[0])


def hash_normal(key: int, first: int, count: int) -> np.ndarray:
    """Elements first..first+count-1 of stream `key` as float64 values
    (each a multiple of 1/32, exactly representable in bf16)."""
    with np.errstate(over="ignore"):
        i = np.arange(first, first + count, dtype=np.uint64)
        z = _mix64(np.uint64(key) + (i + np.uint64(1)) * GOLDEN_GAMMA)
    s = np.zeros(count, dtype=np.int64)
    for f in range(12):
        s += ((z >> np.uint64(5 * f)) & np.uint64(31)).astype(np.int64)
    return (s - 186).astype(np.float64) / 32.0
