"""Thin Python binding of the LLA C ABI (include/lla.h) via ctypes.

Argument marshalling only: every step of the decode / encode path runs in
the HIP kernels of liblla.so.  torch supplies device memory and streams.
The library must be built (``looped_transformer_decode_amd.build``); this
module raises instead of falling back to anything else when it is missing.
"""
from __future__ import annotations

import ctypes
import os
from fractions import Fraction

import torch

# LLA_LIBRARY selects another build of the same library (the host-side
# sanitizer build, _build/liblla_san.so); the default is the in-tree build.
LIB_PATH = os.environ.get("LLA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "liblla.so")

LLA_PER_HEAD, LLA_2D = 0, 1
LLA_DT_F32, LLA_DT_BF16 = 0, 1
STATUS = ["LLA_OK", "LLA_E_NULL", "LLA_E_SHAPE", "LLA_E_DTYPE", "LLA_E_RANGE",
          "LLA_E_WORKSPACE", "LLA_E_UNSUPPORTED", "LLA_E_VARIANT", "LLA_E_HIP",
          "LLA_E_OVERFLOW", "LLA_E_SCRATCH"]
_TORCH_DT = {LLA_DT_F32: torch.float32, LLA_DT_BF16: torch.bfloat16}
_DT_NAME = {"f32": LLA_DT_F32, "bf16": LLA_DT_BF16}
_VARIANT_NAME = {"per_head": LLA_PER_HEAD, "2d": LLA_2D}


class LlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class StoreDesc(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("loops", ctypes.c_int32),
                ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("data", ctypes.c_void_p)]


_lib = None
_P, _I32, _I64, _SZ, _F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                           ctypes.c_size_t, ctypes.c_float)
_SIGS = {
    "lla_status_string": ([_I32], ctypes.c_char_p),
    "lla_store_check": ([_P], _I32),
    "lla_store_bytes": ([_P], _SZ),
    "lla_store_offset": ([_P, _I32, _I32, _I32, _I32, _I32], _I64),
    "lla_compression_ratio": ([_P, _P, _P], _I32),
    "lla_rope_table_bytes": ([_P], _SZ),
    "lla_rope_table_fill": ([_P, _P, _SZ], _I32),
    "lla_encode_append": ([_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _P], _I32),
    "lla2d_encode_append": ([_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _P], _I32),
    "lla_decode_workspace_bytes": ([_P, _I32], _SZ),
    "lla_decode_auto_splits": ([_P], _I32),
    "lla_decode_attn": ([_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _SZ, _I32, _P],
                        _I32),
    "lla2d_decode_attn": ([_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _SZ, _I32,
                           _P], _I32),
    "lla_decode_attn_noalloc": ([_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _F, _P, _I32, _P],
                                _I32),
    "lla_decode_path": ([_P], ctypes.c_char_p),
    "lla_decode_inflight_workspace_bytes": ([_P, _I32, _I32], _SZ),
    "lla_decode_attn_inflight": ([_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F,
                                  _P, _P, _SZ, _I32, _P], _I32),
    "lla_kv_cache_check": ([_P], _I32),
    "lla_kv_cache_bytes": ([_P], _SZ),
    "lla_kv_rope_table_bytes": ([_P], _SZ),
    "lla_kv_rope_table_fill": ([_P, _P, _SZ], _I32),
    "lla_kv_fill_from_store": ([_P, _I32, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P], _I32),
    "lla_kv_append": ([_P, _I32, _I32, _P, _P, _P, _I32, _P, _P], _I32),
    "lla_kv_decode_workspace_bytes": ([_P, _I32], _SZ),
    "lla_kv_decode_auto_splits": ([_P], _I32),
    "lla_kv_decode_attn": ([_P, _I32, _I32, _P, _P, _P, _F, _P, _P, _SZ, _I32, _P], _I32),
    "lla_svd_init_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "lla_svd_init": ([_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I32, _P, _SZ, _P],
                     _I32),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded liblla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m looped_transformer_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lla_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise LlaError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class KvCacheDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("loops", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("data", ctypes.c_void_p)]


class LatentStore:
    """A latent store: the descriptor plus the device tensor that holds it.

    tensor shape [B, D, N, H', r_k + r_v] (H' = H per-head, 1 for LLA-2D),
    torch dtype float32 or bfloat16.  ``tensor`` may be supplied (it must be
    contiguous and of that shape) or is allocated uninitialised on
    ``device``; ``device=None`` creates a descriptor without memory (host-only
    queries such as sizes and offsets)."""

    def __init__(self, variant="per_head", dtype="bf16", *, batch, layers, max_ctx, heads,
                 d_head, loops, r_k, r_v, rope_base=10000.0, tensor=None, device=None):
        self.variant = _VARIANT_NAME.get(variant, variant)
        self.dtype = _DT_NAME.get(dtype, dtype)
        self.batch, self.layers, self.max_ctx = batch, layers, max_ctx
        self.heads, self.d_head, self.loops, self.r_k, self.r_v = heads, d_head, loops, r_k, r_v
        self.rope_base = rope_base
        self.store_heads = 1 if self.variant == LLA_2D else heads
        self.shape = (batch, layers, max_ctx, self.store_heads, r_k + r_v)
        if tensor is None and device is not None:
            tensor = torch.empty(self.shape, dtype=_TORCH_DT[self.dtype], device=device)
        if tensor is not None:
            if tuple(tensor.shape) != self.shape or not tensor.is_contiguous():
                raise ValueError(f"store tensor must be contiguous {self.shape}")
            if tensor.dtype != _TORCH_DT[self.dtype]:
                raise ValueError(f"store tensor dtype must be {_TORCH_DT[self.dtype]}")
        self.tensor = tensor

    @property
    def torch_dtype(self):
        return _TORCH_DT[self.dtype]

    def desc(self) -> StoreDesc:
        return StoreDesc(self.variant, self.dtype, self.batch, self.layers, self.max_ctx,
                         self.heads, self.d_head, self.loops, self.r_k, self.r_v,
                         self.rope_base, _ptr(self.tensor))


# ---------------------------------------------------------------- host-only
def lla_store_check(store: LatentStore) -> None:
    d = store.desc()
    _check(lib().lla_store_check(ctypes.byref(d)), "lla_store_check")


def lla_store_bytes(store: LatentStore) -> int:
    d = store.desc()
    return lib().lla_store_bytes(ctypes.byref(d))


def lla_store_offset(store: LatentStore, b, layer, pos, head, comp) -> int:
    d = store.desc()
    return lib().lla_store_offset(ctypes.byref(d), b, layer, pos, head, comp)


def lla_compression_ratio(store: LatentStore) -> Fraction:
    d = store.desc()
    num, den = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().lla_compression_ratio(ctypes.byref(d), ctypes.byref(num), ctypes.byref(den)),
           "lla_compression_ratio")
    return Fraction(num.value, den.value)


def lla_rope_table_bytes(store: LatentStore) -> int:
    d = store.desc()
    return lib().lla_rope_table_bytes(ctypes.byref(d))


def lla_rope_table_fill(store: LatentStore) -> torch.Tensor:
    """Host (CPU) uint8 tensor holding the RoPE table."""
    d = store.desc()
    n = lib().lla_rope_table_bytes(ctypes.byref(d))
    if n == 0:
        raise LlaError(lib().lla_store_check(ctypes.byref(d)) or 2, "lla_rope_table_bytes")
    host = torch.empty(n, dtype=torch.uint8)
    _check(lib().lla_rope_table_fill(ctypes.byref(d), host.data_ptr(), n), "lla_rope_table_fill")
    return host


def rope_table(store: LatentStore, device) -> torch.Tensor:
    """The RoPE table copied to ``device``."""
    return lla_rope_table_fill(store).to(device)


def lla_decode_workspace_bytes(store: LatentStore, n_splits: int = 0) -> int:
    d = store.desc()
    return lib().lla_decode_workspace_bytes(ctypes.byref(d), n_splits)


def lla_decode_auto_splits(store: LatentStore) -> int:
    d = store.desc()
    return lib().lla_decode_auto_splits(ctypes.byref(d))


def lla_decode_path(store: LatentStore) -> str | None:
    d = store.desc()
    r = lib().lla_decode_path(ctypes.byref(d))
    return None if r is None else r.decode()


def lla_decode_inflight_workspace_bytes(store: LatentStore, n_q: int, n_splits: int = 0) -> int:
    d = store.desc()
    return lib().lla_decode_inflight_workspace_bytes(ctypes.byref(d), n_q, n_splits)


def workspace(store: LatentStore, n_splits: int = 0, device=None, n_q: int = 1) -> torch.Tensor:
    n = (lla_decode_workspace_bytes(store, n_splits) if n_q == 1
         else lla_decode_inflight_workspace_bytes(store, n_q, n_splits))
    dev = device if device is not None else store.tensor.device
    return torch.empty(max(n, 4), dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------- launching
def _need(t, dtype, shape, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _encode(fn, store, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v, start_pos, n_new,
            stream):
    s = store
    width = s.d_head * (s.heads if s.variant == LLA_2D else 1)
    K = s.loops * width
    hs = s.store_heads
    if n_new is None:
        n_new = x_k.shape[1]
    _need(x_k, s.torch_dtype, (s.batch, n_new, hs, K) if s.variant == LLA_PER_HEAD
          else (s.batch, n_new, K), "x_k")
    _need(x_v, s.torch_dtype, tuple(x_k.shape), "x_v")
    _need(mu_k, torch.float32, (hs, K) if s.variant == LLA_PER_HEAD else (K,), "mu_k")
    _need(mu_v, torch.float32, tuple(mu_k.shape), "mu_v")
    _need(w_down_k, s.torch_dtype, (hs, K, s.r_k) if s.variant == LLA_PER_HEAD
          else (K, s.r_k), "w_down_k")
    _need(w_down_v, s.torch_dtype, (hs, K, s.r_v) if s.variant == LLA_PER_HEAD
          else (K, s.r_v), "w_down_v")
    _need(start_pos, torch.int32, (s.batch,), "start_pos")
    d = s.desc()
    _check(fn(ctypes.byref(d), layer, _ptr(x_k), _ptr(x_v), _ptr(mu_k), _ptr(mu_v),
              _ptr(w_down_k), _ptr(w_down_v), _ptr(start_pos), n_new, _stream(stream)),
           fn.__name__)


def lla_encode_append(store, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v, start_pos,
                      n_new=None, stream=None):
    """c = (x - mu) W_down for n_new tokens per sequence (per-head store)."""
    _encode(lib().lla_encode_append, store, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v,
            start_pos, n_new, stream)


def lla2d_encode_append(store, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v, start_pos,
                        n_new=None, stream=None):
    """LLA-2D encode: one latent per token over the [t][h][d] stack."""
    _encode(lib().lla2d_encode_append, store, layer, x_k, x_v, mu_k, mu_v, w_down_k, w_down_v,
            start_pos, n_new, stream)


def _decode(fn, store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos, rope, out,
            ws, softmax_scale, n_splits, stream):
    s = store
    H, d = s.heads, s.d_head
    _need(q, torch.float32, (s.batch, H, d), "q")
    if s.variant == LLA_PER_HEAD:
        _need(w_up_k_t, s.torch_dtype, (H, d, s.r_k), "w_up_k_t")
        _need(w_up_v_t, s.torch_dtype, (H, d, s.r_v), "w_up_v_t")
        _need(mu_k_t, torch.float32, (H, d), "mu_k_t")
        _need(mu_v_t, torch.float32, (H, d), "mu_v_t")
    else:
        _need(w_up_k_t, s.torch_dtype, (H * d, s.r_k), "w_up_k_t")
        _need(w_up_v_t, s.torch_dtype, (H * d, s.r_v), "w_up_v_t")
        _need(mu_k_t, torch.float32, (H * d,), "mu_k_t")
        _need(mu_v_t, torch.float32, (H * d,), "mu_v_t")
    _need(pos, torch.int32, (s.batch,), "pos")
    _need(out, torch.float32, (s.batch, H, d), "out")
    dsc = s.desc()
    _check(fn(ctypes.byref(dsc), layer, loop, _ptr(q), _ptr(w_up_k_t), _ptr(w_up_v_t),
              _ptr(mu_k_t), _ptr(mu_v_t), _ptr(pos), _ptr(rope), float(softmax_scale), _ptr(out),
              _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), n_splits,
              _stream(stream)), fn.__name__)
    return out


def lla_decode_attn(store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos, rope_table,
                    out, workspace, softmax_scale=0.0, n_splits=0, stream=None):
    """Decode-time attention at (layer, loop) over a per-head latent store."""
    return _decode(lib().lla_decode_attn, store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t,
                   mu_v_t, pos, rope_table, out, workspace, softmax_scale, n_splits, stream)


def lla_decode_attn_noalloc(store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos,
                            rope_table, out, softmax_scale=0.0, n_splits=0, stream=None):
    """lla_decode_attn without a workspace: the split partials go to the
    library's static per-device scratch (LLA_NOALLOC_SCRATCH_BYTES); calls
    that overlap on one GPU race."""
    s = store
    H, d = s.heads, s.d_head
    _need(q, torch.float32, (s.batch, H, d), "q")
    _need(w_up_k_t, s.torch_dtype, (H, d, s.r_k), "w_up_k_t")
    _need(w_up_v_t, s.torch_dtype, (H, d, s.r_v), "w_up_v_t")
    _need(mu_k_t, torch.float32, (H, d), "mu_k_t")
    _need(mu_v_t, torch.float32, (H, d), "mu_v_t")
    _need(pos, torch.int32, (s.batch,), "pos")
    _need(out, torch.float32, (s.batch, H, d), "out")
    dsc = s.desc()
    _check(lib().lla_decode_attn_noalloc(ctypes.byref(dsc), layer, loop, _ptr(q), _ptr(w_up_k_t),
                                         _ptr(w_up_v_t), _ptr(mu_k_t), _ptr(mu_v_t), _ptr(pos),
                                         _ptr(rope_table), float(softmax_scale), _ptr(out),
                                         n_splits, _stream(stream)), "lla_decode_attn_noalloc")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # LLA_NOALLOC_SCRATCH_BYTES of include/lla.h


def lla2d_decode_attn(store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos,
                      rope_table, out, workspace, softmax_scale=0.0, n_splits=0, stream=None):
    """LLA-2D decode: one latent per token decodes all H heads."""
    return _decode(lib().lla2d_decode_attn, store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t,
                   mu_v_t, pos, rope_table, out, workspace, softmax_scale, n_splits, stream)


def lla_decode_attn_inflight(store, layer, loop, q, k_new, v_new, w_up_k_t, w_up_v_t, mu_k_t,
                             mu_v_t, pos0, rope_table, out, workspace, softmax_scale=0.0,
                             n_splits=0, stream=None):
    """Multi-query causal decode with the exact in-flight self-term: query i of
    sequence b (position pos0[b] + i) attends store slots < pos0[b] and the
    in-flight tokens 0..i (q, k_new, v_new, out: [B, n_q, H, d] float32)."""
    s = store
    H, d = s.heads, s.d_head
    if q.dim() != 4:
        raise ValueError("q must be [B, n_q, H, d]")
    n_q = q.shape[1]
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out")):
        _need(t, torch.float32, (s.batch, n_q, H, d), nm)
    if s.variant == LLA_PER_HEAD:
        _need(w_up_k_t, s.torch_dtype, (H, d, s.r_k), "w_up_k_t")
        _need(w_up_v_t, s.torch_dtype, (H, d, s.r_v), "w_up_v_t")
        _need(mu_k_t, torch.float32, (H, d), "mu_k_t")
        _need(mu_v_t, torch.float32, (H, d), "mu_v_t")
    else:
        _need(w_up_k_t, s.torch_dtype, (H * d, s.r_k), "w_up_k_t")
        _need(w_up_v_t, s.torch_dtype, (H * d, s.r_v), "w_up_v_t")
        _need(mu_k_t, torch.float32, (H * d,), "mu_k_t")
        _need(mu_v_t, torch.float32, (H * d,), "mu_v_t")
    _need(pos0, torch.int32, (s.batch,), "pos0")
    dsc = s.desc()
    f = lib().lla_decode_attn_inflight
    _check(f(ctypes.byref(dsc), layer, loop, n_q, _ptr(q), _ptr(k_new), _ptr(v_new),
             _ptr(w_up_k_t), _ptr(w_up_v_t), _ptr(mu_k_t), _ptr(mu_v_t), _ptr(pos0),
             _ptr(rope_table), float(softmax_scale), _ptr(out), _ptr(workspace),
             0 if workspace is None else workspace.numel() * workspace.element_size(), n_splits,
             _stream(stream)), "lla_decode_attn_inflight")
    return out


# ------------------------------------------------- uncompressed K/V cache
class KvCache:
    """An uncompressed K/V cache [B, D, L, N, H, 2, d] (keys stored after
    RoPE): L = T loops for the serving fast path, 1 for the final-loop-reuse
    control.  ``tensor`` as for LatentStore."""

    def __init__(self, dtype="bf16", *, batch, layers, loops, max_ctx, heads, d_head,
                 rope_base=10000.0, tensor=None, device=None):
        self.dtype = _DT_NAME.get(dtype, dtype)
        self.batch, self.layers, self.loops, self.max_ctx = batch, layers, loops, max_ctx
        self.heads, self.d_head, self.rope_base = heads, d_head, rope_base
        self.shape = (batch, layers, loops, max_ctx, heads, 2, d_head)
        if tensor is None and device is not None:
            tensor = torch.empty(self.shape, dtype=_TORCH_DT[self.dtype], device=device)
        if tensor is not None:
            if tuple(tensor.shape) != self.shape or not tensor.is_contiguous():
                raise ValueError(f"cache tensor must be contiguous {self.shape}")
            if tensor.dtype != _TORCH_DT[self.dtype]:
                raise ValueError(f"cache tensor dtype must be {_TORCH_DT[self.dtype]}")
        self.tensor = tensor

    @property
    def torch_dtype(self):
        return _TORCH_DT[self.dtype]

    def desc(self) -> KvCacheDesc:
        return KvCacheDesc(self.dtype, self.batch, self.layers, self.loops, self.max_ctx,
                           self.heads, self.d_head, self.rope_base, _ptr(self.tensor))


def lla_kv_cache_check(cache: KvCache) -> None:
    d = cache.desc()
    _check(lib().lla_kv_cache_check(ctypes.byref(d)), "lla_kv_cache_check")


def lla_kv_cache_bytes(cache: KvCache) -> int:
    d = cache.desc()
    return lib().lla_kv_cache_bytes(ctypes.byref(d))


def lla_kv_rope_table_bytes(cache: KvCache) -> int:
    d = cache.desc()
    return lib().lla_kv_rope_table_bytes(ctypes.byref(d))


def lla_kv_rope_table_fill(cache: KvCache) -> torch.Tensor:
    """Host (CPU) uint8 tensor holding the cache's RoPE table."""
    d = cache.desc()
    n = lib().lla_kv_rope_table_bytes(ctypes.byref(d))
    if n == 0:
        raise LlaError(lib().lla_kv_cache_check(ctypes.byref(d)) or 2, "lla_kv_rope_table_bytes")
    host = torch.empty(n, dtype=torch.uint8)
    _check(lib().lla_kv_rope_table_fill(ctypes.byref(d), host.data_ptr(), n),
           "lla_kv_rope_table_fill")
    return host


def lla_kv_decode_workspace_bytes(cache: KvCache, n_splits: int = 0) -> int:
    d = cache.desc()
    return lib().lla_kv_decode_workspace_bytes(ctypes.byref(d), n_splits)


def lla_kv_decode_auto_splits(cache: KvCache) -> int:
    d = cache.desc()
    return lib().lla_kv_decode_auto_splits(ctypes.byref(d))


def kv_workspace(cache: KvCache, n_splits: int = 0, device=None) -> torch.Tensor:
    n = lla_kv_decode_workspace_bytes(cache, n_splits)
    dev = device if device is not None else cache.tensor.device
    return torch.empty(max(n, 4), dtype=torch.uint8, device=dev)


def lla_kv_fill_from_store(store, layer, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, slot0, n_slots,
                           rope_table, cache, cache_loop, stream=None):
    """Reconstruct loop t (given by w_up_*_t, mu_*_t) of store slots
    [slot0, slot0 + n_slots) into cache[:, layer, cache_loop]."""
    s = store
    H, d = s.heads, s.d_head
    shp = {"k": (H, d, s.r_k), "v": (H, d, s.r_v)} if s.variant == LLA_PER_HEAD else \
          {"k": (H * d, s.r_k), "v": (H * d, s.r_v)}
    _need(w_up_k_t, s.torch_dtype, shp["k"], "w_up_k_t")
    _need(w_up_v_t, s.torch_dtype, shp["v"], "w_up_v_t")
    mshape = (H, d) if s.variant == LLA_PER_HEAD else (H * d,)
    _need(mu_k_t, torch.float32, mshape, "mu_k_t")
    _need(mu_v_t, torch.float32, mshape, "mu_v_t")
    sd, cd = s.desc(), cache.desc()
    _check(lib().lla_kv_fill_from_store(ctypes.byref(sd), layer, _ptr(w_up_k_t), _ptr(w_up_v_t),
                                        _ptr(mu_k_t), _ptr(mu_v_t), slot0, n_slots,
                                        _ptr(rope_table), ctypes.byref(cd), cache_loop,
                                        _stream(stream)), "lla_kv_fill_from_store")


def lla_kv_append(cache, layer, cache_loop, k, v, start_pos, rope_table, n_new=None,
                  stream=None):
    """Rotate k at its slot and write (k, v) [B, n_new, H, d] float32 into
    cache[:, layer, cache_loop, start_pos[b] + j]."""
    c = cache
    if n_new is None:
        n_new = k.shape[1]
    _need(k, torch.float32, (c.batch, n_new, c.heads, c.d_head), "k")
    _need(v, torch.float32, (c.batch, n_new, c.heads, c.d_head), "v")
    _need(start_pos, torch.int32, (c.batch,), "start_pos")
    cd = c.desc()
    _check(lib().lla_kv_append(ctypes.byref(cd), layer, cache_loop, _ptr(k), _ptr(v),
                               _ptr(start_pos), n_new, _ptr(rope_table), _stream(stream)),
           "lla_kv_append")


def lla_kv_decode_attn(cache, layer, cache_loop, q, pos, rope_table, out, workspace,
                       softmax_scale=0.0, n_splits=0, stream=None):
    """Flash-decode over cache[:, layer, cache_loop] for queries q [B, H, d]."""
    c = cache
    _need(q, torch.float32, (c.batch, c.heads, c.d_head), "q")
    _need(pos, torch.int32, (c.batch,), "pos")
    _need(out, torch.float32, (c.batch, c.heads, c.d_head), "out")
    cd = c.desc()
    _check(lib().lla_kv_decode_attn(ctypes.byref(cd), layer, cache_loop, _ptr(q), _ptr(pos),
                                    _ptr(rope_table), float(softmax_scale), _ptr(out),
                                    _ptr(workspace),
                                    0 if workspace is None
                                    else workspace.numel() * workspace.element_size(),
                                    n_splits, _stream(stream)), "lla_kv_decode_attn")
    return out


# ------------------------------------------------------ SVD initialisation
def lla_svd_init_workspace_bytes(groups: int, loops: int, width: int, r: int) -> int:
    return lib().lla_svd_init_workspace_bytes(groups, loops, width, r)


def lla_svd_init(x, loops, width, r, mu, w_down, w_up, sigma=None, workspace=None, iters=0,
                 stream=None):
    """SVD codec initialisation of G codecs from calibration rows x
    [n_cal, G, loops*width] (float32 or bfloat16): writes mu [G, K] (float32),
    w_down [G, K, r], w_up [loops, G, width, r] (x's type) and, if given,
    sigma [G, r] (float32).  Allocates the workspace if none is passed."""
    if x.dim() != 3:
        raise ValueError("x must be [n_cal, G, loops*width]")
    n_cal, G, K = x.shape
    if K != loops * width:
        raise ValueError("x's last dimension must be loops * width")
    dt = {torch.float32: LLA_DT_F32, torch.bfloat16: LLA_DT_BF16}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be float32 or bfloat16")
    _need(x, x.dtype, None, "x")
    _need(mu, torch.float32, (G, K), "mu")
    _need(w_down, x.dtype, (G, K, r), "w_down")
    _need(w_up, x.dtype, (loops, G, width, r), "w_up")
    _need(sigma, torch.float32, (G, r), "sigma")
    if workspace is None:
        n = lla_svd_init_workspace_bytes(G, loops, width, r)
        workspace = torch.empty(max(n, 4), dtype=torch.uint8, device=x.device)
    _check(lib().lla_svd_init(dt, G, n_cal, loops, width, r, _ptr(x), _ptr(mu), _ptr(w_down),
                              _ptr(w_up), _ptr(sigma), iters, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)),
           "lla_svd_init")
