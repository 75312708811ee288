"""Device-side filling of large synthetic buffers (synth/libllasynth.so):
the counter-based generator of synth/gen.py, evaluated on the GPU."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllasynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run `python -m looped_transformer_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                                 ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        L.synth_fill.restype = ctypes.c_int
        _lib = L
    return _lib


def fill_hash_normal(t: torch.Tensor, key: int, first: int = 0, scale: float = 1.0) -> torch.Tensor:
    """t.view(-1)[i] = scale * hash_normal(key, first + i) (float32 or bf16)."""
    if t.dtype not in (torch.float32, torch.bfloat16) or not t.is_contiguous():
        raise ValueError("contiguous float32 / bfloat16 tensor expected")
    dt = 1 if t.dtype == torch.bfloat16 else 0
    err = _load().synth_fill(t.data_ptr(), t.numel(), dt, ctypes.c_uint64(key & (2**64 - 1)),
                             first, scale, torch.cuda.current_stream(t.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_fill failed: hipError {err}")
    return t
