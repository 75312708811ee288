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
        L.synth_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.synth_read_stream.restype = ctypes.c_int
        L.synth_write_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_void_p]
        L.synth_write_stream.restype = ctypes.c_int
        L.synth_mfma_spin.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
        L.synth_mfma_spin.restype = ctypes.c_int
        L.synth_mfma_valu_overlap.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
        L.synth_mfma_valu_overlap.restype = ctypes.c_int
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


def read_stream(src: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Launch the streaming-read kernel over all of src (bytes a multiple of
    16) with `blocks` workgroups; sink must hold blocks * 256 * 16 bytes."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < blocks * 256 * 16:
        raise ValueError("sink too small")
    err = _load().synth_read_stream(src.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                    torch.cuda.current_stream(src.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_read_stream failed: hipError {err}")


def write_stream(dst: torch.Tensor, blocks: int, src: torch.Tensor = None) -> None:
    """Launch the streaming-write kernel over all of dst (bytes a multiple of
    16) with `blocks` workgroups: a fixed pattern, or a copy of src (the same
    size) when given."""
    nbytes = dst.numel() * dst.element_size()
    if src is not None and src.numel() * src.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    err = _load().synth_write_stream(None if src is None else src.data_ptr(), dst.data_ptr(),
                                     nbytes, blocks,
                                     torch.cuda.current_stream(dst.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_write_stream failed: hipError {err}")


def mfma_spin(blocks: int, iters: int, sink: torch.Tensor) -> None:
    """Launch the register-only MFMA kernel: blocks x 4 waves, each 4 * iters
    v_mfma_f32_32x32x16_bf16; sink: float32, at least blocks * 256 values."""
    if sink.numel() < blocks * 256 or sink.dtype != torch.float32:
        raise ValueError("sink too small")
    err = _load().synth_mfma_spin(blocks, iters, sink.data_ptr(),
                                  torch.cuda.current_stream(sink.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_mfma_spin failed: hipError {err}")


def mfma_valu_overlap(blocks: int, iters: int, mode: int, sink: torch.Tensor) -> None:
    """Launch the two-pipe overlap kernel: blocks x 8 waves; mode 1 = MFMA
    waves only, 2 = vector-ALU waves only, 3 = both (one of each per SIMD);
    sink: float32, at least blocks * 512 values."""
    if sink.numel() < blocks * 512 or sink.dtype != torch.float32:
        raise ValueError("sink too small")
    err = _load().synth_mfma_valu_overlap(blocks, iters, mode, sink.data_ptr(),
                                          torch.cuda.current_stream(sink.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_mfma_valu_overlap failed: hipError {err}")
