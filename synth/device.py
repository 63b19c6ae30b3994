"""Device side of the seeded input generator (ctypes over synth/libbloomsynth.so).

Fills GPU tensors with exactly the values ``synth.values`` defines on the
host, so large inputs can be made in HBM without a host round trip.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import MODE_ABS_F32, MODE_BF16, MODE_F32, scale_f32, tensor_key

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbloomsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build with `python -m bloom_bf16_optimizer_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.synth_stream_copy.restype = ctypes.c_int
        lib.synth_stream_copy.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_void_p]
        _lib = lib
    return _lib


def fill_(t: torch.Tensor, seed: int, stream: int, sigma: float, offset: float = 0.0, start: int = 0) -> torch.Tensor:
    """Fills a contiguous GPU tensor in place (bf16 -> MODE_BF16, float32 -> MODE_F32)."""
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("fill_ needs a contiguous GPU tensor")
    mode = {torch.bfloat16: MODE_BF16, torch.float32: MODE_F32}[t.dtype]
    return _fill(t, seed, stream, sigma, offset, start, mode)


def fill_abs_(t: torch.Tensor, seed: int, stream: int, sigma: float, start: int = 0) -> torch.Tensor:
    """Fills a float32 GPU tensor with |values| (MODE_ABS_F32)."""
    if t.dtype != torch.float32:
        raise TypeError("fill_abs_ needs float32")
    return _fill(t, seed, stream, sigma, 0.0, start, MODE_ABS_F32)


def _fill(t, seed, stream, sigma, offset, start, mode):
    rc = _load().synth_fill(t.data_ptr(), t.numel(), start, tensor_key(seed, stream), float(scale_f32(sigma)),
                            float(np.float32(offset)), int(offset != 0.0), mode,
                            torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed with code {rc}")
    return t


def stream_copy(outs, ins) -> None:
    """Plain streaming copy (the bandwidth ceiling bench.py compares kernels with).

    ``outs`` (1 or 2) and ``ins`` (1 or 2) are contiguous GPU tensors of one
    common byte size, a multiple of 16; every output receives the XOR of the
    inputs (a copy for one input).  Enqueued on the current stream.
    """
    nbytes = outs[0].numel() * outs[0].element_size()
    for t in (*outs, *ins):
        if not (t.is_cuda and t.is_contiguous()) or t.numel() * t.element_size() != nbytes:
            raise ValueError("stream_copy needs contiguous GPU tensors of one byte size")
    if nbytes % 16:
        raise ValueError("stream_copy needs a multiple of 16 bytes")
    o = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
    i = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
    rc = _load().synth_stream_copy(o, len(outs), i, len(ins), nbytes // 16, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_copy failed with code {rc}")
