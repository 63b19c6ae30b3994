"""ctypes loader for libbloomkern.so (the C ABI of include/bloom_kernels.h).

Argument marshalling only.  Importing torch first matters: the library's HIP
runtime dependency (libamdhip64.so.7) then resolves to the runtime PyTorch has
already loaded, so streams and device pointers are shared.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads PyTorch's HIP runtime before the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbloomkern.so")

c_void_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_size = ctypes.c_size_t


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("max_grad_norm", ctypes.c_double), ("step", ctypes.c_int64),
                ("sumsq_in_workspace", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AdamWSegment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("length", ctypes.c_int64), ("weight_decay", ctypes.c_double)]


# name -> (restype, argtypes)
SIGNATURES = {
    "bloom_abi_version": (ctypes.c_int, []),
    "bloom_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bloom_last_error": (ctypes.c_char_p, []),
    "bloom_layernorm_fwd": (ctypes.c_int, [c_void_p] * 6 + [c_i64, c_i64, c_f32, c_void_p]),
    "bloom_layernorm_bwd_workspace_size": (c_size, [c_i64, c_i64]),
    "bloom_layernorm_bwd": (ctypes.c_int, [c_void_p] * 9 + [c_size, c_i64, c_i64, c_void_p]),
    "bloom_layernorm_bwd_noalloc": (ctypes.c_int, [c_void_p] * 8 + [c_i64, c_i64, c_void_p]),
    "bloom_layernorm_residual_fwd": (ctypes.c_int, [c_void_p] * 8 + [c_i64, c_i64, c_f32, c_void_p]),
    "bloom_layernorm_residual_bwd": (ctypes.c_int, [c_void_p] * 10 + [c_size, c_i64, c_i64, c_void_p]),
    "bloom_alibi_slopes": (ctypes.c_int, [c_i32, c_i32, c_i32, ctypes.POINTER(c_f32)]),
    "bloom_alibi_softmax_fwd": (ctypes.c_int, [c_void_p, c_void_p, c_i64, c_i32, c_i64, c_i32, c_i32,
                                               c_f32, c_void_p]),
    "bloom_alibi_softmax_bwd": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i32, c_i64, c_f32,
                                               c_void_p]),
    "bloom_alibi_attention_fwd": (ctypes.c_int, [c_void_p] * 5 + [c_i64, c_i32, c_i64, c_i32, c_i32, c_i32, c_f32,
                                                 c_void_p]),
    "bloom_alibi_attention_bwd_workspace_size": (c_size, [c_i64, c_i32, c_i64]),
    "bloom_alibi_attention_bwd": (ctypes.c_int, [c_void_p] * 8 + [c_i64, c_i32, c_i64, c_i32, c_i32, c_i32, c_f32,
                                                 c_void_p, c_size, c_void_p]),
    "bloom_bias_gelu_fwd": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p]),
    "bloom_bias_gelu_bwd_workspace_size": (c_size, [c_i64, c_i64]),
    "bloom_bias_gelu_bwd": (ctypes.c_int, [c_void_p] * 6 + [c_size, c_i64, c_i64, c_void_p]),
    "bloom_bf16_grad_accumulate": (ctypes.c_int, [c_void_p, c_void_p, c_i64, c_i32, c_void_p]),
    "bloom_bf16_adamw_workspace_size": (c_size, [c_i64]),
    "bloom_bf16_grad_accumulate_sumsq": (ctypes.c_int, [c_void_p, c_void_p, c_i64, c_i32, c_void_p, c_size,
                                                        c_void_p]),
    "bloom_bf16_grad_accumulate_many": (ctypes.c_int, [c_void_p, ctypes.POINTER(c_void_p), c_i32, c_i64, c_i32,
                                                       c_void_p, c_size, c_void_p]),
    "bloom_bf16_adamw_step": (ctypes.c_int, [c_void_p] * 5 + [c_i64, ctypes.POINTER(AdamWHParams), c_void_p,
                                             c_void_p, c_size, c_void_p]),
    "bloom_bf16_adamw_step_segments": (ctypes.c_int, [c_void_p] * 5 + [c_i64, ctypes.POINTER(AdamWHParams),
                                                      ctypes.POINTER(AdamWSegment), c_i32, c_void_p,
                                                      c_void_p, c_size, c_void_p]),
    "bloom_lr_warmup_cosine": (ctypes.c_int, [c_i64, ctypes.c_double, ctypes.c_double, c_i64, c_i64,
                                              ctypes.POINTER(ctypes.c_double)]),
}

_lib = None


class BloomError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the kernel library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bloom_bf16_optimizer_amd.build` "
                           "(the kernels have no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(name: str, status: int) -> None:
    if status != 0:
        lib = load()
        raise BloomError(name, status, lib.bloom_last_error().decode())
