"""C-ABI contract tests that need no GPU.

The library must load and export every function include/*.h declares, and
argument validation (which runs on the host before anything is enqueued) must
return the documented status for bad input.  No call here reaches a kernel.
"""

import ctypes
import glob
import os
import re

import pytest

from bloom_bf16_optimizer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, WORKSPACE, HPARAM = 0, 1, 2, 3, 4, 5


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(bloom_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libbloomkern.so not built")
    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ["bloom_alibi_attention_fwd", "bloom_alibi_attention_bwd", "bloom_bf16_grad_accumulate_many",
                     "bloom_bf16_adamw_step_segments", "bloom_lr_warmup_cosine",
                     "bloom_layernorm_fwd", "bloom_layernorm_bwd", "bloom_layernorm_residual_fwd",
                     "bloom_layernorm_residual_bwd", "bloom_alibi_softmax_fwd",
                     "bloom_alibi_softmax_bwd", "bloom_bias_gelu_fwd", "bloom_bias_gelu_bwd",
                     "bloom_bf16_grad_accumulate", "bloom_bf16_adamw_step", "bloom_alibi_slopes"]:
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_version_and_strings(lib):
    assert lib.bloom_abi_version() == 8
    assert lib.bloom_status_string(0) == b"ok"
    assert lib.bloom_status_string(4) == b"workspace too small"
    assert lib.bloom_status_string(99) == b"unknown status"


def test_slopes_host_only(lib):
    buf = (ctypes.c_float * 28)()
    assert lib.bloom_alibi_slopes(112, 0, 28, buf) == OK
    assert buf[7] == 0.5 and buf[15] == 0.25
    assert lib.bloom_alibi_slopes(112, 100, 28, buf) == SHAPE
    assert lib.bloom_alibi_slopes(8, 0, 8, None) == NULL


def test_slopes_match_oracle_bit_for_bit(lib):
    import numpy as np
    from oracle.alibi import alibi_slopes_f32
    for total, off, heads in [(8, 0, 8), (16, 0, 16), (112, 0, 28), (112, 84, 28), (112, 0, 112),
                              (6, 0, 6), (1, 0, 1), (100, 0, 100), (256, 0, 256)]:
        buf = (ctypes.c_float * heads)()
        assert lib.bloom_alibi_slopes(total, off, heads, buf) == OK
        got = np.frombuffer(buf, dtype=np.float32)
        assert np.array_equal(got, alibi_slopes_f32(total, off, heads)), (total, off, heads)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails before any launch


def test_layernorm_validation(lib):
    p = FAKE
    f = lib.bloom_layernorm_fwd
    assert f(p, p, p, p, p, p, 4, 12, 1e-5, None) == SHAPE          # hidden not a multiple of 8
    assert f(p, p, p, p, p, p, 4, 0, 1e-5, None) == SHAPE
    assert f(p, p, p, p, p, p, 4, 65544, 1e-5, None) == SHAPE
    assert f(p, p, p, p, p, p, -1, 16, 1e-5, None) == SHAPE
    assert f(p, p, p, p, p, p, 4, 16, 0.0, None) == HPARAM
    assert f(p, p, p, p, p, p, 0, 16, 1e-5, None) == OK              # empty: no-op
    assert f(None, p, p, p, p, p, 4, 16, 1e-5, None) == NULL
    assert f(p + 8, p, p, p, p, p, 4, 16, 1e-5, None) == ALIGN
    assert b"x" in lib.bloom_last_error()
    b = lib.bloom_layernorm_bwd
    assert b(p, p, p, p, p, p, p, p, None, 0, 4, 16, None) == WORKSPACE
    assert b(p, p, p, p, p, p, p, p, p, 16, 4, 16, None) == WORKSPACE
    assert b(p, p, p, p, p, p, p, p, p + 4, 1 << 20, 4, 16, None) == ALIGN
    assert lib.bloom_layernorm_bwd_workspace_size(4, 12) == 0


def test_layernorm_noalloc_validation(lib):
    """The allocation-free backward: host checks before any scratch lookup or launch."""
    p = FAKE
    f = lib.bloom_layernorm_bwd_noalloc
    assert f(p, p, p, p, p, p, p, p, 4, 12, None) == SHAPE
    assert f(p, p, p, p, p, p, p, p, 0, 16, None) == OK               # empty: no-op
    # 256 partial rows of 2 x 65536 floats (128 MiB) exceed the 32 MiB static scratch
    assert lib.bloom_layernorm_bwd_workspace_size(2048, 65536) > (32 << 20)
    assert f(p, p, p, p, p, p, p, p, 2048, 65536, None) == WORKSPACE
    assert b"scratch" in lib.bloom_last_error()
    # BLOOM-176B's width fits
    assert lib.bloom_layernorm_bwd_workspace_size(2048, 14336) <= (32 << 20)


def test_layernorm_residual_validation(lib):
    p = FAKE
    f = lib.bloom_layernorm_residual_fwd
    assert f(p, p, p, p, p, p, p, p, 4, 12, 1e-5, None) == SHAPE
    assert f(p, p, p, p, p, p, p, p, 4, 16, -1.0, None) == HPARAM
    assert f(p, None, p, p, p, p, p, p, 4, 16, 1e-5, None) == NULL
    assert f(p, p, p, p, None, p, p, p, 4, 16, 1e-5, None) == NULL
    assert f(p, p, p, p, p + 8, p, p, p, 4, 16, 1e-5, None) == ALIGN
    assert f(p, p, p, p, p, p, p, p, 0, 16, 1e-5, None) == OK
    b = lib.bloom_layernorm_residual_bwd
    ws = lib.bloom_layernorm_bwd_workspace_size(4, 16)
    assert b(p, None, p, p, p, p, p, p, p, p, ws, 4, 16, None) == NULL
    assert b(p, p, p, p, p, p, p, p, p, p, ws - 16, 4, 16, None) == WORKSPACE
    assert b(p, p, p, p, p, p, p, p, p, p, ws, 0, 16, None) == OK


def test_softmax_validation(lib):
    p = FAKE
    f = lib.bloom_alibi_softmax_fwd
    assert f(p, p, 1, 4, 100, 0, 4, 0.1, None) == SHAPE              # seq not a multiple of 8
    assert f(p, p, 1, 4, 16392, 0, 4, 0.1, None) == SHAPE
    assert f(p, p, 1, 4, 64, 2, 4, 0.1, None) == SHAPE               # heads outside the model
    assert f(p, p, 1, 300, 64, 0, 300, 0.1, None) == SHAPE
    assert f(p, p, 1, 4, 64, 0, 4, float("inf"), None) == HPARAM
    assert f(p, p, 0, 4, 64, 0, 4, 0.1, None) == OK
    assert f(p, None, 1, 4, 64, 0, 4, 0.1, None) == NULL
    g = lib.bloom_alibi_softmax_bwd
    assert g(p, p, p, 1, 4, 60, 0.1, None) == SHAPE
    assert g(p, p, p + 2, 1, 4, 64, 0.1, None) == ALIGN


def test_gelu_validation(lib):
    p = FAKE
    assert lib.bloom_bias_gelu_fwd(p, p, p, 4, 10, None) == SHAPE
    assert lib.bloom_bias_gelu_fwd(p, p, None, 4, 16, None) == NULL
    assert lib.bloom_bias_gelu_fwd(p, p, p, 0, 16, None) == OK
    assert lib.bloom_bias_gelu_bwd(p, p, p, p, p, None, 0, 4, 16, None) == WORKSPACE
    need = lib.bloom_bias_gelu_bwd_workspace_size(100, 64)
    assert need == 4 * 64 * 4  # ceil(100 / 32) partial rows of 64 floats
    assert lib.bloom_bias_gelu_bwd(p, p, p, p, p, p, need - 4, 100, 64, None) == WORKSPACE


def test_optimizer_validation(lib):
    p = FAKE
    hp = _lib.AdamWHParams(6e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 0, 0)
    ws = lib.bloom_bf16_adamw_workspace_size(1000)
    assert ws > 0
    step = lib.bloom_bf16_adamw_step
    assert step(p, p, p, p, p, 1000, None, None, p, ws, None) == NULL
    for field, bad in [("lr", -1.0), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0),
                       ("weight_decay", float("nan")), ("max_grad_norm", 0.0), ("step", 0),
                       ("sumsq_in_workspace", 2), ("reserved", 1)]:
        h = _lib.AdamWHParams(6e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 0, 0)
        setattr(h, field, bad)
        assert step(p, p, p, p, p, 1000, ctypes.byref(h), None, p, ws, None) == HPARAM, field
    assert step(p, p, p, p, p, 1000, ctypes.byref(hp), None, p, ws - 8, None) == WORKSPACE
    assert step(p, p, p, p + 8, p, 1000, ctypes.byref(hp), None, p, ws, None) == ALIGN
    assert step(p, p, p, p, p, 1000, ctypes.byref(hp), p + 2, p, ws, None) == ALIGN
    assert step(p, p, p, p, p, 0, ctypes.byref(hp), None, None, 0, None) == OK
    assert step(p, p, p, p, p, -5, ctypes.byref(hp), None, p, ws, None) == SHAPE
    fused = lib.bloom_bf16_grad_accumulate_sumsq
    assert fused(p, p, 1000, 0, None, 0, None) == WORKSPACE
    assert fused(p, p, 1000, 0, p, ws - 8, None) == WORKSPACE
    assert fused(p, p, 1000, 0, p + 8, ws, None) == ALIGN
    assert fused(p, p, 0, 0, None, 0, None) == OK
    # the workspace holds one FP64 partial per 1024-element workgroup (grid rounded to 8)
    assert lib.bloom_bf16_adamw_workspace_size(3_670_000_000) >= 8 * (3_670_000_000 // 1024)
    acc = lib.bloom_bf16_grad_accumulate
    assert acc(p, p, -1, 1, None) == SHAPE
    assert acc(p, None, 10, 1, None) == NULL
    assert acc(p, p, 0, 0, None) == OK
    many = lib.bloom_bf16_grad_accumulate_many
    ptrs = (ctypes.c_void_p * 17)(*([p] * 17))
    assert many(p, ptrs, 0, 1000, 1, None, 0, None) == SHAPE                # no micro-batch
    assert many(p, ptrs, 17, 1000, 1, None, 0, None) == SHAPE               # more than BLOOM_MAX_ACCUM_BATCH
    assert many(p, None, 2, 1000, 1, None, 0, None) == NULL
    assert many(p, (ctypes.c_void_p * 2)(p, None), 2, 1000, 1, None, 0, None) == NULL
    assert many(p, (ctypes.c_void_p * 2)(p, p + 8), 2, 1000, 1, None, 0, None) == ALIGN
    assert many(p + 4, ptrs, 2, 1000, 1, None, 0, None) == ALIGN
    assert many(p, ptrs, 2, 1000, 1, p, ws - 8, None) == WORKSPACE
    assert many(p, ptrs, 2, -1, 1, None, 0, None) == SHAPE
    assert many(p, ptrs, 2, 0, 1, None, 0, None) == OK                      # empty: nothing enqueued


def test_adamw_segments_validation(lib):
    p = FAKE
    hp = _lib.AdamWHParams(6e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 1, 0, 0)
    ws = lib.bloom_bf16_adamw_workspace_size(1000)
    seg = _lib.AdamWSegment
    step = lib.bloom_bf16_adamw_step_segments

    def call(segs, n=1000):
        arr = (seg * len(segs))(*[seg(*s) for s in segs])
        return step(p, p, p, p, p, n, ctypes.byref(hp), arr, len(segs), None, p, ws, None)

    assert call([(0, 600, 0.01), (608, 392, 0.0)]) == SHAPE        # gap
    assert call([(0, 604, 0.01), (604, 396, 0.0)]) == ALIGN        # second offset not a multiple of 8
    assert call([(0, 600, 0.01), (600, 300, 0.0)]) == SHAPE        # does not reach n
    assert call([(0, 1000, -1.0)]) == HPARAM
    assert call([(0, 1000, float("inf"))]) == HPARAM
    assert step(p, p, p, p, p, 1000, ctypes.byref(hp), None, 1, None, p, ws, None) == NULL
    assert call([(0, 0, 0.01)], n=0) == OK


def test_lr_schedule_host_function_matches_oracle(lib):
    from oracle.optimizer import lr_warmup_cosine
    out = ctypes.c_double()
    for t in [1, 2, 250, 499, 500, 501, 1000, 24875, 50250, 99999, 100000, 123456]:
        assert lib.bloom_lr_warmup_cosine(t, 6e-5, 1e-6, 500, 100000, ctypes.byref(out)) == OK
        want = lr_warmup_cosine(t, 6e-5, 1e-6, 500, 100000)
        assert abs(out.value - want) <= 1e-15 * want, t
    assert lib.bloom_lr_warmup_cosine(7, 1.0, 0.0, 0, 10, ctypes.byref(out)) == OK
    assert abs(out.value - lr_warmup_cosine(7, 1.0, 0.0, 0, 10)) < 1e-16
    assert lib.bloom_lr_warmup_cosine(0, 6e-5, 1e-6, 500, 100000, ctypes.byref(out)) == HPARAM
    assert lib.bloom_lr_warmup_cosine(5, 1e-6, 6e-5, 500, 100000, ctypes.byref(out)) == HPARAM
    assert lib.bloom_lr_warmup_cosine(5, 6e-5, 1e-6, 500, 500, ctypes.byref(out)) == HPARAM
    assert lib.bloom_lr_warmup_cosine(5, 6e-5, 1e-6, 500, 1000, None) == NULL


def test_attention_validation(lib):
    p = FAKE
    f = lib.bloom_alibi_attention_fwd
    assert f(p, p, p, p, p, 1, 4, 100, 128, 0, 4, 0.1, None) == SHAPE       # seq not a multiple of 8
    assert f(p, p, p, p, p, 1, 4, 64, 96, 0, 4, 0.1, None) == SHAPE        # head_dim not 32/64/128
    assert f(p, p, p, p, p, 1, 4, 64, 128, 2, 4, 0.1, None) == SHAPE       # heads outside the model
    assert f(p, p, p, p, p, 1, 4, 64, 128, 0, 4, float("nan"), None) == HPARAM
    assert f(p, p, p, p, p, 1, 4, 64, 128, 0, 4, -0.1, None) == HPARAM    # the scale must be positive
    assert f(p, p, p, p, p, 1, 4, 64, 128, 0, 4, 0.0, None) == HPARAM
    assert f(p, p, p, None, p, 1, 4, 64, 128, 0, 4, 0.1, None) == NULL
    assert f(p, p, p, p + 8, p, 1, 4, 64, 128, 0, 4, 0.1, None) == ALIGN
    assert f(p, p, p, p, p, 0, 4, 64, 128, 0, 4, 0.1, None) == OK           # empty


def test_attention_bwd_validation(lib):
    p = FAKE
    ws = lib.bloom_alibi_attention_bwd_workspace_size(1, 4, 64)
    assert ws >= 4 * 4 * 64 and ws % 256 == 0
    assert lib.bloom_alibi_attention_bwd_workspace_size(-1, 4, 64) == 0
    assert lib.bloom_alibi_attention_bwd_workspace_size(1, 4, 1 << 30) == 0
    f = lib.bloom_alibi_attention_bwd
    ok = (1, 4, 64, 128, 0, 4, 0.1)
    assert f(p, p, p, p, p, p, p, p, 1, 4, 100, 128, 0, 4, 0.1, p, ws, None) == SHAPE   # seq not a multiple of 8
    assert f(p, p, p, p, p, p, p, p, 1, 4, 64, 96, 0, 4, 0.1, p, ws, None) == SHAPE    # head_dim
    assert f(p, p, p, p, p, p, p, p, 1, 4, 64, 128, 2, 4, 0.1, p, ws, None) == SHAPE   # heads outside the model
    assert f(p, p, p, p, p, p, p, p, 1, 4, 64, 128, 0, 4, float("inf"), p, ws, None) == HPARAM
    assert f(p, p, p, p, p, p, p, p, 1, 4, 64, 128, 0, 4, 0.0, p, ws, None) == HPARAM
    assert f(p, p, p, None, p, p, p, p, *ok, p, ws, None) == NULL                         # dout
    assert f(p, p, p, p, p, p, None, p, *ok, p, ws, None) == NULL                         # dk
    assert f(p, p, p, p, p + 4, p, p, p, *ok, p, ws, None) == ALIGN                       # lse
    assert f(p, p, p, p, p, p, p, p, *ok, None, ws, None) == WORKSPACE
    assert f(p, p, p, p, p, p, p, p, *ok, p, ws - 16, None) == WORKSPACE
    assert f(p, p, p, p, p, p, p, p, *ok, p + 8, ws, None) == ALIGN
    assert f(p, p, p, p, p, p, p, p, 0, 4, 64, 128, 0, 4, 0.1, None, 0, None) == OK    # empty: nothing enqueued
