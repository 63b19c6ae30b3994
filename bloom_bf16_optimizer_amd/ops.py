"""Python binding of the C ABI, one function per entry point, same names.

Each function takes PyTorch tensors that already live on the GPU, checks
dtype, device, contiguity and shape agreement, and passes raw pointers, sizes
and the current HIP stream to the library.  Outputs are caller-allocated
tensors, written in place; nothing is computed here.  There is no CPU
fallback: a missing library or a non-GPU tensor raises.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import AdamWHParams, AdamWSegment, check

BF16 = torch.bfloat16
F32 = torch.float32


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None, dtype: torch.dtype, name: str) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _rows_cols(t: torch.Tensor) -> tuple[int, int]:
    return (t.numel() // t.shape[-1], t.shape[-1]) if t.dim() > 0 else (0, 0)


def _same(a: torch.Tensor, b: torch.Tensor, what: str) -> None:
    if a.shape != b.shape:
        raise ValueError(f"{what}: shapes {tuple(a.shape)} and {tuple(b.shape)} differ")


def bloom_abi_version() -> int:
    return _lib.load().bloom_abi_version()


def bloom_alibi_slopes(total_heads: int, head_offset: int, heads: int) -> list[float]:
    lib = _lib.load()
    buf = (ctypes.c_float * max(heads, 1))()
    check("bloom_alibi_slopes", lib.bloom_alibi_slopes(total_heads, head_offset, heads, buf))
    return [buf[k] for k in range(heads)]


def bloom_layernorm_fwd(x, gamma, beta, y, mean, rstd, eps: float) -> None:
    rows, hidden = _rows_cols(x)
    _same(x, y, "x/y")
    if gamma.numel() != hidden or beta.numel() != hidden or mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("gamma/beta must have `hidden` and mean/rstd `rows` elements")
    lib = _lib.load()
    check("bloom_layernorm_fwd", lib.bloom_layernorm_fwd(
        _ptr(x, BF16, "x"), _ptr(gamma, BF16, "gamma"), _ptr(beta, BF16, "beta"), _ptr(y, BF16, "y"),
        _ptr(mean, F32, "mean"), _ptr(rstd, F32, "rstd"), rows, hidden, eps, _stream()))


def bloom_layernorm_bwd_workspace_size(rows: int, hidden: int) -> int:
    return _lib.load().bloom_layernorm_bwd_workspace_size(rows, hidden)


def bloom_layernorm_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace) -> None:
    rows, hidden = _rows_cols(x)
    _same(x, dy, "x/dy")
    _same(x, dx, "x/dx")
    if gamma.numel() != hidden or dgamma.numel() != hidden or dbeta.numel() != hidden:
        raise ValueError("gamma/dgamma/dbeta must have `hidden` elements")
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must have `rows` elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_layernorm_bwd", lib.bloom_layernorm_bwd(
        _ptr(dy, BF16, "dy"), _ptr(x, BF16, "x"), _ptr(gamma, BF16, "gamma"), _ptr(mean, F32, "mean"),
        _ptr(rstd, F32, "rstd"), _ptr(dx, BF16, "dx"), _ptr(dgamma, BF16, "dgamma"),
        _ptr(dbeta, BF16, "dbeta"), _ptr(workspace, workspace.dtype, "workspace"), wsb, rows, hidden,
        _stream()))


def bloom_layernorm_bwd_noalloc(dy, x, gamma, mean, rstd, dx, dgamma, dbeta) -> None:
    """bloom_layernorm_bwd without a workspace (the library's static scratch)."""
    rows, hidden = _rows_cols(x)
    _same(x, dy, "x/dy")
    _same(x, dx, "x/dx")
    if gamma.numel() != hidden or dgamma.numel() != hidden or dbeta.numel() != hidden:
        raise ValueError("gamma/dgamma/dbeta must have `hidden` elements")
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must have `rows` elements")
    lib = _lib.load()
    check("bloom_layernorm_bwd_noalloc", lib.bloom_layernorm_bwd_noalloc(
        _ptr(dy, BF16, "dy"), _ptr(x, BF16, "x"), _ptr(gamma, BF16, "gamma"), _ptr(mean, F32, "mean"),
        _ptr(rstd, F32, "rstd"), _ptr(dx, BF16, "dx"), _ptr(dgamma, BF16, "dgamma"),
        _ptr(dbeta, BF16, "dbeta"), rows, hidden, _stream()))


def bloom_layernorm_residual_fwd(x, residual, gamma, beta, h, y, mean, rstd, eps: float) -> None:
    rows, hidden = _rows_cols(x)
    for t, name in ((residual, "residual"), (h, "h"), (y, "y")):
        _same(x, t, f"x/{name}")
    if gamma.numel() != hidden or beta.numel() != hidden or mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("gamma/beta must have `hidden` and mean/rstd `rows` elements")
    lib = _lib.load()
    check("bloom_layernorm_residual_fwd", lib.bloom_layernorm_residual_fwd(
        _ptr(x, BF16, "x"), _ptr(residual, BF16, "residual"), _ptr(gamma, BF16, "gamma"),
        _ptr(beta, BF16, "beta"), _ptr(h, BF16, "h"), _ptr(y, BF16, "y"), _ptr(mean, F32, "mean"),
        _ptr(rstd, F32, "rstd"), rows, hidden, eps, _stream()))


def bloom_layernorm_residual_bwd(dy, dres, h, gamma, mean, rstd, dh, dgamma, dbeta, workspace) -> None:
    rows, hidden = _rows_cols(h)
    for t, name in ((dy, "dy"), (dres, "dres"), (dh, "dh")):
        _same(h, t, f"h/{name}")
    if gamma.numel() != hidden or dgamma.numel() != hidden or dbeta.numel() != hidden:
        raise ValueError("gamma/dgamma/dbeta must have `hidden` elements")
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must have `rows` elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_layernorm_residual_bwd", lib.bloom_layernorm_residual_bwd(
        _ptr(dy, BF16, "dy"), _ptr(dres, BF16, "dres"), _ptr(h, BF16, "h"), _ptr(gamma, BF16, "gamma"),
        _ptr(mean, F32, "mean"), _ptr(rstd, F32, "rstd"), _ptr(dh, BF16, "dh"), _ptr(dgamma, BF16, "dgamma"),
        _ptr(dbeta, BF16, "dbeta"), _ptr(workspace, workspace.dtype, "workspace"), wsb, rows, hidden,
        _stream()))


def _softmax_shape(t: torch.Tensor):
    if t.dim() != 4 or t.shape[2] != t.shape[3]:
        raise ValueError("scores must be [batch, heads, seq, seq]")
    return t.shape[0], t.shape[1], t.shape[2]


def bloom_alibi_softmax_fwd(scores, probs, head_offset: int, total_heads: int, scale: float) -> None:
    b, h, s = _softmax_shape(scores)
    _same(scores, probs, "scores/probs")
    lib = _lib.load()
    check("bloom_alibi_softmax_fwd", lib.bloom_alibi_softmax_fwd(
        _ptr(scores, BF16, "scores"), _ptr(probs, BF16, "probs"), b, h, s, head_offset, total_heads,
        scale, _stream()))


def bloom_alibi_softmax_bwd(probs, dprobs, dscores, scale: float) -> None:
    b, h, s = _softmax_shape(probs)
    _same(probs, dprobs, "probs/dprobs")
    _same(probs, dscores, "probs/dscores")
    lib = _lib.load()
    check("bloom_alibi_softmax_bwd", lib.bloom_alibi_softmax_bwd(
        _ptr(probs, BF16, "probs"), _ptr(dprobs, BF16, "dprobs"), _ptr(dscores, BF16, "dscores"),
        b, h, s, scale, _stream()))


def bloom_alibi_attention_fwd(q, k, v, o, lse, head_offset: int, total_heads: int, scale: float) -> None:
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, seq, head_dim]")
    b, h, s, d = q.shape
    for t, name in ((k, "k"), (v, "v"), (o, "o")):
        _same(q, t, f"q/{name}")
    if lse.numel() != b * h * s:
        raise ValueError("lse must have batch*heads*seq elements")
    lib = _lib.load()
    check("bloom_alibi_attention_fwd", lib.bloom_alibi_attention_fwd(
        _ptr(q, BF16, "q"), _ptr(k, BF16, "k"), _ptr(v, BF16, "v"), _ptr(o, BF16, "o"), _ptr(lse, F32, "lse"),
        b, h, s, d, head_offset, total_heads, scale, _stream()))


def bloom_alibi_attention_bwd_workspace_size(batch: int, heads: int, seq: int) -> int:
    return _lib.load().bloom_alibi_attention_bwd_workspace_size(batch, heads, seq)


def bloom_alibi_attention_bwd(q, k, v, dout, lse, dq, dk, dv, head_offset: int, total_heads: int, scale: float,
                              workspace) -> None:
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, seq, head_dim]")
    b, h, s, d = q.shape
    for t, name in ((k, "k"), (v, "v"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _same(q, t, f"q/{name}")
    if lse.numel() != b * h * s:
        raise ValueError("lse must have batch*heads*seq elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_alibi_attention_bwd", lib.bloom_alibi_attention_bwd(
        _ptr(q, BF16, "q"), _ptr(k, BF16, "k"), _ptr(v, BF16, "v"), _ptr(dout, BF16, "dout"),
        _ptr(lse, F32, "lse"), _ptr(dq, BF16, "dq"), _ptr(dk, BF16, "dk"), _ptr(dv, BF16, "dv"),
        b, h, s, d, head_offset, total_heads, scale, _ptr(workspace, workspace.dtype, "workspace"), wsb, _stream()))


def bloom_bias_gelu_fwd(x, bias, y) -> None:
    rows, cols = _rows_cols(x)
    _same(x, y, "x/y")
    if bias.numel() != cols:
        raise ValueError("bias must have `cols` elements")
    lib = _lib.load()
    check("bloom_bias_gelu_fwd", lib.bloom_bias_gelu_fwd(
        _ptr(x, BF16, "x"), _ptr(bias, BF16, "bias"), _ptr(y, BF16, "y"), rows, cols, _stream()))


def bloom_bias_gelu_bwd_workspace_size(rows: int, cols: int) -> int:
    return _lib.load().bloom_bias_gelu_bwd_workspace_size(rows, cols)


def bloom_bias_gelu_bwd(dy, x, bias, dx, dbias, workspace) -> None:
    rows, cols = _rows_cols(x)
    _same(x, dy, "x/dy")
    _same(x, dx, "x/dx")
    if bias.numel() != cols or dbias.numel() != cols:
        raise ValueError("bias/dbias must have `cols` elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_bias_gelu_bwd", lib.bloom_bias_gelu_bwd(
        _ptr(dy, BF16, "dy"), _ptr(x, BF16, "x"), _ptr(bias, BF16, "bias"), _ptr(dx, BF16, "dx"),
        _ptr(dbias, BF16, "dbias"), _ptr(workspace, workspace.dtype, "workspace"), wsb, rows, cols,
        _stream()))


def bloom_bf16_grad_accumulate(grad_acc, grad, first_microbatch: bool) -> None:
    if grad_acc.numel() != grad.numel():
        raise ValueError("grad_acc and grad must have the same number of elements")
    lib = _lib.load()
    check("bloom_bf16_grad_accumulate", lib.bloom_bf16_grad_accumulate(
        _ptr(grad_acc, F32, "grad_acc"), _ptr(grad, BF16, "grad"), grad.numel(), int(bool(first_microbatch)),
        _stream()))


def bloom_bf16_grad_accumulate_sumsq(grad_acc, grad, first_microbatch: bool, workspace) -> None:
    if grad_acc.numel() != grad.numel():
        raise ValueError("grad_acc and grad must have the same number of elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_bf16_grad_accumulate_sumsq", lib.bloom_bf16_grad_accumulate_sumsq(
        _ptr(grad_acc, F32, "grad_acc"), _ptr(grad, BF16, "grad"), grad.numel(), int(bool(first_microbatch)),
        _ptr(workspace, workspace.dtype, "workspace"), wsb, _stream()))


def bloom_bf16_grad_accumulate_many(grad_acc, grads, first_microbatch: bool, workspace=None) -> None:
    """grad_acc accumulates the bf16 tensors of `grads` in order (one pass)."""
    grads = list(grads)
    for k, g in enumerate(grads):
        if g.numel() != grad_acc.numel():
            raise ValueError(f"grads[{k}] and grad_acc must have the same number of elements")
    arr = (ctypes.c_void_p * max(len(grads), 1))(*[_ptr(g, BF16, f"grads[{k}]") for k, g in enumerate(grads)])
    wptr, wsb = None, 0
    if workspace is not None:
        wptr, wsb = _ptr(workspace, workspace.dtype, "workspace"), workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_bf16_grad_accumulate_many", lib.bloom_bf16_grad_accumulate_many(
        _ptr(grad_acc, F32, "grad_acc"), arr, len(grads), grad_acc.numel(), int(bool(first_microbatch)), wptr, wsb,
        _stream()))


def bloom_bf16_adamw_workspace_size(n: int) -> int:
    return _lib.load().bloom_bf16_adamw_workspace_size(n)


def adamw_hparams(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                  max_grad_norm: float, step: int, sumsq_in_workspace: bool = False) -> AdamWHParams:
    return AdamWHParams(lr, beta1, beta2, eps, weight_decay, max_grad_norm, step, int(bool(sumsq_in_workspace)), 0)


def bloom_bf16_adamw_step(master, exp_avg, exp_avg_sq, param_bf16, grad_acc, hp: AdamWHParams,
                          grad_norm_out, workspace) -> None:
    n = master.numel()
    for t, name in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (param_bf16, "param_bf16"),
                    (grad_acc, "grad_acc")):
        if t.numel() != n:
            raise ValueError(f"{name} must have {n} elements")
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_bf16_adamw_step", lib.bloom_bf16_adamw_step(
        _ptr(master, F32, "master"), _ptr(exp_avg, F32, "exp_avg"), _ptr(exp_avg_sq, F32, "exp_avg_sq"),
        _ptr(param_bf16, BF16, "param_bf16"), _ptr(grad_acc, F32, "grad_acc"), n, ctypes.byref(hp),
        _ptr(grad_norm_out, F32, "grad_norm_out"), _ptr(workspace, workspace.dtype, "workspace"), wsb,
        _stream()))


def bloom_bf16_adamw_step_segments(master, exp_avg, exp_avg_sq, param_bf16, grad_acc, hp: AdamWHParams,
                                   segments, grad_norm_out, workspace) -> None:
    """segments: sequence of (offset, length, weight_decay) tiling [0, n)."""
    n = master.numel()
    for t, name in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (param_bf16, "param_bf16"),
                    (grad_acc, "grad_acc")):
        if t.numel() != n:
            raise ValueError(f"{name} must have {n} elements")
    segs = (AdamWSegment * max(len(segments), 1))(*[AdamWSegment(int(o), int(l), float(w))
                                                     for o, l, w in segments])
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    check("bloom_bf16_adamw_step_segments", lib.bloom_bf16_adamw_step_segments(
        _ptr(master, F32, "master"), _ptr(exp_avg, F32, "exp_avg"), _ptr(exp_avg_sq, F32, "exp_avg_sq"),
        _ptr(param_bf16, BF16, "param_bf16"), _ptr(grad_acc, F32, "grad_acc"), n, ctypes.byref(hp), segs,
        len(segments), _ptr(grad_norm_out, F32, "grad_norm_out"), _ptr(workspace, workspace.dtype, "workspace"),
        wsb, _stream()))


def bloom_lr_warmup_cosine(step: int, max_lr: float, min_lr: float, warmup_steps: int, decay_steps: int) -> float:
    out = ctypes.c_double()
    lib = _lib.load()
    check("bloom_lr_warmup_cosine", lib.bloom_lr_warmup_cosine(step, max_lr, min_lr, warmup_steps, decay_steps,
                                                               ctypes.byref(out)))
    return out.value
