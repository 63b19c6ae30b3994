"""BF16Optimizer step: FP32 gradient accumulation, global-norm clip, AdamW, bf16 copy.

Oracle; test infrastructure only.  Sources on the pages:

* page "BLOOM 176B 训练技术概览", section "BF16 优化器": BF16 mixed precision
  with a custom BF16Optimizer that accumulates in FP32 and accumulates the
  gradients of the pipeline micro-batches in FP32;
* page "企业官网建设流程全解析": section 3.3's DeepSpeed config (32 gradient
  accumulation steps, AdamW with lr 6e-5 and weight decay 0.01), section 1's
  FP32 master parameters and moments, section 4.3's global-norm clipping at 1.0;
* page "单机多卡实战：Megatron-DeepSpeed训练类BLOOM模型全流程解析", section 3's
  training config (lr 6e-5, weight decay 0.01, clip_grad 1.0, bf16).

Readings where the pages are silent:

* accumulation: the first micro-batch sets acc = float32(g_1); each later one
  does acc = acc + float32(g_k) as one float32 add, in micro-batch order.  That
  is the defined float32 result, so it is replicated exactly (NumPy float32
  adds are IEEE round-to-nearest-even);
* norm: N = sqrt(sum acc^2), float64;
* clip: c = max_norm / N when N > max_norm, else 1 (a NaN norm compares false
  and leaves c = 1; an infinite norm gives c = 0);
* AdamW (Loshchilov and Hutter, decoupled weight decay) with bias correction,
  step t counted from 1 and eps added to the corrected root:
      g  = c * acc
      m' = b1 m + (1 - b1) g
      v' = b2 v + (1 - b2) g^2
      p' = p - lr * ( (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps) + wd * p )
  evaluated in float64 from the float32 state and the float64 hyperparameters,
  then rounded once to float32;
* bf16 parameter copy: round-to-nearest-even of the float32 master.

Parameter groups and schedule (the "optimizer group splitting" named among the
engineering challenges on page "BLOOM 176B 训练技术概览"; page
"单机多卡实战：Megatron-DeepSpeed训练类BLOOM模型全流程解析", section 3's config:
lr 6e-5, min_lr 1e-6, cosine decay, 500 warmup iterations, 100000 train
iterations).  Readings:

* groups are contiguous segments of the flat buffers, each with its own
  weight decay (e.g. none on biases and LayerNorm weights); the norm and the
  clip coefficient stay global over all segments;
* lr at optimizer step t (1-based): t * max_lr / warmup while t <= warmup;
  then min_lr + (max_lr - min_lr) * (1 + cos(pi * (t - warmup) /
  (decay - warmup))) / 2 up to t = decay (the train iterations); min_lr after.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16


def grad_accumulate(acc, grad_bits, first: bool) -> np.ndarray:
    """One micro-batch: returns the new float32 accumulator."""
    g = (np.asarray(grad_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if first:
        return g.copy()
    acc = np.asarray(acc, dtype=np.float32)
    return (acc + g).astype(np.float32)


def global_norm(acc) -> float:
    a = np.asarray(acc, dtype=np.float32).astype(np.float64)
    return float(np.sqrt(np.dot(a, a)))


def sum_of_squares(acc) -> float:
    a = np.asarray(acc, dtype=np.float32).astype(np.float64)
    return float(np.dot(a, a))


def clip_coefficient(norm: float, max_norm: float) -> float:
    if norm > max_norm:
        return max_norm / norm
    return 1.0


def adamw_f64(p, m, v, g, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, step: int):
    """One AdamW update on float64 arrays; g is the already clipped gradient."""
    m1 = beta1 * m + (1.0 - beta1) * g
    v1 = beta2 * v + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    p1 = p - lr * ((m1 / bc1) / (np.sqrt(v1 / bc2) + eps) + weight_decay * p)
    return p1, m1, v1


def adamw_update(master, m, v, acc, clip: float, lr: float, beta1: float,
                 beta2: float, eps: float, weight_decay: float, step: int,
                 return_f64: bool = False):
    """AdamW on float32 state; returns (master', m', v' as float32, param bf16 bits).

    The float32 state and accumulator are widened exactly, the update is
    evaluated in float64 and each result is rounded once to float32.  With
    ``return_f64`` also returns the float64 values and the term magnitudes used
    by term-scaled comparisons: for p, |p'| + |p|; for m, |m'| + b1|m| +
    (1-b1)|g|; for v, |v'|.
    """
    p = np.asarray(master, dtype=np.float32).astype(np.float64)
    m0 = np.asarray(m, dtype=np.float32).astype(np.float64)
    v0 = np.asarray(v, dtype=np.float32).astype(np.float64)
    g = clip * np.asarray(acc, dtype=np.float32).astype(np.float64)
    p1, m1, v1 = adamw_f64(p, m0, v0, g, lr, beta1, beta2, eps, weight_decay, step)
    p1_32 = p1.astype(np.float32)
    out = (p1_32, m1.astype(np.float32), v1.astype(np.float32), round_to_bf16(p1_32))
    if not return_f64:
        return out
    terms = (np.abs(p1) + np.abs(p),
             np.abs(m1) + beta1 * np.abs(m0) + (1.0 - beta1) * np.abs(g),
             np.abs(v1))
    return out, (p1, m1, v1), terms


def bf16_optimizer_step(master, m, v, acc, lr: float, beta1: float, beta2: float,
                        eps: float, weight_decay: float, max_grad_norm: float, step: int):
    """Norm, clip, AdamW and bf16 copy in that order.

    Returns (master', m', v', param bf16 bits, N, c).
    """
    norm = global_norm(acc)
    c = clip_coefficient(norm, max_grad_norm)
    p1, m1, v1, pb = adamw_update(master, m, v, acc, c, lr, beta1, beta2, eps, weight_decay, step)
    return p1, m1, v1, pb, norm, c


def bf16_optimizer_step_segments(master, m, v, acc, segments, lr: float, beta1: float, beta2: float,
                                 eps: float, max_grad_norm: float, step: int):
    """Global norm and clip over all of acc, then AdamW per segment (offset, length, weight_decay).

    Returns (master', m', v', param bf16 bits, N, c).
    """
    norm = global_norm(acc)
    c = clip_coefficient(norm, max_grad_norm)
    p1 = np.empty(len(acc), dtype=np.float32)
    m1, v1 = np.empty_like(p1), np.empty_like(p1)
    pb = np.empty(len(acc), dtype=np.uint16)
    for off, length, wd in segments:
        sl = slice(off, off + length)
        p1[sl], m1[sl], v1[sl], pb[sl] = adamw_update(master[sl], m[sl], v[sl], acc[sl], c, lr, beta1, beta2,
                                                      eps, wd, step)
    return p1, m1, v1, pb, norm, c


def lr_warmup_cosine(step: int, max_lr: float, min_lr: float, warmup: int, decay: int) -> float:
    """Learning rate at optimizer step ``step`` (1-based), float64."""
    if warmup > 0 and step <= warmup:
        return max_lr * step / warmup
    if step >= decay:
        return min_lr
    ratio = (step - warmup) / (decay - warmup)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + np.cos(np.pi * ratio))
