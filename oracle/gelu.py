"""bias + GeLU forward and backward, float64 (oracle; test infrastructure only).

Follows the "bias + GeLU" fusion listed under "融合 CUDA 核" on page
"BLOOM 176B 训练技术概览" (the MLP's GeLU(XA) of section 2.1 on page
"企业官网建设流程全解析").  The pages do not write GeLU out; the tanh form of
the GELU paper (Hendrycks and Gimpel, arXiv:1606.08415) is used:
    u = x + b,   a = k (u + c u^3),   k = sqrt(2/pi), c = 0.044715
    y = u/2 * (1 + tanh(a))
    y'(u) = (1 + tanh a)/2 + u/2 * (1 - tanh(a)^2) * k * (1 + 3 c u^2)
    dx = dy * y'(u),      dbias = sum over rows of dx (unrounded).
Evaluation.  For a << 0, 1 + tanh(a) cancels in float64 (it is exactly 0 once
a < -19 although the true value is 2 e^(2a)), so the same quantities are
evaluated through the exact identities
    (1 + tanh a)/2 = 1/(1 + e^(-2a)) = s,   1 - tanh(a)^2 = 4 s (1 - s),
    1 - s = 1/(1 + e^(2a)),
which have no cancellation anywhere:  y = u s,  y' = s + 2 k u (1 + 3 c u^2) s (1 - s).
u = x + b is exact in float64.  Outputs are rounded once to bf16.
"""

from __future__ import annotations

import math

import numpy as np

from .bf16 import round_to_bf16, to_f64

K = math.sqrt(2.0 / math.pi)
C = 0.044715


def _s_and_complement(u):
    """s = (1 + tanh a)/2 and 1 - s, each without cancellation."""
    a = K * (u + C * u ** 3)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-2.0 * a))
        sc = 1.0 / (1.0 + np.exp(2.0 * a))
    return s, sc


def gelu(u):
    s, _ = _s_and_complement(u)
    return u * s


def gelu_grad(u):
    s, sc = _s_and_complement(u)
    return s + 2.0 * K * u * (1.0 + 3.0 * C * u * u) * s * sc


def gelu_grad_terms(u):
    """Magnitudes of the two terms of gelu_grad, summed."""
    s, sc = _s_and_complement(u)
    return np.abs(s) + np.abs(2.0 * K * u * (1.0 + 3.0 * C * u * u) * s * sc)


def bias_gelu_fwd(x_bits, bias_bits, return_f64: bool = False):
    """y (bf16 bits) for x [rows, cols], bias [cols] (bf16 bits).

    With ``return_f64`` also returns the unrounded float64 y.
    """
    u = to_f64(x_bits) + to_f64(bias_bits)[None, :]
    y = gelu(u)
    return (round_to_bf16(y), y) if return_f64 else round_to_bf16(y)


def bias_gelu_bwd(dy_bits, x_bits, bias_bits, return_f64: bool = False):
    """dx and dbias as bf16 bits.

    With ``return_f64`` also returns (dx, dbias, per-element magnitude of dx's
    terms, column sums of |dx|) in float64.
    """
    u = to_f64(x_bits) + to_f64(bias_bits)[None, :]
    dy = to_f64(dy_bits)
    dx = dy * gelu_grad(u)
    dbias = dx.sum(axis=0)
    out = (round_to_bf16(dx), round_to_bf16(dbias))
    if not return_f64:
        return out
    return out, (dx, dbias, np.abs(dy) * gelu_grad_terms(u), np.abs(dx).sum(axis=0))
