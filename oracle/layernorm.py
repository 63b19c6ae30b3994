"""LayerNorm forward and backward, float64 (oracle; test infrastructure only).

Follows the fused LayerNorm kernel listed under "融合 CUDA 核" on page
"BLOOM 176B 训练技术概览"; the embedding LayerNorm added after the word
embedding ("架构微调", same page; also section 4.3 of page
"企业官网建设流程全解析") is the same computation on embedding rows.

The pages name the operation only.  The standard definition is used: per row
of width H, mean mu = sum(x)/H, biased variance var = sum((x-mu)^2)/H,
r = 1/sqrt(var + eps) with eps inside the square root, x_hat = (x-mu)*r,
y = x_hat*gamma + beta.  The backward of that definition is, with
g = dy*gamma,
    dx     = r * (g - mean(g) - x_hat * mean(g * x_hat))
    dgamma = sum over rows of dy * x_hat
    dbeta  = sum over rows of dy.
The ``*_f64`` functions take and return float64 arrays.  The others take bf16
bit patterns, compute in float64 and round each bf16 output once at the end;
mean and rstd are returned as float32.

Residual form: section 4.3 of page "企业官网建设流程全解析" fuses LayerNorm
with the residual connection (its kernel is a stub taking output, input,
residual, gamma, beta).  Reading used (BLOOM's blocks are pre-LN, so the sum
is also the residual stream the next block adds to): h = bf16(x + r) is
written out, and y = LayerNorm(h) -- the LayerNorm of the rounded sum, so the
fused operation equals "residual add, then LayerNorm" exactly.  Its backward
takes dy and dres (the gradient reaching h through the residual stream) and
returns dh = dLN(dy; h) + dres, rounded once, which is the gradient of both x
and r; dgamma and dbeta are those of the LayerNorm of h.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16, to_f64


def stats_f64(x: np.ndarray, eps: float):
    """Two-pass mean and r = 1/sqrt(var + eps) per row of x [rows, H]."""
    hidden = x.shape[-1]
    mu = x.sum(axis=-1) / hidden
    var = ((x - mu[:, None]) ** 2).sum(axis=-1) / hidden
    r = 1.0 / np.sqrt(var + eps)
    return mu, r


def layernorm_fwd_f64(x, gamma, beta, eps: float):
    """y, mu, r for x [rows, H], gamma [H], beta [H] (float64)."""
    mu, r = stats_f64(x, eps)
    x_hat = (x - mu[:, None]) * r[:, None]
    return x_hat * gamma[None, :] + beta[None, :], mu, r


def layernorm_bwd_f64(dy, x, gamma, eps: float):
    """dx, dgamma, dbeta and dx's condition magnitude (float64).

    The magnitude r*(|g| + mean|g| + |x_hat|*mean|g*x_hat| + |mean(g*x_hat)|*r*|mu|)
    bounds, times a few float32 units of roundoff per reduction level, the
    error any float32 evaluation of dx can make.
    """
    mu, r = stats_f64(x, eps)
    x_hat = (x - mu[:, None]) * r[:, None]
    g = dy * gamma[None, :]
    mean_g = g.mean(axis=-1)
    mean_gx = (g * x_hat).mean(axis=-1)
    dx = r[:, None] * (g - mean_g[:, None] - x_hat * mean_gx[:, None])
    dgamma = (dy * x_hat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    terms = r[:, None] * (np.abs(g) + np.abs(g).mean(axis=-1)[:, None]
                          + np.abs(x_hat) * np.abs(g * x_hat).mean(axis=-1)[:, None]
                          + (np.abs(mean_gx) * r * np.abs(mu))[:, None])
    return dx, dgamma, dbeta, terms


def _eps64(eps: float) -> float:
    """eps as the float32 value the GPU receives, widened exactly."""
    return float(np.float32(eps))


def layernorm_fwd(x_bits, gamma_bits, beta_bits, eps: float, return_f64: bool = False):
    """y (bf16 bits), mean (float32), rstd (float32) for x [rows, H] (bf16 bits).

    With ``return_f64`` also returns (y, |gamma|*r*mean|x| + |x_hat*gamma| +
    |beta|) in float64: the unrounded output and its condition magnitude (the
    first term carries the rounding of the row mean through x - mu).
    """
    x = to_f64(x_bits)
    gamma = to_f64(gamma_bits)
    beta = to_f64(beta_bits)
    y, mu, r = layernorm_fwd_f64(x, gamma, beta, _eps64(eps))
    out = (round_to_bf16(y), mu.astype(np.float32), r.astype(np.float32))
    if not return_f64:
        return out
    x_hat_gamma = y - beta[None, :]
    terms = (np.abs(gamma)[None, :] * (r * np.abs(x).mean(axis=-1))[:, None] + np.abs(x_hat_gamma)
             + np.abs(beta)[None, :])
    return out, (y, terms)


def layernorm_bwd(dy_bits, x_bits, gamma_bits, eps: float, return_f64: bool = False):
    """dx, dgamma, dbeta as bf16 bits.

    Statistics are recomputed in float64 from x, not taken from the forward's
    float32 outputs.  With ``return_f64`` the float64 results and term
    magnitudes are returned too: (dx, dgamma, dbeta, dx_terms,
    (sum|dy x_hat|, sum|dy|)).
    """
    x = to_f64(x_bits)
    dy = to_f64(dy_bits)
    eps64 = _eps64(eps)
    dx, dgamma, dbeta, terms = layernorm_bwd_f64(dy, x, to_f64(gamma_bits), eps64)
    out = (round_to_bf16(dx), round_to_bf16(dgamma), round_to_bf16(dbeta))
    if not return_f64:
        return out
    mu, r = stats_f64(x, eps64)
    x_hat = (x - mu[:, None]) * r[:, None]
    col_terms = (np.abs(dy * x_hat).sum(axis=0), np.abs(dy).sum(axis=0))
    return out, (dx, dgamma, dbeta, terms, col_terms)


def residual_add(x_bits, r_bits):
    """h = x + r rounded once to bf16 (the sum of two bf16 values is exact in float64)."""
    return round_to_bf16(to_f64(x_bits) + to_f64(r_bits))


def layernorm_residual_fwd(x_bits, r_bits, gamma_bits, beta_bits, eps: float, return_f64: bool = False):
    """(h, y, mean, rstd): h = bf16(x + r) and the LayerNorm of h.

    With ``return_f64`` returns ((h, y, mean, rstd), (y_f64, y_terms)) as
    layernorm_fwd does for the normalised part.
    """
    h = residual_add(x_bits, r_bits)
    res = layernorm_fwd(h, gamma_bits, beta_bits, eps, return_f64=return_f64)
    if not return_f64:
        return (h,) + tuple(res)
    (y, mu, r), f64 = res
    return (h, y, mu, r), f64


def layernorm_residual_bwd_f64(dy, dres, h, gamma, eps: float):
    """dh = dLN(dy; h) + dres, dgamma, dbeta and dh's condition magnitude (float64)."""
    dx, dgamma, dbeta, terms = layernorm_bwd_f64(dy, h, gamma, eps)
    return dx + dres, dgamma, dbeta, terms + np.abs(dres)


def layernorm_residual_bwd(dy_bits, dres_bits, h_bits, gamma_bits, eps: float, return_f64: bool = False):
    """dh, dgamma, dbeta as bf16 bits (statistics recomputed in float64 from h).

    With ``return_f64`` also returns (dh, dgamma, dbeta, dh_terms,
    (sum|dy x_hat|, sum|dy|)) in float64.
    """
    h = to_f64(h_bits)
    dy = to_f64(dy_bits)
    eps64 = _eps64(eps)
    dh, dgamma, dbeta, terms = layernorm_residual_bwd_f64(dy, to_f64(dres_bits), h, to_f64(gamma_bits), eps64)
    out = (round_to_bf16(dh), round_to_bf16(dgamma), round_to_bf16(dbeta))
    if not return_f64:
        return out
    mu, r = stats_f64(h, eps64)
    x_hat = (h - mu[:, None]) * r[:, None]
    col_terms = (np.abs(dy * x_hat).sum(axis=0), np.abs(dy).sum(axis=0))
    return out, (dh, dgamma, dbeta, terms, col_terms)
