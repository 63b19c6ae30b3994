"""Fused causal attention with the ALiBi bias, float64 (oracle; test infrastructure only).

What is computed: the attention of BLOOM's blocks with the ALiBi linear bias
in place of position embeddings (page "BLOOM 176B 训练技术概览", section
"架构微调"; trained at 2048 tokens and extrapolated to 8192, section 4.3 of
page "企业官网建设流程全解析"), i.e. the combined scale + mask + softmax of
"融合 CUDA 核" on the same page applied between Q K^T and V, for each batch b
and head h of the heads one tensor-parallel rank holds:

    z_ij   = scale * (q_i . k_j) - slope_h * (i - j)     for j <= i,  -inf for j > i
    o_i    = sum_j softmax_j(z_i) v_j
    lse_i  = log sum_{j <= i} exp(z_ij)                  (natural log; kept for the backward)

Readings: the scale multiplies q.k only (as in the fused softmax); the slopes
are the ALiBi paper's (see oracle/alibi.py) for the rank's contiguous head
range.  Arithmetic is float64 on the bf16 inputs widened exactly; scale and
the slopes are the float32 values the GPU receives.  ``terms`` is the
condition magnitude sum_j p_ij |v_jd| of each output element.
"""

from __future__ import annotations

import numpy as np

from .alibi import alibi_slopes_f32
from .bf16 import round_to_bf16, to_f64


def attention_fwd_f64(q, k, v, slopes, scale: float, rows=None):
    """q, k, v [B, H, L, D] float64, slopes [H]; rows: query indices to compute (default all).

    Returns (o [B, H, R, D], lse [B, H, R], terms [B, H, R, D]).
    """
    nb, nh, length, dim = q.shape
    qi = np.arange(length) if rows is None else np.asarray(rows)
    j = np.arange(length)[None, :]
    dist = (qi[:, None] - j).astype(np.float64)
    o = np.empty((nb, nh, len(qi), dim))
    lse = np.empty((nb, nh, len(qi)))
    terms = np.empty_like(o)
    for b in range(nb):
        for h in range(nh):
            z = scale * (q[b, h][qi] @ k[b, h].T) - slopes[h] * dist
            z[j > qi[:, None]] = -np.inf
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            ssum = e.sum(axis=1, keepdims=True)
            p = e / ssum
            o[b, h] = p @ v[b, h]
            lse[b, h] = (m + np.log(ssum))[:, 0]
            terms[b, h] = p @ np.abs(v[b, h])
    return o, lse, terms


def attention_fwd(q_bits, k_bits, v_bits, total_heads: int, head_offset: int, scale: float, rows=None,
                  return_f64: bool = False):
    """o as bf16 bits and lse as float32 for bf16 q, k, v [B, H, L, D].

    With ``return_f64`` also returns (o_f64, lse_f64, terms).
    """
    nh = q_bits.shape[1]
    slopes = alibi_slopes_f32(total_heads, head_offset, nh).astype(np.float64)
    o, lse, terms = attention_fwd_f64(to_f64(q_bits), to_f64(k_bits), to_f64(v_bits), slopes,
                                      float(np.float32(scale)), rows)
    out = (round_to_bf16(o), lse.astype(np.float32))
    if not return_f64:
        return out
    return out, (o, lse, terms)
