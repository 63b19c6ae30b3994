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

Backward.  The gradient of the same function with respect to q, k and v for
an upstream gradient do_i of each output row (the training step runs every
forward kernel backward as well, "融合 CUDA 核"), written out with the
softmax Jacobian:

    p_ij  = softmax_j(z_i)                      (0 for j > i)
    dp_ij = do_i . v_j
    ds_ij = p_ij * (dp_ij - sum_k p_ik dp_ik)   (the softmax backward)
    dq_i  = scale * sum_j ds_ij k_j
    dk_j  = scale * sum_i ds_ij q_i
    dv_j  = sum_i p_ij do_i

The slope term has no parameters, so it only enters through p.  The condition
magnitudes bound what a kernel that rounds p and ds to bf16 for its products,
and forms sum_k p_ik dp_ik as do_i . o_i from a bf16 o, can lose: with
A_i = sum_d |do_id| (|o_id| + sum_j p_ij |v_jd|),
    tq_id = scale * sum_j (|ds_ij| + p_ij A_i) |k_jd|,
    tk_jd = scale * sum_i (|ds_ij| + p_ij A_i) |q_id|,
    tv_jd = sum_i p_ij |do_id|.
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


def attention_bwd_f64(q, k, v, do, slopes, scale: float, qrows=None, krows=None, chunk: int = 512):
    """Exact gradients for q, k, v, do [B, H, L, D] float64 and slopes [H].

    qrows / krows: the query rows of dq and the key rows of dk, dv to return
    (default all).  Query rows are processed ``chunk`` at a time, so only a
    [chunk, L] block of the attention matrix exists at once.
    Returns (dq [B,H,Rq,D], dk [B,H,Rk,D], dv [B,H,Rk,D]) and their condition
    magnitudes (tq, tk, tv), same shapes.
    """
    nb, nh, length, dim = q.shape
    qsel = np.arange(length) if qrows is None else np.asarray(qrows)
    ksel = np.arange(length) if krows is None else np.asarray(krows)
    qpos = np.full(length, -1, dtype=np.int64)
    qpos[qsel] = np.arange(len(qsel))
    dq = np.zeros((nb, nh, len(qsel), dim))
    dk = np.zeros((nb, nh, len(ksel), dim))
    dv = np.zeros_like(dk)
    tq, tk, tv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dk)
    j = np.arange(length)[None, :]
    for b in range(nb):
        for h in range(nh):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            for r0 in range(0, length, chunk):
                i = np.arange(r0, min(length, r0 + chunk))[:, None]
                live = j <= i
                z = scale * (qh[i[:, 0]] @ kh.T) - slopes[h] * (i - j)
                z = np.where(live, z, -np.inf)
                e = np.exp(z - z.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)            # exactly 0 where masked
                dob = doh[i[:, 0]]
                dp = dob @ vh.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                o = p @ vh
                a = (np.abs(dob) * (np.abs(o) + p @ np.abs(vh))).sum(axis=1)   # A_i
                w = np.abs(ds) + p * a[:, None]                 # per (i, j) magnitude
                mine = qpos[i[:, 0]]
                sel = mine >= 0
                if sel.any():
                    dq[b, h, mine[sel]] = scale * (ds[sel] @ kh)
                    tq[b, h, mine[sel]] = scale * (w[sel] @ np.abs(kh))
                dk[b, h] += scale * (ds[:, ksel].T @ qh[i[:, 0]])
                tk[b, h] += scale * (w[:, ksel].T @ np.abs(qh[i[:, 0]]))
                dv[b, h] += p[:, ksel].T @ dob
                tv[b, h] += p[:, ksel].T @ np.abs(dob)
    return (dq, dk, dv), (tq, tk, tv)


def attention_bwd(q_bits, k_bits, v_bits, do_bits, total_heads: int, head_offset: int, scale: float,
                  qrows=None, krows=None, return_f64: bool = False):
    """dq, dk, dv as bf16 bits for bf16 q, k, v, do [B, H, L, D].

    With ``return_f64`` also returns the float64 gradients and their
    condition magnitudes.
    """
    nh = q_bits.shape[1]
    slopes = alibi_slopes_f32(total_heads, head_offset, nh).astype(np.float64)
    grads, terms = attention_bwd_f64(to_f64(q_bits), to_f64(k_bits), to_f64(v_bits), to_f64(do_bits), slopes,
                                     float(np.float32(scale)), qrows, krows)
    out = tuple(round_to_bf16(g) for g in grads)
    if not return_f64:
        return out
    return out, grads, terms
