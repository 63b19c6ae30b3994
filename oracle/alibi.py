"""ALiBi slopes and the fused scale + ALiBi bias + causal mask + softmax (oracle).

Test infrastructure only.  Follows the combined "scaling, mask and softmax"
kernel listed under "融合 CUDA 核" on page "BLOOM 176B 训练技术概览", with the
ALiBi linear bias that replaces position embeddings ("架构微调", same page; the
2048 -> 8192 extrapolation of section 4.3 on page "企业官网建设流程全解析").

Slopes.  The pages cite the ALiBi paper (Press, Smith and Lewis,
arXiv:2108.12409, listed under "资源") without restating its rule, so it is
taken from the paper: for n heads with n a power of two, head h (1-based) has
slope 2**(-8h/n), a geometric sequence starting at 2**(-8/n).  Otherwise, with
c the largest power of two below n, the first c heads take the power-of-two
sequence for c, and the remaining n-c heads take, in order, the 1st, 3rd, 5th,
... terms of the power-of-two sequence for 2c.

Forward, for query row i of head h (keys j = 0 .. L-1):
    z_j = scale * s_ij - slope_h * (i - j)        for j <= i
    y_j = exp(z_j - max_k z_k) / sum_k exp(z_k - max_k z_k)
    y_j = +0                                      for j > i (causal mask)
The scale multiplies the raw score only, not the bias (the two are separate
terms of the fused kernel's input).  Backward with respect to the raw scores:
    ds_j = scale * y_j * (dy_j - sum_{k<=i} y_k dy_k)   for j <= i,  +0 otherwise,
with y the stored bf16 forward output.  Arithmetic is float64; scale and the
slopes are the float32 values the GPU receives.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16, to_f64


def _pow2_sequence(n: int) -> list[float]:
    """slope_h = 2**(-8h/n), h = 1..n, for n a power of two (float64)."""
    return [2.0 ** (-8.0 * h / n) for h in range(1, n + 1)]


def alibi_slopes_f64(total_heads: int) -> np.ndarray:
    """All slopes of a model with ``total_heads`` heads, float64."""
    if total_heads <= 0:
        raise ValueError("total_heads must be positive")
    c = 1 << (total_heads.bit_length() - 1)
    slopes = _pow2_sequence(c)
    if c != total_heads:
        slopes += _pow2_sequence(2 * c)[0::2][: total_heads - c]
    return np.array(slopes, dtype=np.float64)


def alibi_slopes_f32(total_heads: int, head_offset: int, heads: int) -> np.ndarray:
    """Slopes of heads head_offset .. head_offset+heads-1, rounded once to float32."""
    s = alibi_slopes_f64(total_heads)
    if head_offset < 0 or heads < 0 or head_offset + heads > total_heads:
        raise ValueError("head range outside the model's heads")
    return s[head_offset: head_offset + heads].astype(np.float32)


def softmax_fwd_f64(s, query_index, slope, scale: float):
    """Forward on score rows s [R, L] (float64); query_index [R]; slope [R]."""
    rows, length = s.shape
    i = np.asarray(query_index, dtype=np.int64)[:, None]
    j = np.arange(length, dtype=np.int64)[None, :]
    live = j <= i
    z = scale * s - np.asarray(slope, dtype=np.float64)[:, None] * (i - j)
    z = np.where(live, z, -np.inf)
    zmax = z.max(axis=-1, keepdims=True)
    e = np.where(live, np.exp(np.where(live, z - zmax, 0.0)), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def softmax_bwd_f64(y, dy, query_index, scale: float):
    """Backward on rows: returns (ds, condition magnitude |scale|*|y|*(|dy| + sum|y dy|))."""
    rows, length = y.shape
    i = np.asarray(query_index, dtype=np.int64)[:, None]
    j = np.arange(length, dtype=np.int64)[None, :]
    live = j <= i
    y = np.where(live, y, 0.0)
    dy = np.where(live, dy, 0.0)
    dot = (y * dy).sum(axis=-1, keepdims=True)
    ds = np.where(live, scale * y * (dy - dot), 0.0)
    abs_dot = np.abs(y * dy).sum(axis=-1, keepdims=True)
    terms = np.where(live, abs(scale) * np.abs(y) * (np.abs(dy) + abs_dot), 0.0)
    return ds, terms


def _chunk_rows(seq: int) -> int:
    return max(1, (1 << 22) // seq)


def softmax_fwd(scores_bits, slopes, scale: float, rows=None, return_f64: bool = False):
    """Forward on [B, NH, L, L] scores (bf16 bits), or on selected flat rows.

    ``slopes`` are the float32 slopes of the NH heads; ``rows`` (optional)
    lists flat row numbers r = (b*NH + h)*L + i, and the result then has
    shape [len(rows), L].  Output: bf16 bits (and, with ``return_f64``, the
    unrounded float64 probabilities of the same rows).
    """
    b, nh, seq, seq2 = scores_bits.shape
    if seq != seq2:
        raise ValueError("scores must be square in the last two dims")
    flat = scores_bits.reshape(-1, seq)
    sel = np.arange(flat.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    sl32 = np.asarray(slopes, dtype=np.float32).astype(np.float64)
    sc = float(np.float32(scale))
    out = np.empty((len(sel), seq), dtype=np.uint16)
    vals = np.empty((len(sel), seq)) if return_f64 else None
    step = _chunk_rows(seq)
    for lo in range(0, len(sel), step):
        r = sel[lo: lo + step]
        y = softmax_fwd_f64(to_f64(flat[r]), r % seq, sl32[(r // seq) % nh], sc)
        out[lo: lo + len(r)] = round_to_bf16(y)
        if return_f64:
            vals[lo: lo + len(r)] = y
    res = out.reshape(scores_bits.shape) if rows is None else out
    if not return_f64:
        return res
    return res, (vals.reshape(scores_bits.shape) if rows is None else vals)


def softmax_bwd(probs_bits, dprobs_bits, scale: float, rows=None, return_terms: bool = False):
    """Backward on [B, NH, L, L] (bf16 bits), or on selected flat rows.

    Returns dscores as bf16 bits (and, with ``return_terms``, the float64
    values and term magnitudes of the selected rows).
    """
    b, nh, seq, _ = probs_bits.shape
    fy = probs_bits.reshape(-1, seq)
    fdy = dprobs_bits.reshape(-1, seq)
    sel = np.arange(fy.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    sc = float(np.float32(scale))
    out = np.empty((len(sel), seq), dtype=np.uint16)
    vals = np.empty((len(sel), seq)) if return_terms else None
    terms = np.empty((len(sel), seq)) if return_terms else None
    step = _chunk_rows(seq)
    for lo in range(0, len(sel), step):
        r = sel[lo: lo + step]
        ds, t = softmax_bwd_f64(to_f64(fy[r]), to_f64(fdy[r]), r % seq, sc)
        out[lo: lo + len(r)] = round_to_bf16(ds)
        if return_terms:
            vals[lo: lo + len(r)] = ds
            terms[lo: lo + len(r)] = t
    res = out.reshape(probs_bits.shape) if rows is None else out
    return (res, vals, terms) if return_terms else res
