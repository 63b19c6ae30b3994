"""Pins for the oracle's fused ALiBi causal attention (CPU only).

Pins: torch's scaled_dot_product_attention in float64 with the ALiBi bias and
causal mask as an explicit additive mask (independent library code); the
composition "scores = Q K^T, then the fused-softmax oracle, then times V";
closed forms for Q = 0 (the weights are a truncated geometric sequence, and
so is the log-sum-exp); constant value rows pass through unchanged.
"""

import numpy as np
import torch

from oracle import alibi as oal
from oracle import attention as oat
from oracle.bf16 import round_to_bf16, to_f64


def _rand(rng, shape, sigma=1.0):
    return round_to_bf16(rng.standard_normal(shape) * sigma)


def test_matches_torch_sdpa_with_alibi_mask():
    rng = np.random.default_rng(31)
    nb, nh, length, dim = 2, 3, 48, 16
    q, k, v = (to_f64(_rand(rng, (nb, nh, length, dim))) for _ in range(3))
    slopes = oal.alibi_slopes_f64(8)[2:5]
    scale = 1.0 / np.sqrt(dim)
    o, lse, _ = oat.attention_fwd_f64(q, k, v, slopes, scale)
    i = np.arange(length)[:, None]
    j = np.arange(length)[None, :]
    bias = -slopes[:, None, None] * (i - j)[None].astype(np.float64)
    bias = np.where(j > i, -np.inf, bias)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(bias)[None], scale=scale).numpy()
    assert np.allclose(o, t, rtol=1e-12, atol=1e-13)
    z = scale * np.einsum("bhid,bhjd->bhij", q, k) + bias[None]
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(z), dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_matches_softmax_oracle_times_v():
    rng = np.random.default_rng(32)
    length, dim = 40, 8
    q, k, v = (to_f64(_rand(rng, (1, 1, length, dim))) for _ in range(3))
    slope, scale = 0.25, 0.3
    o, _, _ = oat.attention_fwd_f64(q, k, v, np.array([slope]), scale)
    s = q[0, 0] @ k[0, 0].T
    p = oal.softmax_fwd_f64(s, np.arange(length), np.full(length, slope), scale)
    assert np.allclose(o[0, 0], p @ v[0, 0], rtol=1e-13, atol=1e-14)


def test_zero_queries_give_geometric_weights():
    length, dim, slope = 64, 4, 0.375
    q = np.zeros((1, 1, length, dim))
    k = np.random.default_rng(33).standard_normal((1, 1, length, dim))
    v = np.zeros((1, 1, length, dim))
    c = 5
    v[0, 0, c, 0] = 1.0                       # one-hot value row c: o[i, 0] = p_ic
    v[0, 0, :, 1] = 2.5                       # a constant column passes through
    o, lse, _ = oat.attention_fwd_f64(q, k, v, np.array([slope]), 0.125)
    r = np.exp(-slope)
    for i in [c, c + 1, 17, length - 1]:
        # p_ij = r^(i-j) (1 - r) / (1 - r^(i+1)) for j <= i
        want = r ** (i - c) * (1 - r) / (1 - r ** (i + 1))
        assert abs(o[0, 0, i, 0] - want) < 1e-15
        assert abs(lse[0, 0, i] - np.log((1 - r ** (i + 1)) / (1 - r))) < 1e-14
    assert np.all(o[0, 0, :c, 0] == 0.0)      # key c is masked for queries before it
    assert np.allclose(o[0, 0, :, 1], 2.5, rtol=0, atol=1e-14)


def test_bf16_wrapper_rows_subset():
    rng = np.random.default_rng(34)
    q, k, v = (_rand(rng, (1, 2, 32, 8)) for _ in range(3))
    (o_all, lse_all) = oat.attention_fwd(q, k, v, 112, 0, 0.3)
    rows = np.array([0, 7, 31])
    (o_sub, lse_sub) = oat.attention_fwd(q, k, v, 112, 0, 0.3, rows=rows)
    assert np.array_equal(o_sub, o_all[:, :, rows]) and np.array_equal(lse_sub, lse_all[:, :, rows])
