"""Pins for the oracle's fused ALiBi causal attention (CPU only).

Pins: torch's scaled_dot_product_attention in float64 with the ALiBi bias and
causal mask as an explicit additive mask (independent library code); the
composition "scores = Q K^T, then the fused-softmax oracle, then times V";
closed forms for Q = 0 (the weights are a truncated geometric sequence, and
so is the log-sum-exp); constant value rows pass through unchanged.

Backward pins: torch autograd in float64 through the same SDPA call; the
composition with the (separately pinned) fused-softmax backward oracle;
central finite differences of the forward oracle; the invariants that the key
gradients sum to zero (softmax is unchanged when every logit of a row moves
together) and that the value gradients sum to the summed upstream gradient
(the weights of a row sum to one); chunking and row selection do not change
the result; the condition magnitudes bound the values.
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


def _alibi_bias(slopes, length):
    i = np.arange(length)[:, None]
    j = np.arange(length)[None, :]
    bias = -slopes[:, None, None] * (i - j)[None].astype(np.float64)
    return np.where(j > i, -np.inf, bias)


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(41)
    nb, nh, length, dim = 2, 3, 40, 16
    q, k, v, do = (to_f64(_rand(rng, (nb, nh, length, dim))) for _ in range(4))
    slopes = oal.alibi_slopes_f64(12)[4:7]
    scale = 0.3
    (dq, dk, dv), _ = oat.attention_bwd_f64(q, k, v, do, slopes, scale, chunk=16)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(_alibi_bias(slopes, length))[None], scale=scale)
    o.backward(torch.from_numpy(do))
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_backward_matches_softmax_backward_oracle():
    rng = np.random.default_rng(42)
    length, dim = 36, 8
    q, k, v, do = (to_f64(_rand(rng, (1, 1, length, dim)))[0, 0] for _ in range(4))
    slope, scale = 0.125, 0.35
    (dq, dk, dv), _ = oat.attention_bwd_f64(q[None, None], k[None, None], v[None, None], do[None, None],
                                            np.array([slope]), scale)
    idx = np.arange(length)
    p = oal.softmax_fwd_f64(q @ k.T, idx, np.full(length, slope), scale)
    dscores, _ = oal.softmax_bwd_f64(p, do @ v.T, idx, scale)   # d loss / d (q . k), scale included
    assert np.allclose(dq[0, 0], dscores @ k, rtol=1e-12, atol=1e-14)
    assert np.allclose(dk[0, 0], dscores.T @ q, rtol=1e-12, atol=1e-14)
    assert np.allclose(dv[0, 0], p.T @ do, rtol=1e-12, atol=1e-14)


def test_backward_finite_differences():
    rng = np.random.default_rng(43)
    length, dim = 12, 4
    q, k, v, do = (rng.standard_normal((1, 2, length, dim)) for _ in range(4))
    slopes = np.array([0.5, 0.0625])
    scale = 0.7
    (dq, dk, dv), _ = oat.attention_bwd_f64(q, k, v, do, slopes, scale, chunk=5)

    def loss(qq, kk, vv):
        o, _, _ = oat.attention_fwd_f64(qq, kk, vv, slopes, scale)
        return float((o * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for (hh, r, d) in ((0, 0, 0), (1, 5, 3), (0, length - 1, 2), (1, 7, 1)):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][0, hh, r, d] += h
            up = loss(*args)
            args[which][0, hh, r, d] -= 2 * h
            down = loss(*args)
            fd = (up - down) / (2 * h)
            assert abs(fd - grad[0, hh, r, d]) <= 1e-7 * (1 + abs(fd)), (which, hh, r, d, fd, grad[0, hh, r, d])


def test_backward_invariants_and_terms():
    rng = np.random.default_rng(44)
    nb, nh, length, dim = 1, 2, 50, 8
    q, k, v, do = (to_f64(_rand(rng, (nb, nh, length, dim))) for _ in range(4))
    slopes = np.array([0.25, 0.03125])
    (dq, dk, dv), (tq, tk, tv) = oat.attention_bwd_f64(q, k, v, do, slopes, 0.2, chunk=64)
    # sum over keys of dk is zero; sum over keys of dv is the sum of the upstream gradients
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)
    assert np.all(tq >= np.abs(dq)) and np.all(tk >= np.abs(dk)) and np.all(tv >= np.abs(dv))
    # equal value rows: dp is constant along each row, so ds and dq, dk vanish
    v_eq = np.broadcast_to(v[:, :, :1], v.shape).copy()
    (dq0, dk0, _), _ = oat.attention_bwd_f64(q, k, v_eq, do, slopes, 0.2)
    assert np.allclose(dq0, 0.0, atol=1e-13) and np.allclose(dk0, 0.0, atol=1e-13)


def test_backward_chunks_and_row_selection():
    rng = np.random.default_rng(45)
    q, k, v, do = (to_f64(_rand(rng, (1, 2, 30, 8))) for _ in range(4))
    slopes = np.array([0.5, 0.25])
    full, tf = oat.attention_bwd_f64(q, k, v, do, slopes, 0.3, chunk=512)
    small, ts = oat.attention_bwd_f64(q, k, v, do, slopes, 0.3, chunk=7)
    for a, b in zip(full + tf, small + ts):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    rows = np.array([0, 13, 29])
    sub, _ = oat.attention_bwd_f64(q, k, v, do, slopes, 0.3, qrows=rows, krows=rows, chunk=11)
    for a, b in zip(full, sub):
        assert np.allclose(a[:, :, rows], b, rtol=1e-13, atol=1e-15)
    bits = oat.attention_bwd(_rand(rng, (1, 2, 16, 8)), _rand(rng, (1, 2, 16, 8)), _rand(rng, (1, 2, 16, 8)),
                             _rand(rng, (1, 2, 16, 8)), 112, 0, 0.3)
    assert all(x.dtype == np.uint16 and x.shape == (1, 2, 16, 8) for x in bits)
