"""Pins for the oracle's ALiBi slopes and causal softmax (CPU only).

Pins: closed-form slope sequences; zero scores give the closed-form geometric
row; slope 0 reduces to the textbook causal softmax (torch.softmax with a -inf
mask, float64); rows sum to 1 and masked entries are exactly +0; invariance to
a per-row shift; finite differences and torch autograd for the backward;
constant upstream gradient gives a zero backward.
"""

import math

import numpy as np
import pytest
import torch

from oracle import alibi
from oracle.bf16 import round_to_bf16, to_f64, ulp


def test_power_of_two_slopes():
    assert np.allclose(alibi.alibi_slopes_f64(8), [2.0 ** -h for h in range(1, 9)], rtol=0, atol=0)
    assert np.allclose(alibi.alibi_slopes_f64(16), [2.0 ** (-h / 2) for h in range(1, 17)], rtol=1e-15)


def test_112_head_slopes():
    s = alibi.alibi_slopes_f64(112)
    assert len(s) == 112
    # heads 0..63: 2^(-(h+1)/8); heads 64..111: 2^(-(2j+1)/16)
    assert np.allclose(s[:64], [2.0 ** (-(h + 1) / 8) for h in range(64)], rtol=1e-15)
    assert np.allclose(s[64:], [2.0 ** (-(2 * j + 1) / 16) for j in range(48)], rtol=1e-15)
    s32 = alibi.alibi_slopes_f32(112, 0, 28)
    assert s32.dtype == np.float32 and float(s32[0]) == float(np.float32(2.0 ** (-1 / 8)))
    assert float(s32[27]) == float(np.float32(2.0 ** (-28 / 8)))
    assert float(s32[7]) == 0.5


def test_non_power_of_two_small():
    # 6 heads: the 4-head sequence (2^-2, 2^-4, 2^-6, 2^-8) then terms 1 and 3 of the 8-head one
    assert np.allclose(alibi.alibi_slopes_f64(6), [2 ** -2, 2 ** -4, 2 ** -6, 2 ** -8, 2 ** -1, 2 ** -3], rtol=0)


def _geometric_row(i, slope):
    rho = math.exp(-slope)
    k = np.arange(i, -1, -1, dtype=np.float64)
    return rho ** k * (1.0 - rho) / (1.0 - rho ** (i + 1))


@pytest.mark.parametrize("slope", [0.5, 2.0 ** (-1 / 8), 2.0 ** -3.5])
def test_zero_scores_give_geometric_rows(slope):
    L = 64
    s = np.zeros((L, L))
    y = alibi.softmax_fwd_f64(s, np.arange(L), np.full(L, slope), 0.25)
    for i in (0, 1, 3, 17, 63):
        assert np.allclose(y[i, : i + 1], _geometric_row(i, slope), rtol=1e-13)
        assert np.all(y[i, i + 1:] == 0.0)
    assert y[0, 0] == 1.0


def test_geometric_row_printed_example():
    # row i = 3 at slope 0.5 (hand value: rho = e^-0.5)
    y = alibi.softmax_fwd_f64(np.zeros((1, 4)), [3], [0.5], 1.0)[0]
    assert np.allclose(y, [0.10153632, 0.16740510, 0.27600434, 0.45505423], atol=5e-9)


def test_slope_zero_is_textbook_causal_softmax():
    rng = np.random.default_rng(5)
    L, scale = 40, 0.3
    s = rng.standard_normal((L, L)) * 3
    y = alibi.softmax_fwd_f64(s, np.arange(L), np.zeros(L), scale)
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), diagonal=1)
    t = torch.softmax((scale * torch.from_numpy(s)).masked_fill(mask, -math.inf), dim=-1).numpy()
    assert np.allclose(y, t, rtol=1e-13, atol=1e-300)


def test_matches_torch_with_bias():
    rng = np.random.default_rng(6)
    L, scale, slope = 33, 1 / math.sqrt(32), 0.3
    s = rng.standard_normal((L, L))
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    bias = torch.from_numpy(-slope * (i - j).astype(np.float64))
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), diagonal=1)
    ts = torch.from_numpy(s).requires_grad_()
    ty = torch.softmax((scale * ts + bias).masked_fill(mask, -math.inf), dim=-1)
    y = alibi.softmax_fwd_f64(s, np.arange(L), np.full(L, slope), scale)
    assert np.allclose(y, ty.detach().numpy(), rtol=1e-13, atol=1e-300)
    dy = rng.standard_normal((L, L))
    ty.backward(torch.from_numpy(dy))
    ds, _ = alibi.softmax_bwd_f64(y, dy, np.arange(L), scale)
    assert np.allclose(ds, ts.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_rows_sum_to_one_and_mask_is_exact_zero():
    rng = np.random.default_rng(7)
    sc = round_to_bf16(rng.standard_normal((2, 3, 50, 50)))
    # garbage above the diagonal must not matter
    sc2 = sc.copy()
    iu = np.triu_indices(50, 1)
    sc2[:, :, iu[0], iu[1]] = 0x7FC0
    slopes = alibi.alibi_slopes_f32(3, 0, 3)
    y = alibi.softmax_fwd(sc, slopes, 0.125)
    y2 = alibi.softmax_fwd(sc2, slopes, 0.125)
    assert np.array_equal(y, y2)
    assert np.all(y[:, :, iu[0], iu[1]] == 0)
    sums = to_f64(y).sum(-1)
    assert np.allclose(sums, 1.0, atol=50 * 2 ** -8)


def test_shift_invariance():
    rng = np.random.default_rng(8)
    L = 30
    s = rng.standard_normal((L, L))
    a = alibi.softmax_fwd_f64(s, np.arange(L), np.full(L, 0.7), 0.5)
    b = alibi.softmax_fwd_f64(s + 13.0, np.arange(L), np.full(L, 0.7), 0.5)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-300)


def test_backward_finite_differences():
    rng = np.random.default_rng(9)
    L, scale, slope = 12, 0.4, 0.25
    s = rng.standard_normal((L, L))
    dy = rng.standard_normal((L, L))
    q = np.arange(L)

    def loss(s_):
        return float((alibi.softmax_fwd_f64(s_, q, np.full(L, slope), scale) * dy).sum())

    y = alibi.softmax_fwd_f64(s, q, np.full(L, slope), scale)
    ds, _ = alibi.softmax_bwd_f64(y, dy, q, scale)
    h = 1e-6
    for idx in [(0, 0), (5, 3), (11, 11), (11, 0), (7, 6)]:
        sp, sm = s.copy(), s.copy()
        sp[idx] += h
        sm[idx] -= h
        fd = (loss(sp) - loss(sm)) / (2 * h)
        assert abs(fd - ds[idx]) < 1e-7
    assert np.all(ds[np.triu_indices(L, 1)] == 0)
    assert np.allclose(ds.sum(-1), 0.0, atol=1e-14)


def test_backward_constant_dy_is_zero():
    rng = np.random.default_rng(10)
    sc = round_to_bf16(rng.standard_normal((1, 2, 20, 20)))
    y = alibi.softmax_fwd(sc, alibi.alibi_slopes_f32(2, 0, 2), 0.2)
    # with y summing to exactly 1, dy = const gives ds = scale*y*(c - c*sum y); sum y of the
    # bf16-rounded y is not exactly 1, so use the float64 form on exact probabilities
    yf = alibi.softmax_fwd_f64(to_f64(sc.reshape(-1, 20)), np.arange(40) % 20,
                               np.repeat(alibi.alibi_slopes_f32(2, 0, 2).astype(np.float64), 20), 0.2)
    ds, _ = alibi.softmax_bwd_f64(yf, np.full((40, 20), 0.37), np.arange(40) % 20, 0.2)
    assert np.allclose(ds, 0.0, atol=1e-16)
    assert y.shape == sc.shape


def test_bf16_wrapper_rounds_float64_result():
    rng = np.random.default_rng(11)
    sc = round_to_bf16(rng.standard_normal((1, 2, 16, 16)))
    slopes = alibi.alibi_slopes_f32(2, 0, 2)
    y = alibi.softmax_fwd(sc, slopes, 0.3)
    flat = to_f64(sc.reshape(-1, 16))
    q = np.arange(32) % 16
    yf = alibi.softmax_fwd_f64(flat, q, np.repeat(slopes.astype(np.float64), 16), float(np.float32(0.3)))
    assert np.all(np.abs(to_f64(y.reshape(-1, 16)) - yf) <= 0.5 * ulp(y.reshape(-1, 16)) + 1e-300)
    rows = np.array([0, 5, 31])
    assert np.array_equal(alibi.softmax_fwd(sc, slopes, 0.3, rows=rows), y.reshape(-1, 16)[rows])
