"""Pins for the oracle's LayerNorm (CPU only).

Pins: the hand-worked row [1, 2, 3, 4]; torch.nn.functional.layer_norm and
torch autograd in float64 (independent library code); the normalised output's
zero mean and variance var/(var+eps); central finite differences of the
backward; per-row sum of dx is zero.
"""

import json
import os
from decimal import Decimal

import numpy as np
import torch

from oracle import layernorm as ln
from oracle.bf16 import round_to_bf16, to_f64, ulp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layernorm_hand.json")


def _rand_bf16(rng, shape, sigma=1.0, offset=0.0):
    return round_to_bf16(rng.standard_normal(shape) * sigma + offset)


def test_hand_worked_row():
    g = json.load(open(GOLDEN))
    x = np.array([g["x"]])
    y, mu, r = ln.layernorm_fwd_f64(x, np.ones(4), np.zeros(4), g["eps"])
    assert abs(mu[0] - float(Decimal(g["mean"]))) == 0.0
    assert abs(r[0] - float(Decimal(g["rstd"]))) < 1e-15
    for a, b in zip(y[0], g["y"]):
        assert abs(a - float(Decimal(b))) < 1e-15


def test_matches_torch_layer_norm():
    rng = np.random.default_rng(1)
    x = _rand_bf16(rng, (64, 384), 1.5, 0.3)
    gamma = _rand_bf16(rng, (384,), 0.02, 1.0)
    beta = _rand_bf16(rng, (384,), 0.02)
    y, mu, r = ln.layernorm_fwd(x, gamma, beta, 1e-5)
    eps = float(np.float32(1e-5))
    t = torch.nn.functional.layer_norm(torch.from_numpy(to_f64(x)), (384,), torch.from_numpy(to_f64(gamma)),
                                       torch.from_numpy(to_f64(beta)), eps).numpy()
    # the oracle's bf16 output is the correctly rounded value of the library's
    err = np.abs(to_f64(y) - t)
    assert np.all(err <= 0.5 * ulp(y) * (1 + 1e-6) + 1e-12)
    tx = torch.from_numpy(to_f64(x))
    assert np.allclose(mu, tx.mean(-1).numpy(), rtol=1e-6, atol=1e-7)
    assert np.allclose(r, (1.0 / torch.sqrt(tx.var(-1, unbiased=False) + eps)).numpy(), rtol=1e-6)


def test_normalised_moments():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 1000)) * 3.0 + 5.0
    eps = 1e-5
    y, mu, r = ln.layernorm_fwd_f64(x, np.ones(1000), np.zeros(1000), eps)
    var = x.var(axis=-1)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-12)
    assert np.allclose(y.var(-1), var / (var + eps), rtol=1e-12)


def test_constant_row_gives_beta():
    x = round_to_bf16(np.full((3, 64), 0.75))
    beta = round_to_bf16(np.linspace(-1, 1, 64))
    gamma = round_to_bf16(np.full(64, 2.0))
    y, mu, r = ln.layernorm_fwd(x, gamma, beta, 1e-5)
    assert np.array_equal(y, np.broadcast_to(beta, y.shape))
    assert np.allclose(r, 1.0 / np.sqrt(np.float32(1e-5)), rtol=1e-6)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(3)
    rows, hid, eps = 3, 24, 1e-5
    x = rng.standard_normal((rows, hid))
    gamma = 1 + 0.1 * rng.standard_normal(hid)
    beta = 0.1 * rng.standard_normal(hid)
    dy = rng.standard_normal((rows, hid))
    dx, dgamma, dbeta, _ = ln.layernorm_bwd_f64(dy, x, gamma, eps)

    def loss(x_, g_, b_):
        return float((ln.layernorm_fwd_f64(x_, g_, b_, eps)[0] * dy).sum())

    h = 1e-6
    for idx in [(0, 0), (1, 7), (2, 23), (0, 11)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (loss(xp, gamma, beta) - loss(xm, gamma, beta)) / (2 * h)
        assert abs(fd - dx[idx]) < 1e-6 * max(1.0, abs(fd))
    for k in [0, 5, 23]:
        gp, gm = gamma.copy(), gamma.copy()
        gp[k] += h
        gm[k] -= h
        fd = (loss(x, gp, beta) - loss(x, gm, beta)) / (2 * h)
        assert abs(fd - dgamma[k]) < 1e-6 * max(1.0, abs(fd))
        bp, bm = beta.copy(), beta.copy()
        bp[k] += h
        bm[k] -= h
        fd = (loss(x, gamma, bp) - loss(x, gamma, bm)) / (2 * h)
        assert abs(fd - dbeta[k]) < 1e-6 * max(1.0, abs(fd))
    assert np.allclose(dx.sum(-1), 0.0, atol=1e-12)


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(4)
    x = _rand_bf16(rng, (32, 256))
    gamma = _rand_bf16(rng, (256,), 0.02, 1.0)
    beta = _rand_bf16(rng, (256,), 0.02)
    dy = _rand_bf16(rng, (32, 256))
    (dxb, dgb, dbb), (dx, dg, db, terms, _) = ln.layernorm_bwd(dy, x, gamma, 1e-5, return_f64=True)
    tx = torch.from_numpy(to_f64(x)).requires_grad_()
    tg = torch.from_numpy(to_f64(gamma)).requires_grad_()
    tb = torch.from_numpy(to_f64(beta)).requires_grad_()
    y = torch.nn.functional.layer_norm(tx, (256,), tg, tb, float(np.float32(1e-5)))
    y.backward(torch.from_numpy(to_f64(dy)))
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.array_equal(dxb, round_to_bf16(tx.grad.numpy())) or \
        np.all(np.abs(to_f64(dxb) - tx.grad.numpy()) <= 0.5 * ulp(dxb) + 1e-12)


# Residual form (section 4.3 of page "企业官网建设流程全解析": LayerNorm fused
# with the residual connection; h = bf16(x + r), y = LayerNorm(h)).

def test_residual_add_rounds_once_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1.0078125 (0x3F81):
    # ties go to the even pattern; a hair above the tie rounds up.
    x = np.array([0x3F80, 0x3F81, 0x3F80, 0x3F80, 0xBF81], dtype=np.uint16)
    r = np.array([0x3B80, 0x3B80, 0x3B81, 0xBF80, 0xBB80], dtype=np.uint16)
    want = np.array([0x3F80, 0x3F82, 0x3F81, 0x0000, 0xBF82], dtype=np.uint16)
    assert np.array_equal(ln.residual_add(x, r), want)


def test_residual_with_zero_residual_is_layernorm():
    rng = np.random.default_rng(5)
    x = _rand_bf16(rng, (8, 96), 2.0, 0.5)
    g = _rand_bf16(rng, (96,), 0.1, 1.0)
    b = _rand_bf16(rng, (96,), 0.1)
    h, y, mu, r = ln.layernorm_residual_fwd(x, np.zeros_like(x), g, b, 1e-5)
    y0, mu0, r0 = ln.layernorm_fwd(x, g, b, 1e-5)
    assert np.array_equal(h, x) and np.array_equal(y, y0)
    assert np.array_equal(mu, mu0) and np.array_equal(r, r0)
    dy = _rand_bf16(rng, (8, 96))
    dh, dg, db = ln.layernorm_residual_bwd(dy, np.zeros_like(dy), h, g, 1e-5)
    dx0, dg0, db0 = ln.layernorm_bwd(dy, x, g, 1e-5)
    assert np.array_equal(dh, dx0) and np.array_equal(dg, dg0) and np.array_equal(db, db0)
    # with no gradient from the LayerNorm output, dh is the residual gradient itself
    dres = _rand_bf16(rng, (8, 96), 0.3)
    dh, dg, db = ln.layernorm_residual_bwd(np.zeros_like(dy), dres, h, g, 1e-5)
    assert np.array_equal(dh, dres)
    assert not np.any(to_f64(dg)) and not np.any(to_f64(db))


def test_residual_backward_matches_finite_differences():
    # loss = sum(w * LN(x + r)) + sum(u * (x + r)); both x and r get dh.
    rng = np.random.default_rng(6)
    rows, hid, eps = 3, 20, 1e-5
    x = rng.standard_normal((rows, hid))
    res = rng.standard_normal((rows, hid))
    gamma = 1 + 0.1 * rng.standard_normal(hid)
    beta = 0.1 * rng.standard_normal(hid)
    w = rng.standard_normal((rows, hid))
    u = rng.standard_normal((rows, hid))
    dh, dgamma, dbeta, _ = ln.layernorm_residual_bwd_f64(w, u, x + res, gamma, eps)

    def loss(x_, r_):
        h_ = x_ + r_
        return float((ln.layernorm_fwd_f64(h_, gamma, beta, eps)[0] * w).sum() + (h_ * u).sum())

    step = 1e-6
    for idx in [(0, 0), (1, 9), (2, 19)]:
        for which in (0, 1):
            p, m = [x.copy(), res.copy()], [x.copy(), res.copy()]
            p[which][idx] += step
            m[which][idx] -= step
            fd = (loss(*p) - loss(*m)) / (2 * step)
            assert abs(fd - dh[idx]) < 1e-6 * max(1.0, abs(fd))
