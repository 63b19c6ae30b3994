"""Pins for the oracle's bias + GeLU (CPU only).

Pins: torch.nn.functional.gelu(approximate='tanh') and torch autograd in
float64 (independent library code); gelu(0) = 0 and gelu'(0) = 1/2; the odd
part gelu(u) - gelu(-u) = u; the limits gelu(u) -> u and -> 0; central finite
differences of the derivative; dbias is the column sum of dx.
"""

import numpy as np
import torch

from oracle import gelu as G
from oracle.bf16 import round_to_bf16, to_f64, ulp


def test_matches_torch_tanh_gelu():
    u = np.linspace(-8, 8, 4001)
    t = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.allclose(G.gelu(u), t, rtol=1e-14, atol=1e-15)


def test_special_values():
    assert G.gelu(np.array([0.0]))[0] == 0.0
    assert G.gelu_grad(np.array([0.0]))[0] == 0.5
    u = np.linspace(-5, 5, 101)
    assert np.allclose(G.gelu(u) - G.gelu(-u), u, rtol=0, atol=1e-14)
    assert np.allclose(G.gelu(np.array([30.0])), 30.0, rtol=1e-15)
    assert abs(G.gelu(np.array([-30.0]))[0]) < 1e-300
    assert np.allclose(G.gelu(np.array([1.0, -1.0, 2.0, -3.0])),
                       [0.8411919906, -0.1588080094, 1.9545976941, -0.0036373921], atol=1e-10)


def test_derivative_finite_differences_and_autograd():
    u = np.linspace(-6, 6, 241)
    h = 1e-6
    fd = (G.gelu(u + h) - G.gelu(u - h)) / (2 * h)
    assert np.allclose(G.gelu_grad(u), fd, atol=1e-8)
    tu = torch.from_numpy(u).requires_grad_()
    torch.nn.functional.gelu(tu, approximate="tanh").sum().backward()
    # both sides cancel in 1 - t^2 and 1 + t in the far negative tail: absolute 1e-14
    assert np.allclose(G.gelu_grad(u), tu.grad.numpy(), rtol=1e-13, atol=1e-14)


def _tanh_form_50_digits(u: float):
    """u/2 (1 + tanh a) and its derivative, evaluated in 120-digit decimal from
    the tanh form itself (tanh a = (e^2a - 1)/(e^2a + 1))."""
    from decimal import Decimal as D, getcontext
    getcontext().prec = 120
    k = D(2) / D("3.14159265358979323846264338327950288419716939937510")
    k = k.sqrt()
    c = D("0.044715")
    x = D(u)
    a = k * (x + c * x ** 3)
    e2 = (2 * a).exp()
    t = (e2 - 1) / (e2 + 1)
    y = x / 2 * (1 + t)
    dy = (1 + t) / 2 + x / 2 * (1 - t * t) * k * (1 + 3 * c * x * x)
    return float(y), float(dy)


def test_far_tails_against_120_digit_tanh_form():
    # float64 1 + tanh(a) is exactly 0 for a < -19; the oracle must still give the
    # true tiny values there (e.g. gelu(-10) = -1.2e-37, a normal bf16 number)
    for u in (-12.0, -10.0, -9.95, -7.0, -5.0, -1.0, -0.75, 0.5, 3.0, 9.0):
        y, dy = _tanh_form_50_digits(u)
        assert abs(G.gelu(np.array([u]))[0] - y) <= 1e-13 * abs(y) + 1e-300, u
        assert abs(G.gelu_grad(np.array([u]))[0] - dy) <= 1e-12 * abs(dy) + 1e-300, u
    assert G.gelu(np.array([-10.0]))[0] < -1e-37


def test_bias_broadcast_and_dbias():
    rng = np.random.default_rng(12)
    x = round_to_bf16(rng.standard_normal((48, 96)))
    b = round_to_bf16(0.02 * rng.standard_normal(96))
    dy = round_to_bf16(rng.standard_normal((48, 96)))
    y = G.bias_gelu_fwd(x, b)
    tx = torch.from_numpy(to_f64(x)).requires_grad_()
    tb = torch.from_numpy(to_f64(b)).requires_grad_()
    ty = torch.nn.functional.gelu(tx + tb, approximate="tanh")
    assert np.all(np.abs(to_f64(y) - ty.detach().numpy()) <= 0.5 * ulp(y) * (1 + 1e-9) + 1e-300)
    ty.backward(torch.from_numpy(to_f64(dy)))
    (dxb, dbb), (dx, db, terms, _) = G.bias_gelu_bwd(dy, x, b, return_f64=True)
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(db, tb.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(terms >= np.abs(dx) - 1e-15)
