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
