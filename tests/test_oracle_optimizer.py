"""Pins for the oracle's BF16Optimizer step (CPU only).

Pins: hand-derived AdamW scalars; torch.optim.AdamW(foreach=False) in float64
with clipping done by hand (independent library code); float32 accumulation
exact on power-of-two data and distinguishable from a float64 sum; the norm of
a constant array; the clipped gradient's norm equals max_norm; moment
invariants; the bf16 copy is the RNE of the float32 master (torch).
"""

import json
import os
from decimal import Decimal

import numpy as np
import pytest
import torch

from oracle import optimizer as opt
from oracle.bf16 import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adamw_hand.json")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    hp = json.load(open(GOLDEN))["hparams"]
    p64 = np.array([case["p"]])
    m64 = np.zeros(1)
    v64 = np.zeros(1)
    for t, g in enumerate(case["grads"], start=1):
        norm = opt.global_norm(np.array([g], dtype=np.float32))
        c = opt.clip_coefficient(norm, hp["max_grad_norm"])
        # the float64 form of the update (state kept in float64 between steps)
        p64, m64, v64 = opt.adamw_f64(p64, m64, v64, c * np.array([g]), hp["lr"], hp["beta1"],
                                      hp["beta2"], hp["eps"], hp["weight_decay"], t)
    assert norm == case["norm"] and c == case["clip"]
    # float64 evaluation of the rule: a few float64 ulps from the 50-digit values
    for got, want in ((p64[0], case["p_final"]), (m64[0], case["m_final"]), (v64[0], case["v_final"])):
        w = float(Decimal(want))
        assert abs(got - w) <= 4e-15 * abs(w), (got, want)


def test_matches_torch_adamw():
    rng = np.random.default_rng(13)
    n = 5000
    p = (0.02 * rng.standard_normal(n)).astype(np.float32)
    m = (1e-4 * rng.standard_normal(n)).astype(np.float32)
    v = np.abs(1e-6 * rng.standard_normal(n)).astype(np.float32)
    acc = (0.05 * rng.standard_normal(n)).astype(np.float32)
    lr, b1, b2, eps, wd, step = 6e-5, 0.9, 0.999, 1e-8, 0.01, 7
    norm = opt.global_norm(acc)
    c = opt.clip_coefficient(norm, 1.0)
    assert c < 1.0
    _, (p1, m1, v1), _ = opt.adamw_update(p, m, v, acc, c, lr, b1, b2, eps, wd, step, return_f64=True)

    tp = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    o = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    st = o.state[tp]
    st["step"] = torch.tensor(float(step - 1), dtype=torch.float64)
    st["exp_avg"] = torch.from_numpy(m.astype(np.float64))
    st["exp_avg_sq"] = torch.from_numpy(v.astype(np.float64))
    tg = torch.from_numpy(acc.astype(np.float64))
    tn = torch.linalg.vector_norm(tg)
    assert abs(tn.item() - norm) < 1e-12 * norm
    tp.grad = tg * (1.0 / tn)  # max_norm / N with max_norm = 1
    o.step()
    # torch applies the decay as p*(1 - lr*wd) before the Adam term: algebraically the same
    assert np.allclose(tp.detach().numpy(), p1, rtol=0, atol=1e-15)
    assert np.allclose(st["exp_avg"].numpy(), m1, rtol=1e-12, atol=1e-20)
    assert np.allclose(st["exp_avg_sq"].numpy(), v1, rtol=1e-12, atol=1e-24)


def test_accumulate_exact_powers_of_two():
    g = round_to_bf16(np.full(10, 2.0 ** -10))
    acc = None
    for k in range(32):
        acc = opt.grad_accumulate(acc, g, first=(k == 0))
    assert acc.dtype == np.float32 and np.all(acc == np.float32(2.0 ** -5))


def test_accumulate_is_sequential_float32():
    # 1 + 2^-24 rounds back to 1 in float32 (tie to even), twice; a float64 sum
    # would give 1 + 2^-23, which float32 holds exactly.
    gs = [round_to_bf16(np.array([x])) for x in (1.0, 2.0 ** -24, 2.0 ** -24)]
    acc = None
    for k, g in enumerate(gs):
        acc = opt.grad_accumulate(acc, g, first=(k == 0))
    assert acc[0] == np.float32(1.0)
    # the first micro-batch overwrites whatever the accumulator held
    acc2 = opt.grad_accumulate(np.full(1, 123.0, dtype=np.float32), gs[0], first=True)
    assert acc2[0] == np.float32(1.0)


def test_norm_and_clip():
    a = np.full(1000, -0.25, dtype=np.float32)
    assert opt.global_norm(a) == 0.25 * np.sqrt(1000.0)
    rng = np.random.default_rng(14)
    acc = (rng.standard_normal(100000) * 0.01).astype(np.float32)
    n = opt.global_norm(acc)
    c = opt.clip_coefficient(n, 1.0)
    assert np.isclose(np.linalg.norm(c * acc.astype(np.float64)), 1.0, rtol=1e-14)
    assert opt.clip_coefficient(0.5, 1.0) == 1.0
    assert opt.clip_coefficient(1.0, 1.0) == 1.0
    assert opt.clip_coefficient(float("nan"), 1.0) == 1.0
    assert opt.clip_coefficient(float("inf"), 1.0) == 0.0


def test_first_step_invariants():
    rng = np.random.default_rng(15)
    n = 10000
    p = (0.02 * rng.standard_normal(n)).astype(np.float32)
    acc = (1e-3 * rng.standard_normal(n)).astype(np.float32)
    z = np.zeros(n, dtype=np.float32)
    (p1, m1, v1, pb), (p64, m64, v64), _ = opt.adamw_update(p, z, z, acc, 1.0, 6e-5, 0.9, 0.999, 1e-8, 0.0, 1,
                                                           return_f64=True)
    # at t = 1 from zero moments the Adam step is g/(|g| + eps): magnitude <= lr
    step = (p.astype(np.float64) - p64) / 6e-5
    assert np.all(np.abs(step) <= 1.0 + 1e-12)
    a64 = np.abs(acc.astype(np.float64))
    assert np.allclose(np.abs(step), a64 / (a64 + 1e-8), rtol=1e-9)
    assert np.all(v1 >= 0)
    # float32 state in, float32 state out: each result is the float64 value rounded once
    assert np.array_equal(p1, p64.astype(np.float32)) and np.array_equal(m1, m64.astype(np.float32))
    t = torch.from_numpy(p1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pb, t)


def test_segments_match_torch_adamw_param_groups():
    """Weight-decay segments with one global clip, against torch's AdamW with
    two parameter groups and the norm over both groups (float64)."""
    rng = np.random.default_rng(17)
    n, cut = 3000, 1800                   # [0, 1800): wd 0.01; [1800, 3000): wd 0 (biases, LayerNorm)
    p = (0.02 * rng.standard_normal(n)).astype(np.float32)
    m = (1e-4 * rng.standard_normal(n)).astype(np.float32)
    v = np.abs(1e-6 * rng.standard_normal(n)).astype(np.float32)
    acc = (0.05 * rng.standard_normal(n)).astype(np.float32)
    lr, b1, b2, eps, step = 6e-5, 0.9, 0.999, 1e-8, 3
    segs = [(0, cut, 0.01), (cut, n - cut, 0.0)]
    p1, m1, v1, pb, norm, c = opt.bf16_optimizer_step_segments(p, m, v, acc, segs, lr, b1, b2, eps, 1.0, step)
    assert c < 1.0

    groups = [torch.nn.Parameter(torch.from_numpy(p[:cut].astype(np.float64))),
              torch.nn.Parameter(torch.from_numpy(p[cut:].astype(np.float64)))]
    o = torch.optim.AdamW([{"params": [groups[0]], "weight_decay": 0.01},
                           {"params": [groups[1]], "weight_decay": 0.0}],
                          lr=lr, betas=(b1, b2), eps=eps, foreach=False)
    for tp, sl in zip(groups, (slice(0, cut), slice(cut, n))):
        tp.grad = torch.from_numpy(acc[sl].astype(np.float64))
        st = o.state[tp]
        st["step"] = torch.tensor(float(step - 1), dtype=torch.float64)
        st["exp_avg"] = torch.from_numpy(m[sl].astype(np.float64))
        st["exp_avg_sq"] = torch.from_numpy(v[sl].astype(np.float64))
    # the global norm over both groups from torch (max_norm = inf: measure only; torch's own clip
    # divides by N + 1e-6, so the gradients are scaled by max_norm / N here instead)
    tn = torch.nn.utils.clip_grad_norm_(groups, max_norm=float("inf"))
    assert abs(tn.item() - norm) < 1e-12 * norm
    for tp in groups:
        tp.grad.mul_(1.0 / tn)
    o.step()
    tp_all = np.concatenate([g.detach().numpy() for g in groups])
    # float32 results vs the float64 library: within one float32 rounding
    assert np.all(np.abs(tp_all - p1) <= np.abs(tp_all) * 2.0 ** -23 + 1e-30)
    # the undecayed segment moved by the Adam term only: p1 differs from a decayed update there
    _, _, _, pb_decayed, _, _ = opt.bf16_optimizer_step(p, m, v, acc, lr, b1, b2, eps, 0.01, 1.0, step)
    assert np.array_equal(pb[:cut], pb_decayed[:cut])


def test_single_segment_is_the_plain_step():
    rng = np.random.default_rng(18)
    n = 777
    p = (0.02 * rng.standard_normal(n)).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    acc = (0.5 * rng.standard_normal(n)).astype(np.float32)
    a = opt.bf16_optimizer_step(p, m, v, acc, 6e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    b = opt.bf16_optimizer_step_segments(p, m, v, acc, [(0, n, 0.01)], 6e-5, 0.9, 0.999, 1e-8, 1.0, 1)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x, y)
    assert a[4:] == b[4:]


def test_lr_schedule_closed_forms():
    """The page's schedule (lr 6e-5, min 1e-6, 500 warmup, 100000 iterations)
    at points where cos takes exact values."""
    f = lambda t: opt.lr_warmup_cosine(t, 6e-5, 1e-6, 500, 100000)
    assert f(1) == 6e-5 / 500 and f(250) == 3e-5 and f(500) == 6e-5
    assert abs(f(50250) - (6e-5 + 1e-6) / 2) < 1e-20          # cos(pi/2) = 0
    quarter = 500 + (100000 - 500) // 4                        # (t - W)/(D - W) = 1/4 exactly? 99500/4 = 24875
    assert abs(f(quarter) - (1e-6 + (6e-5 - 1e-6) * (1 + np.sqrt(0.5)) / 2)) < 1e-18
    assert f(100000) == 1e-6 and f(250000) == 1e-6
    ts = np.arange(500, 100001, 997)
    lrs = np.array([f(int(t)) for t in ts])
    assert np.all(np.diff(lrs) < 0)                            # decays monotonically
    assert opt.lr_warmup_cosine(3, 1.0, 0.0, 0, 10) == (1 + np.cos(np.pi * 0.3)) / 2   # no warmup
