"""Pins for the oracle's bfloat16 rounding (CPU only)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle.bf16 import round_to_bf16, to_f64, ulp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne.json")


def _f32_from_bits(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)


def test_bit_table():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        got = int(round_to_bf16(_f32_from_bits(c["f32"]).astype(np.float64))[0])
        assert got == int(c["bf16"], 16), c


def test_nan_is_quiet_and_keeps_sign():
    x = np.array([np.nan, -np.nan], dtype=np.float64)
    bits = round_to_bf16(x)
    assert int(bits[0]) == 0x7FC0
    assert int(bits[1]) == 0xFFC0


def test_every_bf16_is_a_fixed_point():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = to_f64(allbits)
    finite = np.isfinite(vals)
    assert np.array_equal(round_to_bf16(vals[finite]), allbits[finite])
    inf = np.isinf(vals)
    assert np.array_equal(round_to_bf16(vals[inf]), allbits[inf])


def test_midpoints_round_to_even_bruteforce():
    # every midpoint between consecutive positive finite bf16 values
    lo = np.arange(0, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    hi = lo + np.uint16(1)
    mid = (to_f64(lo) + to_f64(hi)) / 2.0          # exact in float64
    got = round_to_bf16(mid)
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want)
    # a hair either side of each midpoint goes to the nearer neighbour
    eps = (to_f64(hi) - to_f64(lo)) * 2.0 ** -20
    assert np.array_equal(round_to_bf16(mid - eps), lo)
    assert np.array_equal(round_to_bf16(mid + eps), hi)
    assert np.array_equal(round_to_bf16(-mid), want | np.uint16(0x8000))


def test_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    t = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), t)


def test_rounds_once_from_float64():
    # 1 + 2^-8 + 2^-30: float32 would first round to the tie 1 + 2^-8 and then to
    # the even 1.0; a single rounding goes up to 1 + 2^-7.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(round_to_bf16(np.array([x]))[0]) == 0x3F81
    assert int(round_to_bf16(np.array([np.float64(np.float32(x))]))[0]) == 0x3F80


def test_ulp():
    assert ulp(np.array([0x3F80], dtype=np.uint16))[0] == 2.0 ** -7
    assert ulp(np.array([0x0000], dtype=np.uint16))[0] == 2.0 ** -133
    assert ulp(np.array([0xBF00], dtype=np.uint16))[0] == 2.0 ** -8


@pytest.mark.parametrize("v", [3.0e38, -3.0e38])
def test_overflow_to_inf(v):
    assert np.isinf(to_f64(round_to_bf16(np.array([v * 1.2])))[0])
