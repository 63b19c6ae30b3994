"""Shared helpers of the GPU parity tests: device transfer and comparisons.

The tolerances are the ones the hot path is held to:

* bf16 outputs: |gpu - oracle| <= 1e-2 + 7.8e-3 |oracle| (one bf16 ulp in
  relative terms, with an absolute floor), and -- stricter, to catch real
  mistakes that the loose absolute floor would let through -- within one bf16
  spacing of the oracle's unrounded float64 value, plus 2^-126 (the kernels'
  exp2 flushes results below the float32 normal range) plus 2^-17 (128 float32
  roundoff units: reductions of depth up to ~100 plus a few operations) times
  the condition magnitude of the output (the sum of the absolute values of what
  enters it), where the formula can subtract nearly equal terms;
* FP32 optimizer state: |gpu - oracle| <= 1e-6 * T, T the magnitude of the
  update's terms (a pure relative test fails through cancellation, not error);
* the FP32 accumulator and the bf16 parameter copy: bit-exact.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.bf16 import round_to_bf16, to_f64, ulp

BF16_RTOL = 7.8e-3
BF16_ATOL = 1e-2
STATE_RTOL = 1e-6
TERM_REL = 2.0 ** -17
FLUSH = 2.0 ** -126


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> GPU bfloat16 tensor (same shape)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """GPU bfloat16 tensor -> uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_bf16(name: str, got_bits, ref_bits, exact=None, terms=None, strict: bool = True, floor=None):
    """Compares bf16 outputs; returns a short report string; raises on failure.

    ``floor`` (optional) replaces the 2^-126 absolute allowance of the strict
    check, for outputs that multiply a flushed intermediate by a large factor.
    """
    got_bits = np.asarray(got_bits)
    ref_bits = np.asarray(ref_bits)
    assert got_bits.shape == ref_bits.shape, (name, got_bits.shape, ref_bits.shape)
    a = to_f64(got_bits)
    b = to_f64(ref_bits)
    both_nan = np.isnan(a) & np.isnan(b)
    loose_ok = both_nan | (np.abs(a - b) <= BF16_ATOL + BF16_RTOL * np.abs(b))
    n_bad = int((~loose_ok).sum())
    if n_bad:
        idx = np.argwhere(~loose_ok)[:5]
        raise AssertionError(f"{name}: {n_bad} elements outside 1e-2 + 7.8e-3|ref|; first at {idx.tolist()}: "
                             f"gpu {a[tuple(idx[0])]} oracle {b[tuple(idx[0])]}")
    ex = b if exact is None else np.asarray(exact, dtype=np.float64)
    spacing = ulp(round_to_bf16(ex))
    allow = spacing + (FLUSH if floor is None else np.asarray(floor, dtype=np.float64))
    if exact is None:
        allow = allow + 0.5 * ulp(ref_bits)
    if terms is not None:
        allow = allow + TERM_REL * np.asarray(terms, dtype=np.float64)
    err = np.abs(a - ex)
    strict_ok = both_nan | (err <= allow)
    n_strict = int((~strict_ok).sum())
    ulps = np.where(both_nan, 0.0, np.abs(a - b) / ulp(ref_bits))
    report = (f"{name}: n={a.size} bit-equal {np.mean(got_bits == ref_bits):.4f} "
              f"max ulp vs oracle bf16 {float(np.max(ulps)) if ulps.size else 0:.0f}")
    if strict and n_strict:
        idx = np.argwhere(~strict_ok)[:5]
        i0 = tuple(idx[0])
        raise AssertionError(f"{name}: {n_strict} elements beyond one bf16 spacing of the exact value; "
                             f"first at {idx.tolist()}: gpu {a[i0]!r} exact {ex[i0]!r} allow {allow[i0]!r}; "
                             + report)
    print(report)
    return report


def check_state(name: str, got, ref, terms):
    """FP32 state within 1e-6 of the term magnitude."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_nan = np.isnan(got) & np.isnan(ref)
    err = np.abs(got - ref)
    ok = both_nan | (err <= STATE_RTOL * np.asarray(terms)) | (got == ref)
    n_bad = int((~ok).sum())
    scaled = np.where(both_nan | (terms == 0), 0.0, err / np.where(terms == 0, 1.0, terms))
    report = f"{name}: n={got.size} max term-scaled error {float(np.max(scaled)) if scaled.size else 0:.3e}"
    if n_bad:
        i0 = int(np.argwhere(~ok)[0][0])
        raise AssertionError(f"{name}: {n_bad} elements beyond 1e-6 term-scaled; first {i0}: gpu {got[i0]!r} "
                             f"oracle {ref[i0]!r} terms {terms[i0]!r}")
    print(report)
    return report


def gen(shape, seed: int, stream: int, sigma: float, offset: float = 0.0, dtype=torch.bfloat16,
        absolute: bool = False):
    """A synthetic input made on the GPU by the device generator (bit-identical
    to the host generator, see test_gpu_synth) and its host copy (uint16 bf16
    bit patterns, or float32)."""
    from synth import device as sdev
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if absolute:
        sdev.fill_abs_(t, seed, stream, sigma)
    else:
        sdev.fill_(t, seed, stream, sigma, offset)
    host = host_bf16(t) if dtype == torch.bfloat16 else t.cpu().numpy()
    return t, host


def sample_rows(total: int, k: int, seed: int, must=()) -> np.ndarray:
    """k distinct random indices in [0, total) plus the `must` ones (all checked in range)."""
    must = [int(m) for m in must]
    if any(m < 0 or m >= total for m in must):
        raise ValueError(f"sample index out of range [0, {total})")
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=min(k, total), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(list(must), dtype=np.int64)])).astype(np.int64)
