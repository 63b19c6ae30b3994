"""bfloat16 rounding for the oracle (round to nearest, ties to even).

bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits
and 7 stored fraction bits, so 8 significant bits for normal numbers, a
smallest normal of 2**-126 and a smallest subnormal of 2**-133.  The pages
choose BF16 for its FP32-sized exponent (page "BLOOM 176B 训练技术概览",
section "BF16 优化器"; page "企业官网建设流程全解析", section 4.1).

``round_to_bf16`` rounds a float64 value *once* to the nearest bfloat16 (no
detour through float32, which would round twice).  Because every float32 is
exactly a float64, the same function is the float32 -> bfloat16 RNE used for
the optimizer's parameter copy.
"""

from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")      # largest finite bfloat16
BF16_MIN_NORMAL_EXP = -126
BF16_QUANTUM_SUBNORMAL = 2.0 ** -133


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 of each float64 value, ties to even; returns uint16 bits.

    Method: write |x| = f * 2**e with f in [0.5, 1).  A bfloat16 with that
    binade has spacing q = 2**(e-8) (8 significant bits), or 2**-133 below the
    normal range.  x / q is exact, ``np.rint`` rounds it half-to-even, and the
    product by q is exact again.  Results beyond the largest finite bfloat16
    become infinities; NaN becomes the quiet NaN 0x7FC0 with the sign kept.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.where(e - 1 >= BF16_MIN_NORMAL_EXP, np.ldexp(1.0, e - 8), BF16_QUANTUM_SUBNORMAL)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(x / q) * q
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isinf(x), x, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x).astype(np.uint16) << np.uint16(15))
        bits = np.where(nan, sign | np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


def to_f64(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def ulp(bits) -> np.ndarray:
    """Spacing of bfloat16 numbers at the magnitude of each value (float64)."""
    v = np.abs(to_f64(bits))
    _, e = np.frexp(v)
    normal = (e - 1 >= BF16_MIN_NORMAL_EXP) & (v > 0)
    return np.where(normal, np.ldexp(1.0, e - 8), BF16_QUANTUM_SUBNORMAL)
