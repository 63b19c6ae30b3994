"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle's callers.

This module holds no arithmetic of the method being tested.  It only turns a
(seed, stream, element index) triple into a number, so that any element of any
input tensor can be regenerated on its own, on the host (here, in NumPy) or on
the device (``synth/csrc/synth.hip``), with bit-identical results.

Definition (the device kernel implements exactly the same steps):

* ``mix64`` is the output finaliser of SplitMix64 (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014), as published
  with the constants 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB.
* A tensor is named by ``key = mix64(seed * 2**32 + stream)``.
* Draw ``d`` of that tensor is ``mix64(key + (d + 1) * 0x9E3779B97F4A7C15)``
  (mod 2**64), i.e. SplitMix64's counter sequence, addressable at any ``d``.
* Element ``i`` uses draws ``3i, 3i+1, 3i+2``; their twelve 16-bit fields are
  summed to an integer ``S`` (Irwin-Hall with 12 terms: mean 393210,
  standard deviation about 65536).
* The fp32 value is ``fl32(fl32(S - 393210) * fl32(sigma / 65536))`` -- one
  correctly rounded fp32 multiply of an exact integer -- followed, when an
  offset is asked for, by one correctly rounded fp32 add ``fl32(z + offset)``.
  ``sigma / 65536`` and ``offset`` are rounded to fp32 once, on the host.
* bf16 tensors keep the upper 16 bits of that fp32 value (truncation toward
  zero; deliberately *not* the round-to-nearest-even that the optimizer under
  test performs, so that no step of the method lives here).
* ``abs`` tensors take ``|z|``.

Approximate normality is all that is needed: the values have the mean and
standard deviation of the workloads and a support of +-6 sigma.

The device library (``synth/csrc``) also holds a plain streaming copy
(``synth/csrc/ceiling.hip``, ``synth.device.stream_copy``) that the benchmark
times as the bandwidth ceiling of each read/write pattern; like the generator,
it computes nothing of the method.
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
IRWIN_HALL_MEAN = 393210  # 12 * 65535 / 2

MODE_F32 = 0
MODE_BF16 = 1
MODE_ABS_F32 = 2

_CHUNK = 1 << 22


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (for scalars such as the key)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrap-around arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


def tensor_key(seed: int, stream: int) -> int:
    return mix64_int((seed << 32) + stream)


def scale_f32(sigma: float) -> np.float32:
    """fl32(sigma / 65536), the one rounding of the scale."""
    return np.float32(sigma / 65536.0)


def _irwin_hall(key: int, idx: np.ndarray) -> np.ndarray:
    """Integer S - 393210 for each element index (int64)."""
    idx = idx.astype(np.uint64, copy=False)
    s = np.zeros(idx.shape, dtype=np.int64)
    k = np.uint64(key)
    three = np.uint64(3)
    one = np.uint64(1)
    g = np.uint64(GAMMA)
    f = np.uint64(0xFFFF)
    with np.errstate(over="ignore"):
        for d in range(3):
            ctr = idx * three + np.uint64(d) + one
            u = _mix64(k + ctr * g)
            for sh in (0, 16, 32, 48):
                s += ((u >> np.uint64(sh)) & f).astype(np.int64)
    return s - IRWIN_HALL_MEAN


def values_f32(seed: int, stream: int, idx: np.ndarray, sigma: float,
               offset: float = 0.0) -> np.ndarray:
    """fp32 values of elements ``idx`` (any shape of int indices)."""
    centred = _irwin_hall(tensor_key(seed, stream), np.asarray(idx))
    z = centred.astype(np.float32) * scale_f32(sigma)
    if offset != 0.0:
        z = z + np.float32(offset)
    return z


def values(seed: int, stream: int, idx: np.ndarray, sigma: float,
           offset: float = 0.0, mode: int = MODE_F32) -> np.ndarray:
    """Elements ``idx`` in the storage form of ``mode``.

    MODE_F32 -> float32; MODE_BF16 -> uint16 bf16 bit patterns;
    MODE_ABS_F32 -> float32 absolute values.
    """
    z = values_f32(seed, stream, idx, sigma, offset)
    if mode == MODE_F32:
        return z
    if mode == MODE_ABS_F32:
        return np.abs(z)
    if mode == MODE_BF16:
        return (z.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown mode {mode}")


def tensor(seed: int, stream: int, n: int, sigma: float, offset: float = 0.0,
           mode: int = MODE_F32, start: int = 0) -> np.ndarray:
    """Elements ``start .. start+n-1`` of one tensor, generated in chunks."""
    dtype = np.uint16 if mode == MODE_BF16 else np.float32
    out = np.empty(n, dtype=dtype)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        idx = np.arange(start + lo, start + hi, dtype=np.uint64)
        out[lo:hi] = values(seed, stream, idx, sigma, offset, mode)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
