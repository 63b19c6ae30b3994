"""BLOOM fused kernels and BF16Optimizer step for AMD Instinct MI355X (gfx950).

The compute lives in ``libbloomkern.so`` (hand-written HIP, C ABI declared in
``include/bloom_kernels.h``); ``ops`` is the thin PyTorch-tensor binding with
the same entry-point names.  Build with ``python -m bloom_bf16_optimizer_amd.build``.
"""

from . import ops  # noqa: F401
from ._lib import BloomError, LIB_PATH, load  # noqa: F401

__all__ = ["ops", "load", "BloomError", "LIB_PATH"]
