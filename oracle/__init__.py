"""CPU oracle for the BLOOM fused kernels and the BF16Optimizer step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy implementation, in float64, of what the GPU path computes.  It exists to
check the GPU path and must never be on it: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code with ``bloom_bf16_optimizer_amd`` and imports nothing
from it; inputs come from the caller as arrays (bf16 as uint16 bit patterns).

What each function follows (pages and sections):

* ``layernorm``: LayerNorm forward/backward of the fused kernels listed under
  "融合 CUDA 核" on page "BLOOM 176B 训练技术概览"; the embedding LayerNorm of
  "架构微调" on the same page uses the same function.
* ``alibi``: the combined scale + mask + softmax kernel of "融合 CUDA 核", with
  the ALiBi bias of "架构微调" (slope rule of the ALiBi paper the page lists
  under "资源", arXiv:2108.12409).
* ``gelu``: bias + GeLU of "融合 CUDA 核" in the tanh form of the GELU paper
  (Hendrycks and Gimpel, arXiv:1606.08415).
* ``optimizer``: the BF16Optimizer of "BF16 优化器" (FP32 gradient accumulation
  across pipeline micro-batches), global-norm clipping at 1.0 (section 4.3 of
  page "企业官网建设流程全解析"), AdamW with lr 6e-5 and weight decay 0.01
  (section 3.3 of the same page) and the bf16 parameter copy.
* ``bf16``: round-to-nearest-even into bfloat16.

Pinning: every function is checked in ``tests/test_oracle_*.py`` against
closed forms, invariants, finite differences and independent library routines
(PyTorch CPU in float64).  No function here is "parity unpinned".
"""

from . import bf16, layernorm, alibi, gelu, optimizer  # noqa: F401
