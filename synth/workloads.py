"""Shapes, seeds and value distributions of the synthetic BLOOM workloads.

Only data lives here: which tensor of which workload is drawn from which
generator stream with which standard deviation.  The shapes are BLOOM's:
hidden 14336, 112 heads of dimension 128 (28 per tensor-parallel rank at TP=4),
sequence 2048 extended to 8192 for ALiBi extrapolation, a 2048-hidden
"mini BLOOM" of 24 layers, 16 heads and a 250880-token vocabulary, and an
optimizer shard of 3.67e9 elements (176e9 parameters / TP 4 / PP 12).
Sources: page "BLOOM 176B 训练技术概览" (项目概述, 架构微调); page
"Как обучали BLOOM ..." (Тензорный параллелизм от Megatron, hidden size);
page "单机多卡实战：Megatron-DeepSpeed训练类BLOOM模型全流程解析" (section 2's
model table); page "企业官网建设流程全解析" (sections 2.3, 3.3, 4.3).
"""

from __future__ import annotations

from dataclasses import dataclass, field

# Generator stream ids, one per tensor role.
S_LN_X, S_LN_GAMMA, S_LN_BETA, S_LN_DY = 1, 2, 3, 4
S_LN_RES, S_LN_DRES = 5, 6  # residual-stream input and its gradient (fused LayerNorm + residual)
S_SM_SCORES, S_SM_DPROBS = 10, 11
S_ATT_Q, S_ATT_K, S_ATT_V, S_ATT_DO = 12, 13, 14, 15  # fused attention inputs and the output gradient
S_GELU_X, S_GELU_BIAS, S_GELU_DY = 20, 21, 22
S_OPT_PARAM, S_OPT_ACC, S_OPT_M, S_OPT_V = 30, 31, 32, 33
S_OPT_GRAD0 = 100  # micro-batch k (1-based) uses stream S_OPT_GRAD0 + k

LN_EPS = 1e-5
GAMMA_SIGMA, BETA_SIGMA, BIAS_SIGMA = 0.02, 0.02, 0.02
ACT_SIGMA = 1.0
PARAM_SIGMA, GRAD_SIGMA = 0.02, 1e-3
M_SIGMA, V_SIGMA = 1e-4, 1e-6

# AdamW hyperparameters: lr and weight decay from the DeepSpeed config on
# "企业官网建设流程全解析" section 3.3 and the training config on the mini-BLOOM
# page section 3; clip 1.0 from section 4.3 of the former and section 3 of the
# latter.  betas and eps are left open by the pages; the usual AdamW defaults
# are taken.
LR, WEIGHT_DECAY, BETA1, BETA2, ADAM_EPS, MAX_GRAD_NORM = 6e-5, 0.01, 0.9, 0.999, 1e-8, 1.0


@dataclass(frozen=True)
class LNShape:
    rows: int
    hidden: int


@dataclass(frozen=True)
class SoftmaxShape:
    batch: int
    heads: int
    seq: int
    total_heads: int
    head_offset: int
    head_dim: int

    @property
    def scale(self) -> float:
        return 1.0 / self.head_dim ** 0.5


@dataclass(frozen=True)
class GeluShape:
    rows: int
    cols: int


@dataclass(frozen=True)
class OptShape:
    n: int
    microbatches: int       # bf16 grads accumulated before the step (0: acc is drawn directly)
    step: int               # AdamW step count t of the timed/checked step
    zero_moments: bool


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    ln: LNShape | None = None
    ln_bwd: bool = True
    softmax: SoftmaxShape | None = None
    softmax_bwd: bool = True
    gelu: GeluShape | None = None
    opt: OptShape | None = None
    notes: str = field(default="")


# Mini-BLOOM optimizer size: 24 layers * (12 h^2 + 13 h) + vocabulary * h, h = 2048.
MINI_HIDDEN, MINI_LAYERS, VOCAB = 2048, 24, 250880
MINI_OPT_N = MINI_LAYERS * (12 * MINI_HIDDEN ** 2 + 13 * MINI_HIDDEN) + VOCAB * MINI_HIDDEN
SHARD_N = 3_670_000_000

TINY = Workload(
    name="tiny", seed=0,
    ln=LNShape(rows=2 * 128, hidden=256),
    softmax=SoftmaxShape(batch=2, heads=8, seq=128, total_heads=8, head_offset=0, head_dim=32),
    gelu=GeluShape(rows=2 * 128, cols=1024),
    opt=OptShape(n=1_000_000, microbatches=1, step=1, zero_moments=True),
)

MINI = Workload(
    name="mini-bloom-layer", seed=1,
    ln=LNShape(rows=4 * 2048, hidden=2048),
    softmax=SoftmaxShape(batch=4, heads=16, seq=2048, total_heads=16, head_offset=0, head_dim=128),
    gelu=GeluShape(rows=4 * 2048, cols=8192),
    opt=OptShape(n=MINI_OPT_N, microbatches=0, step=100, zero_moments=False),
)

SHARD = Workload(
    name="bloom176b-tp4-shard-layer", seed=2,
    ln=LNShape(rows=2048, hidden=14336),
    softmax=SoftmaxShape(batch=1, heads=28, seq=2048, total_heads=112, head_offset=0, head_dim=128),
    gelu=GeluShape(rows=2048, cols=14336),
)

LONG = Workload(
    name="alibi-long-context-8192", seed=3,
    ln=LNShape(rows=8192, hidden=14336), ln_bwd=False,
    softmax=SoftmaxShape(batch=1, heads=28, seq=8192, total_heads=112, head_offset=0, head_dim=128),
    softmax_bwd=False,
)

OPTIMIZER = Workload(
    name="bf16-optimizer-3.67b-shard", seed=4,
    opt=OptShape(n=SHARD_N, microbatches=32, step=1, zero_moments=True),
)

ALL = (TINY, MINI, SHARD, LONG, OPTIMIZER)
