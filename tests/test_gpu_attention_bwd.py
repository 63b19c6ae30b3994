"""GPU parity: fused causal attention with the ALiBi bias, backward, against the oracle.

The backward takes lse from the forward.  Here it comes from the oracle's
forward (rounded to float32), except in the chained tests, which feed the GPU
forward's own.  The oracle computes the exact gradients from q, k, v and dout.

Tolerance: p is rounded to bf16 before its product with dout (relative
2^-9), ds enters its products as two bf16 parts (relative 2^-17), and the row
sums sum_j p_ij dp_ij are FP32, so an element may differ from the exact
gradient by well under 2^-8 times the oracle's condition magnitude
(scale * sum (|ds| + p A) |k| for dq, the same with |q| for dk, sum p |dout|
for dv) beyond one bf16 spacing; every element must also meet the
1e-2 + 7.8e-3 |ref| bound.
"""

import numpy as np
import pytest
import torch

from synth import workloads as W
from oracle import attention as oat
from parity_helpers import TERM_REL, check_bf16, dev_bf16, dev_f32, gen, host_bf16, require_gpu, sample_rows
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu

G_REL = 2.0 ** -8


def _inputs(seed, b, h, s, d):
    return tuple(gen((b, h, s, d), seed, st, 1.0)[1] for st in (W.S_ATT_Q, W.S_ATT_K, W.S_ATT_V, W.S_ATT_DO))


def _bwd_gpu(q, k, v, do, lse, head_offset, total_heads, scale):
    """Host arrays (bf16 bits; lse float32) in, dq, dk, dv bits out."""
    b, h, s, d = q.shape
    tq, tk, tv, tdo = (dev_bf16(x) for x in (q, k, v, do))
    tl = dev_f32(lse)
    dq, dk, dv = (torch.empty_like(tq) for _ in range(3))
    ws = torch.empty(ops.bloom_alibi_attention_bwd_workspace_size(b, h, s), dtype=torch.uint8, device="cuda")
    ops.bloom_alibi_attention_bwd(tq, tk, tv, tdo, tl, dq, dk, dv, head_offset, total_heads, scale, ws)
    torch.cuda.synchronize()
    return host_bf16(dq), host_bf16(dk), host_bf16(dv)


def _check(tag, got, q, k, v, do, head_offset, total_heads, scale, qrows=None, krows=None):
    ref, exact, terms = oat.attention_bwd(q, k, v, do, total_heads, head_offset, scale, qrows=qrows, krows=krows,
                                          return_f64=True)
    sel = (qrows, krows, krows)
    for name, g, r, e, t, rows in zip(("dq", "dk", "dv"), got, ref, exact, terms, sel):
        if rows is not None:
            g = g[:, :, rows]
        check_bf16(f"{tag} {name}", g, r, exact=e, terms=t * (G_REL / TERM_REL))


def _oracle_lse(q, k, v, head_offset, total_heads, scale):
    return oat.attention_fwd(q, k, v, total_heads, head_offset, scale)[1]


# seq not a multiple of the 128-row workgroup blocks or the 64-row tiles;
# head_offset inside a larger model; every head dimension; several 128-row
# blocks per head with a short last one (2, 4, 1000).
@pytest.mark.parametrize("b,h,s,d,off,tot", [(1, 1, 8, 32, 0, 1), (2, 3, 24, 64, 5, 12), (1, 2, 136, 128, 0, 112),
                                            (1, 2, 200, 64, 100, 112), (3, 1, 72, 32, 3, 6), (1, 1, 264, 128, 0, 16),
                                            (1, 4, 200, 64, 8, 112), (2, 2, 392, 128, 0, 2),
                                            (2, 4, 1000, 64, 4, 16), (1, 256, 24, 32, 0, 256)])
def test_attention_bwd_ragged(b, h, s, d, off, tot):
    require_gpu()
    q, k, v, do = _inputs(51, b, h, s, d)
    scale = 1.0 / d ** 0.5
    lse = _oracle_lse(q, k, v, off, tot, scale)
    got = _bwd_gpu(q, k, v, do, lse, off, tot, scale)
    _check(f"ragged {b}x{h}x{s}x{d}", got, q, k, v, do, off, tot, scale)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl", [W.TINY, W.SHARD], ids=lambda w: w.name)
def test_attention_bwd_workloads(wl):
    """Tiny config (every row) and the 176B shard shape [1, 28, 2048, 128]
    (sampled query rows of dq and key rows of dk, dv)."""
    require_gpu()
    sm = wl.softmax
    q, k, v, do = _inputs(wl.seed, sm.batch, sm.heads, sm.seq, sm.head_dim)
    lse = _oracle_lse(q, k, v, sm.head_offset, sm.total_heads, sm.scale)
    got = _bwd_gpu(q, k, v, do, lse, sm.head_offset, sm.total_heads, sm.scale)
    rows = None
    if sm.seq > 256:
        rows = sample_rows(sm.seq, 64, wl.seed, must=(0, 1, 63, 64, 127, 128, sm.seq - 64, sm.seq - 1))
    _check(wl.name, got, q, k, v, do, sm.head_offset, sm.total_heads, sm.scale, qrows=rows, krows=rows)


@pytest.mark.timeout(900)
def test_attention_fwd_then_bwd_long_context_sampled():
    """The GPU forward's own lse feeds the backward: 2 of the 28 heads of the
    8192-token extrapolation shape, sampled rows (64-query items)."""
    require_gpu()
    sm = W.LONG.softmax
    heads = 2
    q, k, v, do = _inputs(W.LONG.seed, sm.batch, heads, sm.seq, sm.head_dim)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    to = torch.empty_like(tq)
    tl = torch.empty((sm.batch, heads, sm.seq), dtype=torch.float32, device="cuda")
    ops.bloom_alibi_attention_fwd(tq, tk, tv, to, tl, sm.head_offset, sm.total_heads, sm.scale)
    torch.cuda.synchronize()
    got = _bwd_gpu(q, k, v, do, tl.cpu().numpy(), sm.head_offset, sm.total_heads, sm.scale)
    rows = sample_rows(sm.seq, 16, W.LONG.seed, must=(0, 2047, 2048, sm.seq - 1))
    _check("long 8192", got, q, k, v, do, sm.head_offset, sm.total_heads, sm.scale, qrows=rows, krows=rows)


def _wide_items(b, h, s):
    """Whether the backward's query-side kernel takes items of 128 queries on
    this GPU (else 64): when the 128-query items fill two rounds of two
    workgroups per compute unit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return b * h * ((s + 127) // 128) >= 4 * cus


@pytest.mark.timeout(900)
@pytest.mark.parametrize("b,h,s,d,seed", [(1, 64, 2048, 64, 61), (2, 64, 2048, 32, 62)])
def test_attention_bwd_wide_items_sampled(b, h, s, d, seed):
    """Shapes with many query blocks take the 128-query items (the other tests
    take the 64-query ones): the GPU forward's lse feeds the backward, sampled
    query and key rows against the oracle."""
    require_gpu()
    assert _wide_items(b, h, s), "shape no longer selects the 128-query items on this GPU"
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v, do = _inputs(seed, b, h, s, d)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    to = torch.empty_like(tq)
    tl = torch.empty((b, h, s), dtype=torch.float32, device="cuda")
    ops.bloom_alibi_attention_fwd(tq, tk, tv, to, tl, 0, 112, scale)
    torch.cuda.synchronize()
    got = _bwd_gpu(q, k, v, do, tl.cpu().numpy(), 0, 112, scale)
    rows = sample_rows(s, 12, seed, must=(0, 63, 64, 127, 128, s - 1))
    _check(f"wide {b}x{h}x{s}x{d}", got, q, k, v, do, 0, 112, scale, qrows=rows, krows=rows)


@pytest.mark.timeout(900)
def test_attention_fwd_then_bwd_max_seq_16384_sampled():
    """The compiled sequence limit (BLOOM_MAX_SEQ = 16384), one head, the GPU
    forward's lse feeding the backward: sampled query and key rows."""
    require_gpu()
    seq, heads, d = 16384, 1, 128
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    q, k, v, do = _inputs(34, 1, heads, seq, d)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    to = torch.empty_like(tq)
    tl = torch.empty((1, heads, seq), dtype=torch.float32, device="cuda")
    ops.bloom_alibi_attention_fwd(tq, tk, tv, to, tl, 0, 112, scale)
    torch.cuda.synchronize()
    got = _bwd_gpu(q, k, v, do, tl.cpu().numpy(), 0, 112, scale)
    rows = sample_rows(seq, 12, 34, must=(0, 8191, 8192, seq - 1))
    _check("max seq 16384", got, q, k, v, do, 0, 112, scale, qrows=rows, krows=rows)


def test_attention_bwd_chained_and_deterministic():
    require_gpu()
    b, h, s, d = 1, 4, 392, 128
    q, k, v, do = _inputs(52, b, h, s, d)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    to = torch.empty_like(tq)
    tl = torch.empty((b, h, s), dtype=torch.float32, device="cuda")
    ops.bloom_alibi_attention_fwd(tq, tk, tv, to, tl, 0, 112, 0.125)
    torch.cuda.synchronize()
    lse = tl.cpu().numpy()
    first = _bwd_gpu(q, k, v, do, lse, 0, 112, 0.125)
    second = _bwd_gpu(q, k, v, do, lse, 0, 112, 0.125)
    for a, c in zip(first, second):
        assert np.array_equal(a, c)
    _check("chained", first, q, k, v, do, 0, 112, 0.125)
