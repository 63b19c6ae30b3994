"""GPU parity: fused causal attention with the ALiBi bias (forward), against the oracle.

Tolerance: P is rounded to bf16 before the P V product (relative 2^-9 per
weight), the products accumulate in FP32 and the exponentials use the
hardware exp2, so an output element may differ from the exact value by about
2^-8 * sum_j p_j |v_j| (the oracle's condition magnitude) beyond one bf16
spacing; the check passes that magnitude scaled to that bound.  lse is FP32:
within 1e-5 * (1 + |lse|).
"""

import numpy as np
import pytest
import torch

from synth import workloads as W
from oracle import attention as oat
from parity_helpers import TERM_REL, check_bf16, dev_bf16, gen, host_bf16, require_gpu, sample_rows
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu

P_REL = 2.0 ** -8  # bound on the relative effect of the bf16 rounding of P


def _inputs(seed, b, h, s, d):
    return tuple(gen((b, h, s, d), seed, st, 1.0)[1] for st in (W.S_ATT_Q, W.S_ATT_K, W.S_ATT_V))


def _run(q, k, v, head_offset, total_heads, scale):
    b, h, s, d = q.shape
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    to = torch.empty_like(tq)
    tl = torch.empty((b, h, s), dtype=torch.float32, device="cuda")
    ops.bloom_alibi_attention_fwd(tq, tk, tv, to, tl, head_offset, total_heads, scale)
    torch.cuda.synchronize()
    return host_bf16(to), tl.cpu().numpy()


def _check(tag, q, k, v, head_offset, total_heads, scale, rows=None):
    o, lse = _run(q, k, v, head_offset, total_heads, scale)
    (ro, rl), (of, lf, terms) = oat.attention_fwd(q, k, v, total_heads, head_offset, scale, rows=rows,
                                                   return_f64=True)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    check_bf16(f"{tag} o", o, ro, exact=of, terms=terms * (P_REL / TERM_REL))
    err = np.abs(lse.astype(np.float64) - lf)
    assert np.all(err <= 1e-5 * (1 + np.abs(lf))), f"{tag} lse: max err {err.max()}"


@pytest.mark.parametrize("wl", [W.TINY, W.MINI, W.SHARD], ids=lambda w: w.name)
def test_attention_workloads(wl):
    require_gpu()
    s = wl.softmax
    q, k, v = _inputs(wl.seed, s.batch, s.heads, s.seq, s.head_dim)
    rows = None if s.seq <= 256 else sample_rows(s.seq, 96, wl.seed, must=(0, 1, 63, 64, 127, 128, s.seq - 1))
    _check(wl.name, q, k, v, s.head_offset, s.total_heads, s.scale, rows)


@pytest.mark.timeout(900)
def test_attention_long_context_sampled():
    require_gpu()
    wl = W.LONG
    s = wl.softmax
    q, k, v = _inputs(wl.seed, s.batch, 4, s.seq, s.head_dim)   # 4 of the 28 heads: heads 0..3 of 112
    rows = sample_rows(s.seq, 24, wl.seed, must=(0, 2047, 2048, s.seq - 1))
    _check("long 8192", q, k, v, s.head_offset, s.total_heads, s.scale, rows)


@pytest.mark.timeout(900)
def test_attention_max_seq_16384_sampled():
    """The compiled sequence limit (BLOOM_MAX_SEQ = 16384): [1, 2, 16384, 128],
    heads 0..1 of 112, sampled rows."""
    require_gpu()
    seq = 16384
    q, k, v = _inputs(33, 1, 2, seq, 128)
    rows = sample_rows(seq, 24, 33, must=(0, 8191, 8192, seq - 1))
    _check("max seq 16384", q, k, v, 0, 112, float(np.float32(1.0 / np.sqrt(128.0))), rows)


def _one_stream(b, h, s):
    """Whether the forward takes its one-stream-per-workgroup kernel on this
    GPU: when a compute unit's share of the 64-key blocks (two workgroups per
    unit) is at least 1.5x the longest item's, the last query block's."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    qblocks = (s + 127) // 128
    total = b * h * sum((min(s, (qb + 1) * 128) - 1) // 64 + 1 for qb in range(qblocks))
    return 2 * total >= 3 * ((s - 1) // 64 + 1) * 2 * cus


@pytest.mark.timeout(900)
@pytest.mark.parametrize("b,h,s,d,seed", [(1, 28, 8192, 128, 3), (1, 128, 2048, 32, 41), (1, 96, 2048, 64, 42)])
def test_attention_one_stream_kernel_sampled(b, h, s, d, seed):
    """Shapes with many items per compute unit take the one-stream kernel
    (the 8192-token shard shape with all 28 heads among them): sampled rows of
    every head against the oracle."""
    require_gpu()
    assert _one_stream(b, h, s), "shape no longer selects the one-stream kernel on this GPU"
    q, k, v = _inputs(seed, b, h, s, d)
    rows = sample_rows(s, 16, seed, must=(0, 63, 64, 127, 128, s - 1))
    _check(f"one-stream {b}x{h}x{s}x{d}", q, k, v, 0, max(112, h), float(np.float32(1.0 / np.sqrt(d))), rows)


# seq not a multiple of the 128-query or 64-key blocks; head_offset inside a
# larger model; every head dimension.  (1,4,200,64) and (2,2,392,128) have an
# even number of query blocks and (b, h) pairs a multiple of 4, so they take
# the XCD-split workgroup order with a ragged last block.
@pytest.mark.parametrize("b,h,s,d,off,tot", [(1, 1, 8, 32, 0, 1), (2, 3, 24, 64, 5, 12), (1, 2, 136, 128, 0, 112),
                                            (1, 2, 200, 64, 100, 112), (3, 1, 72, 32, 3, 6), (1, 1, 264, 128, 0, 16),
                                            (1, 4, 200, 64, 8, 112), (2, 2, 392, 128, 0, 2), (1, 256, 24, 32, 0, 256)])
def test_attention_ragged(b, h, s, d, off, tot):
    require_gpu()
    q, k, v = _inputs(41, b, h, s, d)
    _check(f"ragged {b}x{h}x{s}x{d}", q, k, v, off, tot, 1.0 / d ** 0.5)


def test_attention_constant_values_and_determinism():
    require_gpu()
    q, k, v = _inputs(42, 1, 2, 192, 64)
    v[:] = v[0, 0, 0]                          # every value row equal: o = that row exactly (weights sum to 1)
    o, _ = _run(q, k, v, 0, 2, 0.125)
    assert np.array_equal(o, np.broadcast_to(v[0, 0, 0], o.shape)) or \
        np.all(np.abs(oat.to_f64(o) - oat.to_f64(v)) <= 2 ** -8 * np.abs(oat.to_f64(v)))
    o2, l2 = _run(q, k, v, 0, 2, 0.125)
    o3, l3 = _run(q, k, v, 0, 2, 0.125)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)
