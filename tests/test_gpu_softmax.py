"""GPU parity: scale + ALiBi + causal mask + softmax, forward and backward."""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from synth import device as sdev
from oracle import alibi as oal
from oracle.bf16 import round_to_bf16, to_f64
from parity_helpers import check_bf16, dev_bf16, gen, host_bf16, require_gpu, sample_rows
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu


def _scores_host(seed, b, h, s, stream=W.S_SM_SCORES):
    return gen((b, h, s, s), seed, stream, W.ACT_SIGMA)[1]


def _fwd_gpu(scores_t, head_offset, total_heads, scale):
    probs = torch.empty_like(scores_t)
    ops.bloom_alibi_softmax_fwd(scores_t, probs, head_offset, total_heads, scale)
    torch.cuda.synchronize()
    return probs


def _bwd_gpu(y_t, dy_t, scale):
    ds = torch.empty_like(y_t)
    ops.bloom_alibi_softmax_bwd(y_t, dy_t, ds, scale)
    torch.cuda.synchronize()
    return ds


def _mask_zero(name, bits):
    s = bits.shape[-1]
    iu = np.triu_indices(s, 1)
    upper = bits[..., iu[0], iu[1]]
    assert np.all(upper == 0), f"{name}: masked entries are not +0"


def _full_check(tag, scores, head_offset, total_heads, scale, dy):
    b, h, s, _ = scores.shape
    slopes = oal.alibi_slopes_f32(total_heads, head_offset, h)
    ts = dev_bf16(scores)
    y = host_bf16(_fwd_gpu(ts, head_offset, total_heads, scale))
    ry, ryf = oal.softmax_fwd(scores, slopes, scale, return_f64=True)
    check_bf16(f"{tag} fwd", y, ry, exact=ryf)
    _mask_zero(f"{tag} fwd", y)
    # backward on the oracle's bf16 forward output (never the GPU's)
    ds = host_bf16(_bwd_gpu(dev_bf16(ry), dev_bf16(dy), scale))
    rds, rdsf, terms = oal.softmax_bwd(ry, dy, scale, return_terms=True)
    check_bf16(f"{tag} bwd", ds, rds, exact=rdsf.reshape(ds.shape), terms=terms.reshape(ds.shape))
    _mask_zero(f"{tag} bwd", ds)


def test_softmax_tiny_config():
    require_gpu()
    wl = W.TINY
    s = wl.softmax
    scores = _scores_host(wl.seed, s.batch, s.heads, s.seq)
    dy = _scores_host(wl.seed, s.batch, s.heads, s.seq, stream=W.S_SM_DPROBS)
    _full_check("tiny", scores, s.head_offset, s.total_heads, s.scale, dy)


@pytest.mark.timeout(900)
def test_softmax_176b_shard_full():
    """[1, 28, 2048, 2048], heads 0..27 of 112: every row checked."""
    require_gpu()
    wl = W.SHARD
    s = wl.softmax
    scores = _scores_host(wl.seed, s.batch, s.heads, s.seq)
    dy = _scores_host(wl.seed, s.batch, s.heads, s.seq, stream=W.S_SM_DPROBS)
    _full_check("176b-shard", scores, s.head_offset, s.total_heads, s.scale, dy)


def _probability_rows(seed, b, h, s):
    """Synthetic inputs with the structure of causal probabilities: |z| on and
    below the diagonal scaled by 1/(E|z| (i+1)) so rows sum to about 1, zeros
    above (float32, truncated to bf16 like every synthetic bf16 input)."""
    z = gen((b * h, s, s), seed, 90, 1.0, dtype=torch.float32, absolute=True)[1]
    z *= (1.0 / (0.7978845608 * np.arange(1, s + 1, dtype=np.float32)))[None, :, None]
    z *= np.tri(s, dtype=np.float32)[None]
    return (z.view(np.uint32) >> 16).astype(np.uint16).reshape(b, h, s, s)


@pytest.mark.timeout(900)
def test_softmax_mini_config_sampled():
    """[4, 16, 2048, 2048]: full launches, oracle on sampled rows."""
    require_gpu()
    wl = W.MINI
    s = wl.softmax
    n = s.batch * s.heads * s.seq * s.seq
    ts = torch.empty(s.batch, s.heads, s.seq, s.seq, dtype=torch.bfloat16, device="cuda")
    sdev.fill_(ts, wl.seed, W.S_SM_SCORES, W.ACT_SIGMA)
    probs = _fwd_gpu(ts, s.head_offset, s.total_heads, s.scale)
    rows_total = n // s.seq
    sel = sample_rows(rows_total, 1500, 7, must=(0, 1, s.seq - 1, rows_total - 1, rows_total - s.seq))
    tsel = torch.from_numpy(sel).cuda()
    scores_rows = host_bf16(ts.view(-1, s.seq)[tsel])
    idx = sel[:, None] * s.seq + np.arange(s.seq)[None, :]
    assert np.array_equal(scores_rows, synth.values(wl.seed, W.S_SM_SCORES, idx, W.ACT_SIGMA, mode=synth.MODE_BF16))
    slopes = oal.alibi_slopes_f32(s.total_heads, s.head_offset, s.heads)
    # rows of a [B, NH, L, L] tensor: the row function with each row's query index and head
    i = sel % s.seq
    h = (sel // s.seq) % s.heads
    yf = oal.softmax_fwd_f64(to_f64(scores_rows), i, slopes.astype(np.float64)[h], float(np.float32(s.scale)))
    got = host_bf16(probs.view(-1, s.seq)[tsel])
    check_bf16("mini fwd (sampled rows)", got, round_to_bf16(yf), exact=yf)
    del probs
    # backward: probability-structured y, dy ~ N(0,1)
    y = _probability_rows(wl.seed, s.batch, s.heads, s.seq)
    ty = dev_bf16(y)
    tdy = torch.empty_like(ty)
    sdev.fill_(tdy, wl.seed, W.S_SM_DPROBS, W.ACT_SIGMA)
    ds = _bwd_gpu(ty, tdy, s.scale)
    dy_rows = host_bf16(tdy.view(-1, s.seq)[tsel])
    dsf, terms = oal.softmax_bwd_f64(to_f64(y.reshape(-1, s.seq)[sel]), to_f64(dy_rows), i, float(np.float32(s.scale)))
    check_bf16("mini bwd (sampled rows)", host_bf16(ds.view(-1, s.seq)[tsel]), round_to_bf16(dsf), exact=dsf,
               terms=terms)


@pytest.mark.timeout(900)
def test_softmax_long_context_8192_sampled():
    """[1, 28, 8192, 8192] forward (3.76 GB per tensor): sampled rows."""
    require_gpu()
    wl = W.LONG
    s = wl.softmax
    ts = torch.empty(s.batch, s.heads, s.seq, s.seq, dtype=torch.bfloat16, device="cuda")
    sdev.fill_(ts, wl.seed, W.S_SM_SCORES, W.ACT_SIGMA)
    probs = _fwd_gpu(ts, s.head_offset, s.total_heads, s.scale)
    rows_total = s.batch * s.heads * s.seq
    sel = sample_rows(rows_total, 600, 8, must=(0, s.seq - 1, s.seq, rows_total - 1, 4095, 4096))
    tsel = torch.from_numpy(sel).cuda()
    scores_rows = host_bf16(ts.view(-1, s.seq)[tsel])
    slopes = oal.alibi_slopes_f32(s.total_heads, s.head_offset, s.heads)
    i = sel % s.seq
    h = (sel // s.seq) % s.heads
    yf = oal.softmax_fwd_f64(to_f64(scores_rows), i, slopes.astype(np.float64)[h], float(np.float32(s.scale)))
    got = host_bf16(probs.view(-1, s.seq)[tsel])
    check_bf16("long fwd (sampled rows)", got, round_to_bf16(yf), exact=yf)
    j = np.arange(s.seq)[None, :]
    assert np.all(got[j > i[:, None]] == 0)


@pytest.mark.timeout(900)
def test_softmax_max_seq_16384_sampled():
    """Rows at the compiled sequence limit (BLOOM_MAX_SEQ = 16384): [1, 2, 16384,
    16384], heads 0..1 of 112, 1.07 GB per tensor; forward and backward on
    sampled rows.  The backward takes the forward's probabilities as y (both
    sides see the same bits; the forward is checked on its own above it)."""
    require_gpu()
    b, h, seq, off, total = 1, 2, 16384, 0, 112
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    ts = torch.empty(b, h, seq, seq, dtype=torch.bfloat16, device="cuda")
    sdev.fill_(ts, 31, W.S_SM_SCORES, W.ACT_SIGMA)
    probs = _fwd_gpu(ts, off, total, scale)
    rows_total = b * h * seq
    sel = sample_rows(rows_total, 96, 31, must=(0, 1, 8191, 8192, seq - 1, seq, rows_total - 1))
    tsel = torch.from_numpy(sel).cuda()
    scores_rows = host_bf16(ts.view(-1, seq)[tsel])
    del ts
    slopes = oal.alibi_slopes_f32(total, off, h)
    i = sel % seq
    hh = (sel // seq) % h
    yf = oal.softmax_fwd_f64(to_f64(scores_rows), i, slopes.astype(np.float64)[hh], scale)
    got = host_bf16(probs.view(-1, seq)[tsel])
    check_bf16("max-seq fwd (sampled rows)", got, round_to_bf16(yf), exact=yf)
    j = np.arange(seq)[None, :]
    assert np.all(got[j > i[:, None]] == 0)
    tdy = torch.empty_like(probs)
    sdev.fill_(tdy, 31, W.S_SM_DPROBS, W.ACT_SIGMA)
    ds = _bwd_gpu(probs, tdy, scale)
    dy_rows = host_bf16(tdy.view(-1, seq)[tsel])
    dsf, terms = oal.softmax_bwd_f64(to_f64(got), to_f64(dy_rows), i, scale)
    gds = host_bf16(ds.view(-1, seq)[tsel])
    check_bf16("max-seq bwd (sampled rows)", gds, round_to_bf16(dsf), exact=dsf, terms=terms)
    assert np.all(gds[j > i[:, None]] == 0)


@pytest.mark.parametrize("b,h,s,off,total", [(1, 1, 8, 0, 1), (2, 3, 24, 1, 5), (1, 2, 136, 0, 2),
                                             (1, 2, 4104, 3, 12), (1, 1, 8200, 0, 1), (3, 4, 64, 60, 64),
                                             (1, 2, 520, 0, 112), (1, 256, 24, 0, 256)])
def test_softmax_ragged_shapes(b, h, s, off, total):
    require_gpu()
    scores = _scores_host(21, b, h, s)
    dy = _scores_host(21, b, h, s, stream=W.S_SM_DPROBS)
    _full_check(f"ragged {b}x{h}x{s}", scores, off, total, 0.125, dy)


def test_softmax_masked_inputs_are_not_read_and_deterministic():
    require_gpu()
    b, h, s = 1, 4, 256
    scores = _scores_host(22, b, h, s)
    nan_scores = scores.copy()
    iu = np.triu_indices(s, 1)
    nan_scores[..., iu[0], iu[1]] = 0x7FC0
    y1 = host_bf16(_fwd_gpu(dev_bf16(scores), 0, 8, 0.3))
    y2 = host_bf16(_fwd_gpu(dev_bf16(nan_scores), 0, 8, 0.3))
    assert np.array_equal(y1, y2)
    dy = _scores_host(22, b, h, s, stream=W.S_SM_DPROBS)
    ynan = y1.copy()
    ynan[..., iu[0], iu[1]] = 0x7FC0
    dynan = dy.copy()
    dynan[..., iu[0], iu[1]] = 0xFF80
    d1 = host_bf16(_bwd_gpu(dev_bf16(y1), dev_bf16(dy), 0.3))
    d2 = host_bf16(_bwd_gpu(dev_bf16(ynan), dev_bf16(dynan), 0.3))
    assert np.array_equal(d1, d2)
    assert np.array_equal(d1, host_bf16(_bwd_gpu(dev_bf16(y1), dev_bf16(dy), 0.3)))


def test_softmax_zero_scores_closed_form():
    """Zero scores give geometric rows y_j = rho^(i-j)(1-rho)/(1-rho^(i+1))."""
    require_gpu()
    s = 512
    slopes = oal.alibi_slopes_f32(112, 0, 28)
    t = torch.zeros(1, 28, s, s, dtype=torch.bfloat16, device="cuda")
    y = host_bf16(_fwd_gpu(t, 0, 112, 0.0883883461356163))
    for hh in (0, 13, 27):
        rho = np.exp(-np.float64(slopes[hh]))
        for i in (0, 1, 100, 511):
            k = np.arange(i, -1, -1, dtype=np.float64)
            want = rho ** k * (1 - rho) / (1 - rho ** (i + 1))
            check_bf16(f"geometric h{hh} i{i}", y[0, hh, i, : i + 1], round_to_bf16(want), exact=want)
    assert int(y[0, 0, 0, 0]) == 0x3F80
