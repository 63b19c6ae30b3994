"""GPU parity: LayerNorm forward/backward through the C ABI against the oracle."""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from synth import device as sdev
from oracle import layernorm as oln
from parity_helpers import check_bf16, dev_bf16, gen, host_bf16, require_gpu, sample_rows
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu


def _inputs_host(seed, rows, hidden):
    x = gen((rows, hidden), seed, W.S_LN_X, W.ACT_SIGMA)[1]
    g = gen((hidden,), seed, W.S_LN_GAMMA, W.GAMMA_SIGMA, offset=1.0)[1]
    b = gen((hidden,), seed, W.S_LN_BETA, W.BETA_SIGMA)[1]
    dy = gen((rows, hidden), seed, W.S_LN_DY, W.ACT_SIGMA)[1]
    return x, g, b, dy


def _run_fwd(x, g, b, eps=W.LN_EPS):
    rows, hidden = x.shape
    tx, tg, tb = dev_bf16(x), dev_bf16(g), dev_bf16(b)
    ty = torch.empty_like(tx)
    tm = torch.empty(rows, dtype=torch.float32, device="cuda")
    tr = torch.empty_like(tm)
    ops.bloom_layernorm_fwd(tx, tg, tb, ty, tm, tr, eps)
    torch.cuda.synchronize()
    return host_bf16(ty), tm.cpu().numpy(), tr.cpu().numpy()


def _run_bwd(dy, x, g, mean, rstd):
    rows, hidden = x.shape
    tdy, tx, tg = dev_bf16(dy), dev_bf16(x), dev_bf16(g)
    tm = torch.from_numpy(mean).cuda()
    tr = torch.from_numpy(rstd).cuda()
    tdx = torch.empty_like(tx)
    tdg = torch.empty(hidden, dtype=torch.bfloat16, device="cuda")
    tdb = torch.empty_like(tdg)
    ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hidden), dtype=torch.uint8, device="cuda")
    ops.bloom_layernorm_bwd(tdy, tx, tg, tm, tr, tdx, tdg, tdb, ws)
    torch.cuda.synchronize()
    return host_bf16(tdx), host_bf16(tdg), host_bf16(tdb)


def _check_fwd(tag, x, g, b, eps=W.LN_EPS):
    y, mu, r = _run_fwd(x, g, b, eps)
    (ry, rmu, rr), (yf, terms) = oln.layernorm_fwd(x, g, b, eps, return_f64=True)
    check_bf16(f"{tag} y", y, ry, exact=yf, terms=terms)
    assert np.allclose(r, rr, rtol=1e-5, atol=0), f"{tag} rstd"
    xs = oln.to_f64(x)
    rms = np.sqrt((xs ** 2).mean(axis=1))
    assert np.all(np.abs(mu.astype(np.float64) - rmu) <= 1e-5 * np.maximum(rms, 1e-30) + 1e-30), f"{tag} mean"
    return rmu, rr


def _check_bwd(tag, dy, x, g, mean, rstd, eps=W.LN_EPS):
    dx, dg, db = _run_bwd(dy, x, g, mean, rstd)
    (rdx, rdg, rdb), (fdx, fdg, fdb, terms, (cg, cb)) = oln.layernorm_bwd(dy, x, g, eps, return_f64=True)
    check_bf16(f"{tag} dx", dx, rdx, exact=fdx, terms=terms)
    # column sums over many rows: float32 partials in another order; condition = sum of |addends|
    check_bf16(f"{tag} dgamma", dg, rdg, exact=fdg, terms=cg)
    check_bf16(f"{tag} dbeta", db, rdb, exact=fdb, terms=cb)


@pytest.mark.parametrize("wl", [W.TINY, W.MINI, W.SHARD], ids=lambda w: w.name)
def test_layernorm_workloads_full(wl):
    require_gpu()
    s = wl.ln
    x, g, b, dy = _inputs_host(wl.seed, s.rows, s.hidden)
    mean, rstd = _check_fwd(wl.name, x, g, b)
    _check_bwd(wl.name, dy, x, g, mean, rstd)


@pytest.mark.timeout(600)
def test_embedding_layernorm_long_context_sampled():
    """Embedding LayerNorm on [8192, 14336] (the 8192-token ALiBi run): full GPU
    launch, oracle on sampled rows (every row is independent)."""
    require_gpu()
    wl = W.LONG
    rows, hidden = wl.ln.rows, wl.ln.hidden
    tx = torch.empty(rows, hidden, dtype=torch.bfloat16, device="cuda")
    sdev.fill_(tx, wl.seed, W.S_LN_X, W.ACT_SIGMA)
    g = synth.tensor(wl.seed, W.S_LN_GAMMA, hidden, W.GAMMA_SIGMA, offset=1.0, mode=synth.MODE_BF16)
    b = synth.tensor(wl.seed, W.S_LN_BETA, hidden, W.BETA_SIGMA, mode=synth.MODE_BF16)
    ty = torch.empty_like(tx)
    tm = torch.empty(rows, dtype=torch.float32, device="cuda")
    tr = torch.empty_like(tm)
    ops.bloom_layernorm_fwd(tx, dev_bf16(g), dev_bf16(b), ty, tm, tr, W.LN_EPS)
    torch.cuda.synchronize()
    sel = sample_rows(rows, 384, 3, must=(0, rows - 1))
    x = host_bf16(tx[torch.from_numpy(sel).cuda()])
    # the device generator's rows are the host generator's rows
    xh = synth.values(wl.seed, W.S_LN_X, (sel[:, None] * hidden + np.arange(hidden)[None, :]),
                      W.ACT_SIGMA, mode=synth.MODE_BF16)
    assert np.array_equal(x, xh)
    (ry, rmu, rr), (yf, terms) = oln.layernorm_fwd(x, g, b, W.LN_EPS, return_f64=True)
    check_bf16("emb-LN y", host_bf16(ty[torch.from_numpy(sel).cuda()]), ry, exact=yf, terms=terms)
    assert np.allclose(tr.cpu().numpy()[sel], rr, rtol=1e-5, atol=0)


def test_layernorm_fwd_across_the_launch_switch():
    """At H = 14336 the forward runs its five-workgroups-per-CU kernel while the
    rows fit in two rounds of four per compute unit (rows <= 8 x CUs) and its
    four-per-CU kernel above that.  Both sides of the switch, every element
    against the oracle; the rows both launches share must come out bit-identical
    (the same arithmetic in the same order)."""
    require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hidden = 14336
    x, g, b, _ = _inputs_host(14, 8 * cus + 1, hidden)
    y_hi, _, r_hi = _run_fwd(x, g, b)
    y_lo, _, r_lo = _run_fwd(x[:-1], g, b)
    assert np.array_equal(y_hi[:-1], y_lo) and np.array_equal(r_hi[:-1], r_lo)
    _check_fwd(f"switch {8 * cus + 1}x{hidden}", x, g, b)
    _check_fwd(f"switch {8 * cus}x{hidden}", x[:-1], g, b)


# (600, 8192), (777, 5120) and (300, 12288) take the streaming backward with
# 2-4 rows per workgroup (counts differ between workgroups); (7, 16384) with one;
# (600, 2048) and (777, 2048) its four-wave team at H = 2048 with two
# workgroups per compute unit, where some workgroups get 1 row and others 2;
# (3, 40000) and (2, 49152) the 1024-thread backward team with 5 and 6
# vectors per thread (rows wider than 4 vectors per thread at 1024 threads).
@pytest.mark.parametrize("rows,hidden", [(1, 8), (3, 1000), (5, 4104), (7, 16384), (33, 2056), (2, 65536),
                                         (130, 64), (9, 4096), (4, 4112), (600, 8192), (777, 5120),
                                         (300, 12288), (600, 2048), (777, 2048), (3, 40000), (2, 49152)])
def test_layernorm_ragged_shapes(rows, hidden):
    require_gpu()
    x, g, b, dy = _inputs_host(11, rows, hidden)
    mean, rstd = _check_fwd(f"ragged {rows}x{hidden}", x, g, b)
    _check_bwd(f"ragged {rows}x{hidden}", dy, x, g, mean, rstd)


def test_layernorm_constant_rows_and_scales():
    require_gpu()
    rows, hidden = 6, 2048
    x, g, b, dy = _inputs_host(12, rows, hidden)
    x[0, :] = 0x3F40  # constant 0.75: variance 0, y = beta exactly
    x[1, :] = 0x0000
    x[2] = oln.round_to_bf16(oln.to_f64(x[2]) * 1000.0)   # large values
    x[3] = oln.round_to_bf16(oln.to_f64(x[3]) * 1e-3 + 7.0)  # small spread, large mean
    y, mu, r = _run_fwd(x, g, b)
    assert np.array_equal(y[0], b) and np.array_equal(y[1], b)
    mean, rstd = _check_fwd("special rows", x, g, b)
    _check_bwd("special rows", dy, x, g, mean, rstd)


def test_layernorm_empty_and_deterministic():
    require_gpu()
    t = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    m = torch.empty(0, dtype=torch.float32, device="cuda")
    ops.bloom_layernorm_fwd(t, g, g, t, m, m, 1e-5)
    x, g, b, dy = _inputs_host(13, 512, 14336)
    mean, rstd = oln.layernorm_fwd(x, g, b, 1e-5)[1:]
    a = _run_bwd(dy, x, g, mean, rstd)
    c = _run_bwd(dy, x, g, mean, rstd)
    for u, v in zip(a, c):
        assert np.array_equal(u, v)
    assert np.array_equal(_run_fwd(x, g, b)[0], _run_fwd(x, g, b)[0])
