"""GPU parity: LayerNorm fused with the residual connection, against the oracle.

h = bf16(x + r) must equal the oracle bit for bit; y must match the oracle
within the LayerNorm tolerance and equal, bit for bit, what the plain
LayerNorm entry point returns for h (the fused form changes no arithmetic).
The backward's dh = dLN(dy; h) + dres is checked against the oracle with the
LayerNorm condition terms plus |dres|.
"""

import numpy as np
import pytest
import torch

from synth import workloads as W
from oracle import layernorm as oln
from parity_helpers import check_bf16, dev_bf16, gen, host_bf16, require_gpu
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu


def _inputs(seed, rows, hidden):
    x = gen((rows, hidden), seed, W.S_LN_X, W.ACT_SIGMA)[1]
    r = gen((rows, hidden), seed, W.S_LN_RES, W.ACT_SIGMA)[1]
    g = gen((hidden,), seed, W.S_LN_GAMMA, W.GAMMA_SIGMA, offset=1.0)[1]
    b = gen((hidden,), seed, W.S_LN_BETA, W.BETA_SIGMA)[1]
    dy = gen((rows, hidden), seed, W.S_LN_DY, W.ACT_SIGMA)[1]
    dres = gen((rows, hidden), seed, W.S_LN_DRES, W.ACT_SIGMA)[1]
    return x, r, g, b, dy, dres


def _fwd(x, r, g, b, eps=W.LN_EPS):
    rows, hidden = x.shape
    tx, tr, tg, tb = dev_bf16(x), dev_bf16(r), dev_bf16(g), dev_bf16(b)
    th, ty = torch.empty_like(tx), torch.empty_like(tx)
    tm = torch.empty(rows, dtype=torch.float32, device="cuda")
    ts = torch.empty_like(tm)
    ops.bloom_layernorm_residual_fwd(tx, tr, tg, tb, th, ty, tm, ts, eps)
    # the plain LayerNorm of the fused output h, for the fused == unfused check
    ty2, tm2, ts2 = torch.empty_like(tx), torch.empty_like(tm), torch.empty_like(ts)
    ops.bloom_layernorm_fwd(th, tg, tb, ty2, tm2, ts2, eps)
    torch.cuda.synchronize()
    return (host_bf16(th), host_bf16(ty), tm.cpu().numpy(), ts.cpu().numpy(),
            host_bf16(ty2), tm2.cpu().numpy(), ts2.cpu().numpy())


def _bwd(dy, dres, h, g, mean, rstd):
    rows, hidden = h.shape
    tdy, tq, th, tg = dev_bf16(dy), dev_bf16(dres), dev_bf16(h), dev_bf16(g)
    tm, ts = torch.from_numpy(mean).cuda(), torch.from_numpy(rstd).cuda()
    tdh = torch.empty_like(th)
    tdg = torch.empty(hidden, dtype=torch.bfloat16, device="cuda")
    tdb = torch.empty_like(tdg)
    ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hidden), dtype=torch.uint8, device="cuda")
    ops.bloom_layernorm_residual_bwd(tdy, tq, th, tg, tm, ts, tdh, tdg, tdb, ws)
    torch.cuda.synchronize()
    return host_bf16(tdh), host_bf16(tdg), host_bf16(tdb)


def _check(tag, x, r, g, b, dy, dres, eps=W.LN_EPS):
    h, y, mu, rs, y2, mu2, rs2 = _fwd(x, r, g, b, eps)
    (rh, ry, rmu, rr), (yf, terms) = oln.layernorm_residual_fwd(x, r, g, b, eps, return_f64=True)
    assert np.array_equal(h, rh), f"{tag} h: {np.count_nonzero(h != rh)} elements differ from bf16(x + r)"
    check_bf16(f"{tag} y", y, ry, exact=yf, terms=terms)
    assert np.array_equal(y, y2) and np.array_equal(mu, mu2) and np.array_equal(rs, rs2), \
        f"{tag}: fused output differs from LayerNorm of h"
    assert np.allclose(rs, rr, rtol=1e-5, atol=0), f"{tag} rstd"
    dh, dg, db = _bwd(dy, dres, h, g, mu, rs)
    (rdh, rdg, rdb), (fdh, fdg, fdb, dterms, (cg, cb)) = oln.layernorm_residual_bwd(dy, dres, h, g, eps,
                                                                                  return_f64=True)
    check_bf16(f"{tag} dh", dh, rdh, exact=fdh, terms=dterms)
    check_bf16(f"{tag} dgamma", dg, rdg, exact=fdg, terms=cg)
    check_bf16(f"{tag} dbeta", db, rdb, exact=fdb, terms=cb)


@pytest.mark.parametrize("wl", [W.TINY, W.MINI, W.SHARD], ids=lambda w: w.name)
def test_layernorm_residual_workloads_full(wl):
    require_gpu()
    s = wl.ln
    _check(wl.name, *_inputs(wl.seed, s.rows, s.hidden))


# (600, 8192) and (777, 5120): streaming backward with a dres slot (2 and 1
# vectors per thread); (7, 16384): a 16-wave team whose ring + dres slot does
# not fit in LDS, so the generic backward; (5, 4104), (3, 1000): generic
# block and wave teams; (600, 2048), (777, 2048): the four-wave team at
# H = 2048, two workgroups per compute unit, 1 or 2 rows per workgroup.
@pytest.mark.parametrize("rows,hidden", [(600, 8192), (777, 5120), (7, 16384), (5, 4104), (3, 1000), (1, 8),
                                         (2, 65536), (600, 2048), (777, 2048), (3, 40000)])
def test_layernorm_residual_ragged(rows, hidden):
    require_gpu()
    _check(f"ragged {rows}x{hidden}", *_inputs(21, rows, hidden))


def test_layernorm_residual_cancellation_and_zero_gradient():
    require_gpu()
    x, r, g, b, dy, dres = _inputs(22, 64, 2048)
    r[0] = x[0] ^ np.uint16(0x8000)  # r = -x: h = +0 exactly, a constant row (y = beta)
    dy[1] = 0                        # no LayerNorm gradient: dh = dres exactly
    h, y, *_ = _fwd(x, r, g, b)
    assert not np.any(oln.to_f64(h[0])) and np.array_equal(y[0], b)
    _check("special rows", x, r, g, b, dy, dres)
