"""GPU parity: bias + GeLU forward/backward through the C ABI against the oracle."""

import numpy as np
import pytest
import torch

from synth import workloads as W
from oracle import gelu as og
from parity_helpers import check_bf16, dev_bf16, gen, host_bf16, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, rows, cols):
    x = gen((rows, cols), seed, W.S_GELU_X, W.ACT_SIGMA)[1]
    b = gen((cols,), seed, W.S_GELU_BIAS, W.BIAS_SIGMA)[1]
    dy = gen((rows, cols), seed, W.S_GELU_DY, W.ACT_SIGMA)[1]
    return x, b, dy


def _fwd(x, b):
    tx = dev_bf16(x)
    ty = torch.empty_like(tx)
    from bloom_bf16_optimizer_amd import ops
    ops.bloom_bias_gelu_fwd(tx, dev_bf16(b), ty)
    torch.cuda.synchronize()
    return host_bf16(ty)


def _bwd(dy, x, b):
    from bloom_bf16_optimizer_amd import ops
    rows, cols = x.shape
    tx = dev_bf16(x)
    tdx = torch.empty_like(tx)
    tdb = torch.empty(cols, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ops.bloom_bias_gelu_bwd_workspace_size(rows, cols), dtype=torch.uint8, device="cuda")
    ops.bloom_bias_gelu_bwd(dev_bf16(dy), tx, dev_bf16(b), tdx, tdb, ws)
    torch.cuda.synchronize()
    return host_bf16(tdx), host_bf16(tdb)


def _check(tag, x, b, dy):
    y = _fwd(x, b)
    ry, ryf = og.bias_gelu_fwd(x, b, return_f64=True)
    # the kernel's logistic factor s = 1/(1 + 2^z) reaches 0 once 2^z overflows
    # (u below about -10, where |y| < 1.5e-37): the absolute floor there scales with |u|
    u = np.abs(og.to_f64(x) + og.to_f64(b)[None, :])
    floor = 2.0 ** -126 * (1.0 + u) ** 3
    check_bf16(f"{tag} y", y, ry, exact=ryf, floor=floor)
    dx, db = _bwd(dy, x, b)
    (rdx, rdb), (fdx, fdb, terms, cterms) = og.bias_gelu_bwd(dy, x, b, return_f64=True)
    check_bf16(f"{tag} dx", dx, rdx, exact=fdx, terms=terms, floor=floor * (1.0 + np.abs(og.to_f64(dy))))
    check_bf16(f"{tag} dbias", db, rdb, exact=fdb, terms=cterms)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", [W.TINY, W.SHARD, W.MINI], ids=lambda w: w.name)
def test_gelu_workloads_full(wl):
    require_gpu()
    x, b, dy = _inputs(wl.seed, wl.gelu.rows, wl.gelu.cols)
    _check(wl.name, x, b, dy)


@pytest.mark.parametrize("rows,cols", [(1, 8), (33, 1000), (100, 14336), (7, 65536), (257, 64), (5, 2056)])
def test_gelu_ragged_shapes(rows, cols):
    require_gpu()
    x, b, dy = _inputs(31, rows, cols)
    _check(f"ragged {rows}x{cols}", x, b, dy)


def test_gelu_wide_range_and_deterministic():
    require_gpu()
    rows, cols = 64, 1024
    x, b, dy = _inputs(32, rows, cols)
    # spread u over [-12, 12] including the region where gelu'(u) crosses zero (u ~ -0.75)
    u = np.linspace(-12.0, 12.0, rows * cols).reshape(rows, cols)
    x = og.round_to_bf16(u)
    _check("wide range", x, b, dy)
    a = _bwd(dy, x, b)
    c = _bwd(dy, x, b)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_gelu_empty():
    require_gpu()
    from bloom_bf16_optimizer_amd import ops
    t = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    ops.bloom_bias_gelu_fwd(t, torch.zeros(64, dtype=torch.bfloat16, device="cuda"), t)
