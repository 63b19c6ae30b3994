"""GPU: the allocation-free LayerNorm backward against the workspace entry point.

bloom_layernorm_bwd_noalloc runs the kernels of bloom_layernorm_bwd with the
column partial sums in the library's static device scratch; on the same
inputs it must give the same bits (dx, dgamma, dbeta), here on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents), and the first result also within the oracle's tolerance.
"""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from oracle import layernorm as oln
from parity_helpers import check_bf16, dev_bf16, host_bf16, require_gpu
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu


def _inputs(seed, rows, hidden):
    n = rows * hidden
    x = synth.tensor(seed, W.S_LN_X, n, 1.0, mode=synth.MODE_BF16).reshape(rows, hidden)
    dy = synth.tensor(seed, W.S_LN_DY, n, 1.0, mode=synth.MODE_BF16).reshape(rows, hidden)
    g = synth.tensor(seed, W.S_LN_GAMMA, hidden, 0.02, 1.0, mode=synth.MODE_BF16)
    b = synth.tensor(seed, W.S_LN_BETA, hidden, 0.02, mode=synth.MODE_BF16)
    return x, dy, g, b


def _both(x, dy, g, b):
    rows, hidden = x.shape
    tx, tdy, tg, tb = dev_bf16(x), dev_bf16(dy), dev_bf16(g), dev_bf16(b)
    y = torch.empty_like(tx)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    ops.bloom_layernorm_fwd(tx, tg, tb, y, mean, rstd, W.LN_EPS)
    outs = []
    for noalloc in (False, True):
        dx = torch.empty_like(tx)
        dgam = torch.empty(hidden, dtype=torch.bfloat16, device="cuda")
        dbet = torch.empty_like(dgam)
        if noalloc:
            ops.bloom_layernorm_bwd_noalloc(tdy, tx, tg, mean, rstd, dx, dgam, dbet)
        else:
            ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hidden), dtype=torch.uint8, device="cuda")
            ops.bloom_layernorm_bwd(tdy, tx, tg, mean, rstd, dx, dgam, dbet, ws)
        torch.cuda.synchronize()
        outs.append((host_bf16(dx), host_bf16(dgam), host_bf16(dbet)))
    return outs


def test_noalloc_matches_workspace_entry_point_twice():
    require_gpu()
    # first the 176B shard row width (28 MiB of partials), then a smaller input
    # on a narrower streaming plan: the second call reuses the scratch with
    # fewer partial rows and must not see the first call's leftovers
    for seed, rows, hidden in ((2, 2048, 14336), (9, 600, 2048)):
        print(f"noalloc case rows={rows} hidden={hidden}", flush=True)
        x, dy, g, b = _inputs(seed, rows, hidden)
        (dx0, dg0, db0), (dx1, dg1, db1) = _both(x, dy, g, b)
        assert np.array_equal(dx0, dx1) and np.array_equal(dg0, dg1) and np.array_equal(db0, db1), (rows, hidden)
        rdx, rdg, rdb = oln.layernorm_bwd(dy, x, g, W.LN_EPS)
        check_bf16(f"noalloc dgamma {rows}x{hidden}", dg1, rdg, strict=False)
        check_bf16(f"noalloc dbeta {rows}x{hidden}", db1, rdb, strict=False)
        check_bf16(f"noalloc dx {rows}x{hidden}", dx1, rdx, strict=False)


def test_noalloc_rejects_inputs_beyond_the_scratch():
    require_gpu()
    rows, hidden = 2048, 65536
    assert ops.bloom_layernorm_bwd_workspace_size(rows, hidden) > (32 << 20)
    # full-size buffers, so that nothing could be out of bounds even if the check were missing
    x = torch.zeros(rows, hidden, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(x)
    g = torch.ones(hidden, dtype=torch.bfloat16, device="cuda")
    dg, db = torch.empty_like(g), torch.empty_like(g)
    mean = torch.zeros(rows, dtype=torch.float32, device="cuda")
    rstd = torch.ones_like(mean)
    from bloom_bf16_optimizer_amd import _lib
    with pytest.raises(_lib.BloomError) as err:
        ops.bloom_layernorm_bwd_noalloc(x, x, g, mean, rstd, dx, dg, db)
    assert err.value.status == 4 and "scratch" in str(err.value)
