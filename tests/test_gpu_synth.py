"""The device generator writes exactly the values the host generator defines."""

import numpy as np
import pytest
import torch

import synth
from synth import device as sdev
from parity_helpers import host_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,mode,sigma,offset", [
    (torch.bfloat16, synth.MODE_BF16, 1.0, 0.0),
    (torch.bfloat16, synth.MODE_BF16, 0.02, 1.0),
    (torch.float32, synth.MODE_F32, 1e-3, 0.0),
    (torch.float32, synth.MODE_ABS_F32, 1e-6, 0.0),
])
def test_device_matches_host(dtype, mode, sigma, offset):
    require_gpu()
    n = 300_007
    t = torch.empty(n, dtype=dtype, device="cuda")
    if mode == synth.MODE_ABS_F32:
        sdev.fill_abs_(t, 4, 33, sigma)
    else:
        sdev.fill_(t, 4, 33, sigma, offset)
    got = host_bf16(t) if dtype == torch.bfloat16 else t.cpu().numpy()
    want = synth.tensor(4, 33, n, sigma, offset, mode)
    assert np.array_equal(got.view(np.uint16 if dtype == torch.bfloat16 else np.uint32),
                          want.view(np.uint16 if dtype == torch.bfloat16 else np.uint32))


def test_device_matches_host_at_large_indices():
    """Element indices beyond 2^32 (the 3.67e9-element shard) and a start offset."""
    require_gpu()
    start = 3_670_000_000 - 5000
    t = torch.empty(5000, dtype=torch.bfloat16, device="cuda")
    sdev.fill_(t, 4, 100 + 32, 1e-3, start=start)
    want = synth.tensor(4, 132, 5000, 1e-3, mode=synth.MODE_BF16, start=start)
    assert np.array_equal(host_bf16(t), want)
