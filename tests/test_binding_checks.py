"""The Python binding's argument checks: tensors that are not on the GPU, of
the wrong dtype, not contiguous or of disagreeing shapes are refused before
anything reaches the library, and a status from the library surfaces as a
BloomError that names the entry point.  The first group runs on the CPU (the
checks fire before any device call); the second needs a GPU tensor to get past
the device check."""

import pytest
import torch

from bloom_bf16_optimizer_amd import _lib, ops
from parity_helpers import require_gpu

bf = torch.bfloat16
f32 = torch.float32


def _cpu(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def test_cpu_tensors_are_refused():
    x, y = _cpu(4, 64), _cpu(4, 64)
    g, b = _cpu(64), _cpu(64)
    m, r = _cpu(4, dtype=f32), _cpu(4, dtype=f32)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bloom_layernorm_fwd(x, g, b, y, m, r, 1e-5)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bloom_bias_gelu_fwd(x, g, y)
    s = _cpu(1, 2, 16, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bloom_alibi_softmax_fwd(s, torch.zeros_like(s), 0, 2, 0.25)
    acc = _cpu(1024, dtype=f32)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bloom_bf16_grad_accumulate(acc, _cpu(1024), True)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bloom_bf16_grad_accumulate_many(acc, [_cpu(1024), _cpu(1024)], True)


def test_shape_disagreements_are_refused():
    with pytest.raises(ValueError, match="shapes"):
        ops.bloom_layernorm_fwd(_cpu(4, 64), _cpu(64), _cpu(64), _cpu(4, 32), _cpu(4, dtype=f32),
                                _cpu(4, dtype=f32), 1e-5)
    with pytest.raises(ValueError, match="bias"):
        ops.bloom_bias_gelu_fwd(_cpu(4, 64), _cpu(32), _cpu(4, 64))
    with pytest.raises(ValueError, match="same number of elements"):
        ops.bloom_bf16_grad_accumulate_many(_cpu(1024, dtype=f32), [_cpu(1024), _cpu(512)], True)
    q = _cpu(1, 2, 16, 32)
    with pytest.raises(ValueError):
        ops.bloom_alibi_attention_fwd(q, _cpu(1, 2, 8, 32), q, torch.zeros_like(q), _cpu(1, 2, 16, dtype=f32), 0, 2,
                                      0.25)


@pytest.mark.gpu
def test_dtype_and_contiguity_are_refused_on_the_gpu():
    require_gpu()
    x = torch.zeros(4, 64, dtype=bf, device="cuda")
    g, b = torch.ones(64, dtype=bf, device="cuda"), torch.zeros(64, dtype=bf, device="cuda")
    m, r = torch.empty(4, dtype=f32, device="cuda"), torch.empty(4, dtype=f32, device="cuda")
    with pytest.raises(TypeError, match="bfloat16"):
        ops.bloom_layernorm_fwd(x.float(), g, b, torch.empty_like(x).float(), m, r, 1e-5)
    xt = torch.zeros(64, 4, dtype=bf, device="cuda").t()          # [4, 64] view, not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        ops.bloom_layernorm_fwd(xt, g, b, torch.empty(4, 64, dtype=bf, device="cuda"), m, r, 1e-5)
    with pytest.raises(TypeError, match="float32"):
        ops.bloom_layernorm_fwd(x, g, b, torch.empty_like(x), m.to(bf), r, 1e-5)


@pytest.mark.gpu
def test_library_status_surfaces_as_bloom_error():
    require_gpu()
    # seq = 12 is not a multiple of 8: the library refuses it before any launch
    s = torch.zeros(1, 1, 12, 12, dtype=bf, device="cuda")
    with pytest.raises(_lib.BloomError) as e:
        ops.bloom_alibi_softmax_fwd(s, torch.zeros_like(s), 0, 1, 0.25)
    assert "bloom_alibi_softmax_fwd" in str(e.value)
    # eps must be positive
    x = torch.zeros(4, 64, dtype=bf, device="cuda")
    g, b = torch.ones(64, dtype=bf, device="cuda"), torch.zeros(64, dtype=bf, device="cuda")
    with pytest.raises(_lib.BloomError):
        ops.bloom_layernorm_fwd(x, g, b, torch.empty_like(x), torch.empty(4, dtype=f32, device="cuda"),
                                torch.empty(4, dtype=f32, device="cuda"), 0.0)
    torch.cuda.synchronize()
