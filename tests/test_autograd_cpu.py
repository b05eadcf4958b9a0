"""Host-side behaviour of the Python layer: argument checks that fire before
any library call, and the PAMM linear layer's plain-linear paths."""
import pytest
import torch

import activation_compression_pamm_amd as pamm
from activation_compression_pamm_amd.autograd import PammLinear, generators_for


def test_generator_count_follows_the_ratio():
    assert generators_for(32768, 512) == 64
    assert generators_for(1000, 512) == 1      # at least one generator
    assert generators_for(100, 1) == 100       # k = n at ratio 1
    assert generators_for(10**6, 1) == pamm.MAX_K
    assert generators_for(5, 0) == 5           # a ratio below 1 counts as 1


def test_calls_refuse_host_tensors():
    X = torch.zeros(8, 16, dtype=torch.bfloat16)
    g = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="must be on the GPU"):
        pamm.compress(X, g, 0.0)
    C = torch.zeros(2, 16, dtype=torch.bfloat16)
    f = torch.zeros(8, dtype=torch.int32)
    a = torch.zeros(8)
    with pytest.raises(ValueError, match="must be on the GPU"):
        pamm.wgrad(C, f, a, torch.zeros(8, 24, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on the GPU"):
        pamm.decompress(C, f, a)


def test_layer_outside_training_is_a_plain_linear():
    torch.manual_seed(0)
    layer = PammLinear(16, 24, ratio=4, eps=0.1)
    X = torch.randn(3, 5, 16)
    ref = torch.nn.functional.linear(X, layer.weight, layer.bias)
    layer.eval()
    assert torch.equal(layer(X), ref)
    layer.train()
    with torch.no_grad():
        assert torch.equal(layer(X), ref)
    layer.weight.requires_grad_(False)
    assert torch.equal(layer(X), ref)
    assert "ratio=4" in repr(layer)
