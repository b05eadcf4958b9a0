"""GPU: the transposed output of pamm_wgrad, and the PAMM linear layer's
outputs and gradients against exact and oracle references."""
import sys
import warnings

import numpy as np
import pytest
import torch

import activation_compression_pamm_amd as pamm
from activation_compression_pamm_amd import synth
from activation_compression_pamm_amd.autograd import PammLinear, generators_for
from oracle import oracle as orc

from gpu_util import TOL, rel, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("k", [40, 300])   # 300: the wide product tile
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_transposed_output_is_the_transpose(dtype, k):
    n, d, dout = 3000, 200, 296
    say("transpose_out", dtype, f"n={n} d={d} d_out={dout} k={k}")
    X = synth.clustered_activations(n, d, 16, seed=5, dtype=dtype)
    dY = synth.gradients(n, dout, seed=6, dtype=dtype)
    g = pamm.sample_generators(n, k, 7).cuda()
    C, f, a = pamm.compress(to_dev(X), g, 0.1)
    dYd = to_dev(dY)
    dW = pamm.wgrad(C, f, a, dYd)
    dWt = pamm.wgrad(C, f, a, dYd, transpose_out=True)
    torch.cuda.synchronize()
    assert dWt.shape == (dout, d)
    # the same products summed in the same order, only stored transposed
    assert torch.equal(dWt, dW.t())
    # accumulate into a strided [d_out x d] view; the padding stays untouched
    big = torch.randn(dout, d + 24, device="cuda")
    before = big.clone()
    view = big[:, 8:8 + d]
    pamm.wgrad(C, f, a, dYd, dW=view, accumulate=True, transpose_out=True)
    torch.cuda.synchronize()
    assert torch.equal(view, before[:, 8:8 + d] + dW.t())
    assert torch.equal(big[:, :8], before[:, :8]) and torch.equal(big[:, 8 + d:], before[:, 8 + d:])


@pytest.mark.parametrize("d,dout", [(256, 384), (123, 157)])   # 123, 157: rows off 16 bytes, padded inside
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pamm_linear_outputs_and_gradients(dtype, d, dout):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Bt, S, ratio, eps = 4, 512, 16, 0.1
    n = Bt * S
    say("PammLinear", dtype, f"X [{Bt}x{S}x{d}] -> [{dout}], ratio={ratio} eps={eps}")
    torch.manual_seed(0)
    layer = PammLinear(d, dout, ratio=ratio, eps=eps, seed=11, device="cuda", dtype=tdt)
    X = to_dev(synth.clustered_activations(n, d, 32, seed=12, dtype=dtype)).reshape(Bt, S, d).requires_grad_(True)
    G = torch.randn(Bt, S, dout, device="cuda", generator=torch.Generator(device="cuda").manual_seed(13))
    seed = layer._next_seed
    saved = []
    with torch.autograd.graph.saved_tensors_hooks(lambda t: (saved.append(t), t)[1], lambda t: t):
        Y = layer(X)
    (Y.float() * G).sum().backward()
    torch.cuda.synchronize()
    dY = G.to(tdt).reshape(n, dout)  # the gradient autograd hands the layer

    W64 = layer.weight.detach().double().cpu()
    X64 = X.detach().double().cpu().reshape(n, d)
    dY64 = dY.double().cpu()
    # forward and the exact gradients
    Yref = X64 @ W64.T + layer.bias.detach().double().cpu()
    assert rel(Y.detach().double().cpu().reshape(n, dout).numpy(), Yref.numpy()) <= TOL[dtype]
    assert rel(X.grad.double().cpu().reshape(n, d).numpy(), (dY64 @ W64).numpy()) <= TOL[dtype]
    assert rel(layer.bias.grad.double().cpu().numpy(), dY64.sum(0).numpy()) <= TOL[dtype]
    # the weight gradient: the oracle's wgrad fed the same compressed triple
    k = generators_for(n, ratio)
    g = pamm.sample_generators(n, k, seed)
    Xp = torch.zeros((n, (d + 7) // 8 * 8), dtype=tdt, device="cuda")   # rows 16-byte multiples
    Xp[:, :d] = X.detach().reshape(n, d)
    C, f, a = pamm.compress(Xp[:, :d], g.cuda(), eps)
    dW_o = orc.wgrad(to_host(C), to_host(f), to_host(a), to_host(dY))
    assert layer.weight.grad.is_contiguous()
    assert rel(layer.weight.grad.double().cpu().numpy().T, dW_o) <= TOL[dtype]
    # what the backward pass keeps: the triple and W, never X
    assert sorted(tuple(t.shape) for t in saved) == sorted([(k, d), (n,), (n,), (dout, d)])
    nbytes = sum(t.numel() * t.element_size() for t in saved)
    dt = pamm.BF16 if dtype == "bf16" else pamm.F32
    assert nbytes == pamm.compressed_nbytes(n, k, d, dt) + layer.weight.numel() * layer.weight.element_size()
    say("PammLinear", dtype, "ok", f"k={k} saved {nbytes} bytes, X is {X.numel() * X.element_size()}")


def test_pamm_linear_with_every_row_a_generator_is_exact():
    # ratio 1: k = n, every token is its own generator with alpha = 1
    n, d, dout = 1024, 128, 96
    say("PammLinear ratio=1", f"n={n} d={d} d_out={dout}")
    layer = PammLinear(d, dout, ratio=1, eps=0.0, device="cuda", dtype=torch.float32)
    X = to_dev(synth.random_matrix(n, d, 21, "f32")).requires_grad_(True)
    dY = to_dev(synth.random_matrix(n, dout, 22, "f32"))
    layer(X).backward(dY)
    torch.cuda.synchronize()
    exact = dY.double().cpu().T @ X.detach().double().cpu()
    assert rel(layer.weight.grad.double().cpu().numpy(), exact.numpy()) <= TOL["f32"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pamm_linear_training_step_does_not_synchronize(dtype):
    # Forward and backward enqueue work only: the generator draw goes to
    # page-locked memory and uploads without a stream synchronisation, and no
    # step reads a device value back.  torch's sync debug mode raises on any
    # synchronising torch operation.
    n, d, dout = 4096, 256, 384
    say("PammLinear no sync", f"{dtype} n={n} d={d} d_out={dout}")
    layer = PammLinear(d, dout, ratio=64, eps=0.1, device="cuda", dtype=dtype)
    X = torch.randn(n, d, device="cuda", dtype=dtype, requires_grad=True)
    dY = torch.randn(n, dout, device="cuda", dtype=dtype)
    layer(X).backward(dY)                 # first call: library load, allocator warm-up
    torch.cuda.synchronize()
    layer.zero_grad(set_to_none=True)
    X.grad = None
    probe = torch.zeros(1, device="cuda")
    prev = torch.cuda.get_sync_debug_mode()
    with warnings.catch_warnings():   # torch warns that the mode is a prototype
        warnings.simplefilter("ignore")
        torch.cuda.set_sync_debug_mode("error")
    try:
        with pytest.raises(RuntimeError):
            probe.item()                  # the mode is live: a read-back raises
        for _ in range(2):
            layer(X).backward(dY)
    finally:
        torch.cuda.set_sync_debug_mode(prev)
    torch.cuda.synchronize()
    assert torch.isfinite(layer.weight.grad.float()).all() and torch.isfinite(X.grad.float()).all()


def test_error_sweep_runs_and_reports_sane_values():
    from activation_compression_pamm_amd import sweep
    say("sweep", "llama1b_sweep k=64 eps=0,0.1")
    res = sweep.run([64], [0.0, 0.1])
    r0, r1 = res["rows"]
    assert r0["kept_fraction"] == 1.0                  # eps = 0 keeps every row
    assert 0.0 < r1["kept_fraction"] < 1.0
    assert 0.0 < r0["rel_error"] < 1.0 and 0.0 < r1["rel_error"] < 1.0
    assert "| 64 | 512 | 0.0 |" in sweep.to_markdown(res)
