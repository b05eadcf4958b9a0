"""GPU: pamm_wgrad_noalloc (the weight gradient with the library's fixed
scratch array as workspace, for callers that cannot allocate) against
pamm_wgrad with a caller workspace, through the C ABI.  Two calls in a row,
the second on a smaller input, then the first again: the shared array keeps
each call's leftovers, which must not leak into the next result."""
import sys

import numpy as np
import pytest
import torch

import activation_compression_pamm_amd as pamm
from activation_compression_pamm_amd import synth

from gpu_util import check_wgrad, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


CASES = [
    # n, d, d_out, k, eps, dtype, transpose_out, accumulate
    (20000, 512, 1536, 64, 0.1, "bf16", False, False),
    (3000, 256, 384, 16, 0.0, "bf16", True, True),     # smaller, transposed, accumulating
    (1500, 128, 200, 24, 0.1, "f32", False, False),
    (20000, 512, 1536, 64, 0.1, "bf16", False, False),  # the first again after smaller calls
]


def test_noalloc_matches_workspace_call():
    for i, (n, d, dout, k, eps, dtype, tr, acc) in enumerate(CASES):
        say("noalloc", f"call {i}: n={n} d={d} d_out={dout} k={k} {dtype} transpose_out={tr} accumulate={acc}")
        X = synth.clustered_activations(n, d, max(2, k // 2), seed=500 + i, dtype=dtype)
        dY = synth.gradients(n, dout, seed=600 + i, dtype=dtype)
        g = torch.from_numpy(pamm.sample_generators(n, k, 700 + i).numpy()).cuda()
        C, f, a = pamm.compress(to_dev(X), g, eps)
        dYd = to_dev(dY)
        shape = (dout, d) if tr else (d, dout)
        init = torch.randn(shape, device="cuda") if acc else torch.zeros(shape, device="cuda")
        ref = pamm.wgrad(C, f, a, dYd, dW=init.clone(), accumulate=acc, transpose_out=tr)
        # the no-allocation call writes into a buffer filled with garbage first
        got = torch.full(shape, float("nan"), device="cuda")
        if acc:
            got.copy_(init)
        pamm.wgrad_noalloc(C, f, a, dYd, got, accumulate=acc, transpose_out=tr)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: differs from pamm_wgrad"
        # and to the oracle's wgrad of the same triple
        dW = to_host(got) - (to_host(init) if acc else 0.0)
        check_wgrad(to_host(C), to_host(f), to_host(a), dY, dW.T if tr else dW)
        say("noalloc", f"call {i} ok")


def test_noalloc_refuses_too_large_without_launch():
    # 65536 tokens x 12288 outputs with 4096 generators: beyond the array;
    # refused on the host before anything is enqueued (no tensor is touched)
    k, d, n, dout = 4096, 8, 65536, 12288
    C = torch.zeros((k, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(n, dtype=torch.int32, device="cuda")
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    dY = torch.empty((n, dout), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((d, dout), 5.0, device="cuda")
    with pytest.raises(pamm.PammError, match="scratch array"):
        pamm.wgrad_noalloc(C, f, a, dY, dW)
    torch.cuda.synchronize()
    assert torch.all(dW == 5.0)
