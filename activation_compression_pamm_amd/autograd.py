"""PAMM inside a PyTorch linear layer.

"QKV Projections Require a Fraction of Their Memory", section 2
"Metodologia": the method plugs into the projection's training step without
touching the weights or inference.  The forward pass computes Y = X W^T + b
exactly and, instead of saving the input X for the weight gradient, saves
the compressed triple (C, f, alpha) of "Algoritmo in Due Fasi".  The backward
pass computes

    dX     = dY W                      exactly (plain library GEMM),
    W.grad = (C^T B~)^T                from the triple (pamm_wgrad, written
                                       directly in W's [out x in] layout),
    b.grad = sum of the rows of dY     exactly.

k, the number of generators, is n / ratio for the n tokens of a batch (the
page's k/b ratio, down to 1/512), at least 1 and at most n and MAX_K.
Generators are drawn on the host from a per-call seed, so a training run is
reproducible.
"""
from __future__ import annotations

import torch

from . import MAX_K, _empty_rows, compress, sample_generators, wgrad

__all__ = ["PammLinearFunction", "PammLinear", "generators_for"]


def _aligned_rows(t2):
    """t2 [rows x cols] itself when its rows are contiguous and start a
    multiple of 16 bytes apart (what the library's calls ask of their
    inputs), else a copy into a buffer with rows padded to 16 bytes."""
    if t2.stride(1) == 1 and (t2.stride(0) * t2.element_size()) % 16 == 0 and t2.data_ptr() % 16 == 0:
        return t2
    out = _empty_rows(t2.shape[0], t2.shape[1], t2.dtype, t2.device)
    out.copy_(t2)
    return out


def generators_for(n: int, ratio: int) -> int:
    """Generator count for n tokens at compression ratio n/k = ratio."""
    return max(1, min(n, MAX_K, n // max(1, int(ratio))))


class PammLinearFunction(torch.autograd.Function):
    """Y = X W^T (+ b) whose backward approximates W's gradient with PAMM.

    X [..., d] (bf16 or fp32, on the GPU), W [d_out x d] and b [d_out] of the
    same dtype.  Only (C, f, alpha) and W are saved for the backward pass."""

    @staticmethod
    def forward(ctx, X, W, b, k: int, eps: float, seed: int):
        d = X.shape[-1]
        X2 = X.reshape(-1, d)
        if not X2.is_contiguous():
            X2 = X2.contiguous()
        Xc = _aligned_rows(X2)   # X2 itself unless d leaves its rows off 16 bytes
        # generators: drawn on the host into page-locked memory and uploaded
        # asynchronously ahead of the projection, so the upload neither syncs
        # the stream nor waits behind the GEMM (torch keeps the host buffer
        # alive until the copy has run)
        gen = sample_generators(X2.shape[0], k, seed, pin=True).to(X.device, non_blocking=True)
        Y = torch.nn.functional.linear(X2, W, b)
        C, f, alpha = compress(Xc, gen, eps)
        ctx.save_for_backward(C, f, alpha, W)
        ctx.has_bias = b is not None
        ctx.x_shape = X.shape
        return Y.reshape(*X.shape[:-1], W.shape[0])

    @staticmethod
    def backward(ctx, dY):
        C, f, alpha, W = ctx.saved_tensors
        dY2 = dY.reshape(-1, dY.shape[-1])
        if not dY2.is_contiguous():
            dY2 = dY2.contiguous()
        dX = dW = db = None
        if ctx.needs_input_grad[0]:
            dX = (dY2 @ W).reshape(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            dW = wgrad(C, f, alpha, _aligned_rows(dY2), transpose_out=True)
            if dW.dtype != W.dtype:
                dW = dW.to(W.dtype)
            if not dW.is_contiguous():  # rows padded to 16 bytes when in_features is ragged
                dW = dW.contiguous()
        if ctx.has_bias and ctx.needs_input_grad[2]:
            db = dY2.float().sum(0).to(dY2.dtype)
        return dX, dW, db, None, None, None


class PammLinear(torch.nn.Linear):
    """nn.Linear whose training-time weight gradient comes from PAMM.

    ratio: tokens per generator (n/k); eps: cosine threshold below which a
    token is dropped from the weight gradient (0 keeps every token); seed:
    first generator seed, advanced by one per training forward pass.
    Evaluation, no-grad and frozen-weight passes are a plain linear layer."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, *, ratio: int = 512,
                 eps: float = 0.0, seed: int = 0, device=None, dtype=None):
        super().__init__(in_features, out_features, bias=bias, device=device, dtype=dtype)
        self.ratio = int(ratio)
        self.eps = float(eps)
        self._next_seed = int(seed)

    def forward(self, X):
        if not (self.training and torch.is_grad_enabled() and self.weight.requires_grad):
            return torch.nn.functional.linear(X, self.weight, self.bias)
        n = X.numel() // X.shape[-1]
        seed = self._next_seed
        self._next_seed += 1
        return PammLinearFunction.apply(X, self.weight, self.bias, generators_for(n, self.ratio), self.eps, seed)

    def extra_repr(self) -> str:
        return super().extra_repr() + f", ratio={self.ratio}, eps={self.eps}"
