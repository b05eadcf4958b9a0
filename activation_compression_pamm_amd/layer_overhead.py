"""Cost of a PAMM linear layer against a plain one, forward + backward.

"QKV Projections Require a Fraction of Their Memory", section 2
"Metodologia": PAMM plugs into a projection's training step; section 4
reports end-to-end throughput within a few percent of the baseline.  This
times one training step of the QKV projection alone, on synthetic tensors of
the llama-7B QKV shape (X [16 x 2048 x 4096] bf16, W [12288 x 4096], bias):

  plain    nn.Linear: forward Y = X W^T + b, backward dX = dY W, W.grad =
           dY^T X, b.grad (X saved for the backward pass);
  pamm     PammLinear (ratio 512, eps 0.1): the same forward plus the
           generator draw and pamm_compress, backward dX = dY W, W.grad
           from pamm_wgrad, b.grad (only (C, f, alpha) saved).

Each variant runs `warmup` untimed steps, then `steps` timed steps between
two synchronisations (wall clock).  Also reported: the bytes each layer keeps
for its backward pass (beyond the weight).

    python -m activation_compression_pamm_amd.layer_overhead [--steps 20] [--warmup 5] [--json]
"""
from __future__ import annotations

import argparse
import json
import time


def run(steps: int, warmup: int, batch: int = 16, seq: int = 2048, d: int = 4096, d_out: int = 12288,
        ratio: int = 512, eps: float = 0.1) -> dict:
    import torch

    from activation_compression_pamm_amd import synth
    from activation_compression_pamm_amd.autograd import PammLinear, generators_for

    dev = "cuda"
    n = batch * seq
    torch.manual_seed(0)
    Xb = synth.clustered_activations(n, d, 256, seed=1002, dtype="bf16")
    import numpy as np
    X0 = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(batch, seq, d)
    G = (torch.randn(batch, seq, d_out, device=dev) * 1e-2).to(torch.bfloat16)
    plain = torch.nn.Linear(d, d_out, device=dev, dtype=torch.bfloat16)
    pamm_layer = PammLinear(d, d_out, ratio=ratio, eps=eps, seed=7, device=dev, dtype=torch.bfloat16)
    with torch.no_grad():
        pamm_layer.weight.copy_(plain.weight)
        pamm_layer.bias.copy_(plain.bias)

    def saved_bytes(layer):
        total = 0

        def pack(t):
            nonlocal total
            if t.data_ptr() not in (layer.weight.data_ptr(),):
                total += t.numel() * t.element_size()
            return t

        X = X0.detach().requires_grad_(True)
        with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
            Y = layer(X)
        Y.backward(G)
        return total

    def time_layer(layer):
        X = X0.detach().requires_grad_(True)
        for _ in range(warmup):
            layer.zero_grad(set_to_none=True)
            X.grad = None
            layer(X).backward(G)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.zero_grad(set_to_none=True)
            X.grad = None
            layer(X).backward(G)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    res = {"shape": {"tokens": n, "d": d, "d_out": d_out, "k": generators_for(n, ratio), "eps": eps,
                     "dtype": "bf16"},
           "steps": steps, "warmup": warmup}
    for name, layer in (("plain", plain), ("pamm", pamm_layer), ("plain_again", plain)):
        res[f"{name}_ms"] = round(1e3 * time_layer(layer), 3)
    res["plain_saved_bytes"] = saved_bytes(plain)
    res["pamm_saved_bytes"] = saved_bytes(pamm_layer)
    plain_ms = min(res["plain_ms"], res["plain_again_ms"])
    res["pamm_vs_plain"] = round(res["pamm_ms"] / plain_ms, 4)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--json", action="store_true")
    a = ap.parse_args()
    res = run(a.steps, a.warmup)
    if a.json:
        print(json.dumps(res))
    else:
        for k, v in res.items():
            print(f"{k}: {v}")


if __name__ == "__main__":
    main()
