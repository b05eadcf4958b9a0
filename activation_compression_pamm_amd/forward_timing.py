"""Timing of the fused forward pass against the two-call forward pass.

"QKV Projections Require a Fraction of Their Memory", section 2
"Metodologia", "Algoritmo in Due Fasi": the compressed form of the
projection's input is computed during the forward pass.  Two ways to do that
on one GPU, on seeded synthetic bf16 inputs of the QKV projection's shapes:

  separate   Y = X W^T + b by the library GEMM (torch.nn.functional.linear),
             then pamm_compress, which reads X again
  fused      pamm_forward_compress: one pass over X computes Y and the
             compression together

Per call: `warmup` untimed calls, then `reps` calls, each bracketed by HIP
events on the stream it runs on; the median, less the median of an empty
event pair.  The separate variant is timed as one interval around both calls.

    python -m activation_compression_pamm_amd.forward_timing [--reps 20] [--warmup 3] [--json]
"""
from __future__ import annotations

import argparse
import json
import sys

SHAPES = [
    # name, n, d, d_out, k, eps
    ("llama7b_qkv", 32768, 4096, 12288, 64, 0.1),
    ("llama1b_qkv k=64", 32768, 2048, 6144, 64, 0.1),
    ("llama1b_qkv k=1024", 32768, 2048, 6144, 1024, 0.1),
]


def run(reps: int, warmup: int) -> list:
    import numpy as np
    import torch

    import activation_compression_pamm_amd as pamm
    from activation_compression_pamm_amd import synth

    st = torch.cuda.current_stream()

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        emp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for _ in range(warmup):
            fn()
        for (a, b), (c, e) in zip(evs, emp):
            a.record(st)
            fn()
            b.record(st)
            c.record(st)
            e.record(st)
        torch.cuda.synchronize()
        t = np.median([a.elapsed_time(b) for a, b in evs]) - np.median([c.elapsed_time(e) for c, e in emp])
        return float(t) * 1e3  # microseconds

    out = []
    for name, n, d, d_out, k, eps in SHAPES:
        print(f"[forward_timing] {name}", file=sys.stderr, flush=True)
        Xh = synth.clustered_activations(n, d, 256, seed=11, dtype="bf16")
        X = torch.from_numpy(Xh.view(np.int16)).view(torch.bfloat16).cuda()
        W = (torch.randn(d_out, d, device="cuda") * 0.02).to(torch.bfloat16)
        b = (torch.randn(d_out, device="cuda") * 0.02).to(torch.bfloat16)
        g = pamm.sample_generators(n, k, 5).cuda()
        Y = torch.empty((n, d_out), dtype=torch.bfloat16, device="cuda")
        C = torch.empty((k, d), dtype=torch.bfloat16, device="cuda")
        f = torch.empty(n, dtype=torch.int32, device="cuda")
        a = torch.empty(n, dtype=torch.float32, device="cuda")
        cws = torch.empty(max(1, pamm.compress_workspace_size(n, d, k, pamm.BF16)), dtype=torch.uint8, device="cuda")
        fws = torch.empty(pamm.forward_compress_workspace_size(n, d, k), dtype=torch.uint8, device="cuda")

        def gemm_only():
            torch.addmm(b, X, W.t(), out=Y)

        def sep():
            torch.addmm(b, X, W.t(), out=Y)
            pamm.compress(X, g, eps, C=C, f=f, alpha=a, workspace=cws)

        def comp_only():
            pamm.compress(X, g, eps, C=C, f=f, alpha=a, workspace=cws)

        def fused():
            pamm.forward_compress(X, W, g, eps, bias=b, Y=Y, C=C, f=f, alpha=a, workspace=fws)

        r = {"shape": name, "n": n, "d": d, "d_out": d_out, "k": k,
             "gemm_us": round(timed(gemm_only), 1), "compress_us": round(timed(comp_only), 1),
             "separate_us": round(timed(sep), 1), "fused_us": round(timed(fused), 1)}
        flops = 2.0 * n * d * (d_out + k)
        r["fused_tflops"] = round(flops / (r["fused_us"] * 1e-6) / 1e12, 1)
        r["gemm_tflops"] = round(2.0 * n * d * d_out / (r["gemm_us"] * 1e-6) / 1e12, 1)
        r["fused_vs_separate"] = round(r["fused_us"] / r["separate_us"], 4)
        out.append(r)
        del X, W, Y
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args()
    res = run(args.reps, args.warmup)
    for r in res:
        print(json.dumps(r) if args.json else " ".join(f"{k}={v}" for k, v in r.items()))


if __name__ == "__main__":
    main()
