"""Per-workload timing of compress and wgrad on one GPU.

For each synthetic workload (the shapes of "QKV Projections Require a
Fraction of Their Memory", section 4 "Risultati Sperimentali"; inputs from `synth`),
this times `pamm_compress` and `pamm_wgrad` separately with HIP events on
the stream they run on:

  * `warmup` untimed calls, then `reps` timed calls of each;
  * before every timed call a 512 MiB buffer is overwritten, so the
    256 MiB memory-side cache holds none of the call's inputs;
  * median, 10th and 90th percentile of the per-call times, less the
    median interval of an empty event pair timed the same way (the event
    packets themselves take a few microseconds).

Derived figures per call (algorithmic work, not counter readings):

  compress  bytes = n*d*s (X) + k*d*s (C) + 8n (f, alpha);
            flops = 2*n*d*k; fraction of the dtype's MFMA peak and of HBM
  wgrad     bytes of dY read densely (n*d_out*s) and of the kept rows only
            (kept*d_out*s), plus the dW write (4*d*d_out)

For bf16 inputs the vendor GEMM of the same product (torch.mm of X and C^T,
bf16 output, no argmax) is timed the same way, as a reference point.

    python -m activation_compression_pamm_amd.report [--workload W] [--k K]
        [--reps 50] [--warmup 5] [--json]

Without --workload every workload runs, the 1B sweep at each of its k.
Progress goes to stderr; the result is one JSON line per run (--json) or a
markdown table.
"""
from __future__ import annotations

import argparse
import json
import sys

HBM_PEAK = 8.0e12                      # bytes/s
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}  # dense flop/s


def _pct(ts, q):
    import numpy as np
    return float(np.percentile(np.asarray(ts), q))


def run_one(name: str, k: int | None, reps: int, warmup: int) -> dict:
    import numpy as np
    import torch

    import activation_compression_pamm_amd as pamm
    from activation_compression_pamm_amd import synth

    def log(*a):
        print(f"[report] {name} k={k}:", *a, file=sys.stderr, flush=True)

    log("generating inputs")
    X, dY, p = synth.make_config(name, k=k)
    n, d, dout, kk, eps = p["n"], p["d"], p["d_out"], p["k"], p["eps"]
    dt = "bf16" if X.dtype == np.uint16 else "f32"
    s = 2 if dt == "bf16" else 4

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    Xd, dYd = dev(X), dev(dY)
    del X, dY
    g = pamm.sample_generators(n, kk, synth.generator_seed(name)).cuda()
    code = pamm.BF16 if dt == "bf16" else pamm.F32
    C = torch.empty((kk, d), dtype=Xd.dtype, device="cuda")
    f = torch.empty(n, dtype=torch.int32, device="cuda")
    al = torch.empty(n, dtype=torch.float32, device="cuda")
    dW = torch.empty((d, dout), dtype=torch.float32, device="cuda")
    cws = torch.empty(max(1, pamm.compress_workspace_size(n, d, kk, code)), dtype=torch.uint8, device="cuda")
    wws = torch.empty(max(1, pamm.wgrad_workspace_size(n, kk, d, dout, code)), dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def comp():
        pamm.compress(Xd, g, eps, C=C, f=f, alpha=al, workspace=cws)

    def wgr():
        pamm.wgrad(C, f, al, dYd, dW=dW, workspace=wws)

    def timed(fn, sub=0.0):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for _ in range(reps):
            flush.fill_(1)
            e0.record(st)
            fn()
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 - sub)  # us
        return ts

    log("timing an empty event pair")
    pair = _pct(timed(lambda: None), 50)
    log("timing compress")
    tc = timed(comp, pair)
    log("timing wgrad")
    tw = timed(wgr, pair)
    kept = int((f >= 0).sum().item())
    vendor = None
    if dt == "bf16":
        # reference point, not part of the path: the vendor GEMM (torch.mm,
        # hipBLASLt) of the same product S = X C^T with a bf16 output and no
        # argmax, timed the same way
        Ct = C.t().contiguous()
        S = torch.empty((n, kk), dtype=torch.bfloat16, device="cuda")
        log("timing the vendor GEMM X C^T")
        vendor = timed(lambda: torch.mm(Xd, Ct, out=S), pair)
        del Ct, S

    cb = n * d * s + kk * d * s + 8 * n
    cf = 2.0 * n * d * kk
    med_c, med_w = _pct(tc, 50), _pct(tw, 50)
    dense, skip, dwb = n * dout * s, kept * dout * s, 4 * d * dout
    out = {
        "workload": name, "n": n, "d": d, "d_out": dout, "k": kk, "eps": eps, "dtype": dt,
        "reps": reps, "warmup": warmup, "cache": "512 MiB overwritten before each timed call",
        "event_pair_us_subtracted": pair,
        "compress_us": {"median": med_c, "p10": _pct(tc, 10), "p90": _pct(tc, 90)},
        "compress_gbs": cb / med_c / 1e3,
        "compress_hbm_frac": cb / (med_c * 1e-6) / HBM_PEAK,
        "compress_mfma_frac": cf / (med_c * 1e-6) / MFMA_PEAK[dt],
        "wgrad_us": {"median": med_w, "p10": _pct(tw, 10), "p90": _pct(tw, 90)},
        "kept_fraction": kept / n,
        "wgrad_dy_dense_gbs": dense / med_w / 1e3,
        "wgrad_dy_kept_gbs": skip / med_w / 1e3,
        "wgrad_dw_write_gbs": dwb / med_w / 1e3,
        "step_tokens_per_s": n / ((med_c + med_w) * 1e-6),
    }
    if vendor is not None:
        med_v = _pct(vendor, 50)
        out["vendor_gemm_us"] = {"median": med_v, "p10": _pct(vendor, 10), "p90": _pct(vendor, 90)}
        out["vendor_gemm_mfma_frac"] = cf / (med_v * 1e-6) / MFMA_PEAK[dt]
    del Xd, dYd, flush
    torch.cuda.empty_cache()
    log("done")
    return out


def to_markdown(rows) -> str:
    lines = ["| workload | k | compress µs median (p10–p90) | compress GB/s | MFMA frac | wgrad µs median (p10–p90) "
             "| kept | dY GB/s dense / kept | tokens/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        c, w = r["compress_us"], r["wgrad_us"]
        lines.append(
            f"| {r['workload']} | {r['k']} | {c['median']:.1f} ({c['p10']:.1f}–{c['p90']:.1f}) | "
            f"{r['compress_gbs']:.0f} | {r['compress_mfma_frac']:.3f} | "
            f"{w['median']:.1f} ({w['p10']:.1f}–{w['p90']:.1f}) | {r['kept_fraction']:.3f} | "
            f"{r['wgrad_dy_dense_gbs']:.0f} / {r['wgrad_dy_kept_gbs']:.0f} | {r['step_tokens_per_s'] / 1e6:.1f} M |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default=None)
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--reps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--json", action="store_true", help="one JSON line per run instead of a table")
    args = ap.parse_args()
    from activation_compression_pamm_amd import synth
    runs = []
    if args.workload:
        runs.append((args.workload, args.k))
    else:
        for name, p in synth.CONFIGS.items():
            for k in p.get("k_sweep", (p["k"],)):
                runs.append((name, k))
    rows = []
    for name, k in runs:
        r = run_one(name, k, args.reps, args.warmup)
        rows.append(r)
        if args.json:
            print(json.dumps(r), flush=True)
    if not args.json:
        print(to_markdown(rows))


if __name__ == "__main__":
    main()
