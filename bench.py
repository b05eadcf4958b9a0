#!/usr/bin/env python3
"""Throughput of the PAMM hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
pamm_compress (similarity contraction + fused argmax/alpha/eps epilogue) and
pamm_wgrad (counting sort of kept rows, alpha-weighted segmented reduction,
generator product) on the llama-7B QKV workload (n = 16 x 2048 tokens,
d = 4096, d_out = 3 x 4096, k = 64 generators (512x), eps = 0.1, bf16),
with every input resident in HBM before timing starts.  Two input batches
alternate so that no step finds its inputs in the memory-side cache.  Every
step has its own generator set (a new seed per step).  The sets depend only on
(n, k, seed), so they are pipelined: each step draws, on the host, the set of
the step 16 ahead into page-locked memory, and every 16th step uploads the
next 16 sets with one copy on the stream, without a sync.  So each timed step
does one draw (overlapping the GPU's work) and a sixteenth of an upload (one
upload per step would add a few microseconds of GPU timeline each).

The default times 2000 steps (about 0.3 s): under this load the core clock
dips for the first few milliseconds after the GPU leaves idle and recovers
after about a hundred steps, so a window of 100 steps reads mostly the dip
(about 9% fewer tokens/s) while a long-running job sees the steady state.

Prints one JSON line: tokens/s for the whole job, per-call times, a roofline
entry for the dominant kernel (HIP events around its launches on the stream
it runs on) and the CPU oracle timed on the whole step on the host's
cores (cpu_baseline).  An event record costs the GPU a few microseconds,
so events bracket the calls of every --sample-every'th timed step only, and
each such step also records an empty event pair whose interval (the cost of
the event packets themselves) is subtracted from the per-call intervals.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PAMM compress+wgrad tokens/sec; MFMA % peak and HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# HBM bytes per compress launch on the llama-7B QKV workload, from the
# FETCH_SIZE/WRITE_SIZE counters scaled by what they read for a plain copy of
# known size; used while the kernel sources still match the ones profiled
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "compress_llama7b_qkv_traffic.json")
# generator sets uploaded together (see step() in main)
GEN_BATCH = 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="llama7b_qkv")
    p.add_argument("--sample-every", type=int, default=10,
                   help="record per-call HIP events on every this many'th timed step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-threads", type=int, default=max(1, min(16, os.cpu_count() or 1)),
                   help="host threads for the oracle's timing (default: the host's cores, at most 16)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (known bytes) to scale memory counters")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch.
    Profiling it with the FETCH_SIZE / WRITE_SIZE counters gives the factor
    that turns those counters into bytes."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4, "copy_calibration_bytes_written": dst.numel() * 4,
                      "launches": 3}))


def algorithmic(p, kept):
    """Bytes and flops each call must move/compute (2-byte elements)."""
    n, d, dout, k = p["n"], p["d"], p["d_out"], p["k"]
    s = 2 if p["dtype"] == "bf16" else 4
    compress_bytes = n * d * s + k * d * s + 8 * n          # read X, write C, write f and alpha
    compress_flops = 2.0 * n * d * k
    nk = int(round(kept * n))
    reduce_bytes = nk * dout * s + 8 * n                     # read kept dY rows, f and alpha
    product_bytes = 4 * d * dout                             # write dW (fp32)
    product_flops = 2.0 * d * k * dout
    return compress_bytes, compress_flops, reduce_bytes, product_bytes, product_flops


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(X, dY, gen_idx, p, threads):
    """Time the oracle (plain C, fp64) on the host cores over the whole step:
    compress of every row (row chunks) and the B~ sums plus generator product
    of every output column (column chunks), the chunks spread over a pool of
    `threads` threads.  The oracle's C calls release the GIL."""
    import concurrent.futures as cf

    import numpy as np
    from oracle import oracle as orc

    n, dout = p["n"], p["d_out"]
    rows = np.array_split(np.arange(n), 8 * threads)
    cols = np.array_split(np.arange(dout), 4 * threads)
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        parts = list(ex.map(lambda r: orc.compress(X, gen_idx, p["eps"], rows=r), rows))
        t1 = time.perf_counter()
        C = parts[0]["C"]
        f = np.concatenate([q["f"] for q in parts])
        a = np.concatenate([q["alpha"] for q in parts])
        list(ex.map(lambda c: orc.wgrad(C, f, a, dY, cols=c), cols))
        t2 = time.perf_counter()
    est = t2 - t0
    return {
        "value": n / est,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"the whole step (compress of all {n} rows, wgrad of all {dout} output columns) on {threads} "
                   f"threads: compress {t1 - t0:.2f} s, wgrad {t2 - t1:.2f} s"),
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_compression_pamm_amd as pamm
    from activation_compression_pamm_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    name = args.workload
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    X, dY, p = synth.make_config(name)
    n, d, dout, k, eps = p["n"], p["d"], p["d_out"], p["k"], p["eps"]

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    # Two batches alternate from step to step (the second is a row permutation
    # of the first, in its own buffers): together they far exceed the 256 MB
    # memory-side cache, so no step reads data a previous step left cached.
    Xd, dYd = dev(X), dev(dY)
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(12345)).cuda()
    Xb = [Xd, Xd[perm].contiguous()]
    dYb = [dYd, dYd[perm].contiguous()]
    dt_code = pamm.BF16 if p["dtype"] == "bf16" else pamm.F32
    C = torch.empty((k, d), dtype=Xd.dtype, device="cuda")
    f = torch.empty(n, dtype=torch.int32, device="cuda")
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    dW = torch.empty((d, dout), dtype=torch.float32, device="cuda")
    cws = torch.empty(max(pamm.compress_workspace_size(n, d, k, dt_code), 1), dtype=torch.uint8, device="cuda")
    wws = torch.empty(pamm.wgrad_workspace_size(n, k, d, dout, dt_code), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    host_sampling = []             # seconds per generator draw (a1), every step
    # a1 pipelined: step i draws the set of step i + GEN_BATCH on the host into
    # one of two page-locked batch buffers; the last step of a batch uploads
    # the next batch with one copy on the stream (no sync).  Before a buffer
    # is refilled the host waits for the event of its previous upload.
    B = GEN_BATCH
    gen_host = torch.zeros((2, B, max(k, 1)), dtype=torch.int32, pin_memory=True)
    gen_dev = torch.zeros((2, B, max(k, 1)), dtype=torch.int32, device="cuda")
    uploaded = [torch.cuda.Event(), torch.cuda.Event()]

    def draw(i):
        buf = (i // B) % 2
        t = time.perf_counter()
        pamm.load_library().pamm_sample_generators(n, k, synth.generator_seed(name) + i,
                                                   ctypes.c_void_p(gen_host[buf, i % B].data_ptr()))
        host_sampling.append(time.perf_counter() - t)

    def upload(buf):
        gen_dev[buf].copy_(gen_host[buf], non_blocking=True)
        uploaded[buf].record(stream)

    for i in range(B):
        draw(i)
    upload(0)

    def step(i, ev=None):
        """One pass of the whole path for step i: compress with its generator
        set, a1 for step i + GEN_BATCH on the host, wgrad (and the upload of
        the next batch after the last step of a batch)."""
        buf, row = (i // B) % 2, i % B
        if ev is not None:
            ev[0].record(stream)
        pamm.compress(Xb[i % 2], gen_dev[buf, row, :k], eps, C=C, f=f, alpha=a, workspace=cws)
        if ev is not None:
            ev[1].record(stream)
        if row == 0:
            uploaded[1 - buf].synchronize()   # the other buffer's last upload has run
        draw(i + B)
        pamm.wgrad(C, f, a, dYb[i % 2], dW=dW, workspace=wws)
        if ev is not None:
            ev[2].record(stream)
            ev[3].record(stream)
        if row == B - 1:
            upload(1 - buf)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    host_sampling.clear()
    kept = float((f >= 0).float().mean().item())

    # sampled steps sit mid-window: the first timed step follows a host sync,
    # and its events would also time the host catching up with the GPU
    every = max(1, args.sample_every)
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for i in range(every // 2, args.steps, every)} or {0: [torch.cuda.Event(enable_timing=True) for _ in range(4)]}
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs.get(i))
    t_submit = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps
    t_event = sum(e[2].elapsed_time(e[3]) for e in evs.values()) / len(evs)  # ms, empty pair
    t_comp = sum(e[0].elapsed_time(e[1]) for e in evs.values()) / len(evs) - t_event
    t_wgrad = sum(e[1].elapsed_time(e[2]) for e in evs.values()) / len(evs) - t_event
    kept = float((f >= 0).float().mean().item())

    cb, cf, rb, pb, pf = algorithmic(p, kept)
    comp_gbs = cb / (t_comp * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": "compress_rs_kernel (pamm_compress)", "achieved": round(comp_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
                "traffic": None, "algorithmic_bytes_per_launch": cb, "avg_launch_us": round(t_comp * 1e3, 2)}
    if name == "llama7b_qkv" and os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_source_hash") == source_hash():
                roofline["traffic"] = tr["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            pass

    out = {
        "metric": METRIC,
        "value": round(n / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["dtype"],
        "data": "synthetic (clustered activations, Gaussian gradients; seeded)",
        "config": {"workload": name, "n_tokens": n, "d": d, "d_out": dout, "k": k, "eps": eps,
                   "compression": f"{n // k}x"},
        "roofline": roofline,
        "calls": {
            "compress_us": round(t_comp * 1e3, 2),
            "compress_gbs": round(comp_gbs, 1),
            "compress_mfma_frac": round(cf / (t_comp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "wgrad_us": round(t_wgrad * 1e3, 2),
            "wgrad_alg_gbs": round((rb + pb) / (t_wgrad * 1e-3) / 1e9, 1),
            "kept_fraction": round(kept, 4),
            "host_sampling_us": round(1e6 * sum(host_sampling) / max(1, len(host_sampling)), 2),
            "host_submit_us_per_step": round(t_submit * 1e6 / args.steps, 2),
            "event_sampled_steps": len(evs),
            "event_pair_us_subtracted": round(t_event * 1e3, 2),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the whole step", file=sys.stderr, flush=True)
        g0 = pamm.sample_generators(n, k, synth.generator_seed(name) + args.warmup).numpy()
        out["cpu_baseline"] = cpu_baseline(X, dY, g0, p, args.cpu_threads)
    print(json.dumps(out), flush=True)


def source_hash() -> str:
    """Hash of the sources the compress kernel is built from (its file and
    the headers it includes), with comments and blank lines removed, so that
    documentation edits keep the profiled traffic figure attached."""
    import hashlib
    import re
    h = hashlib.sha256()
    src = os.path.join(ROOT, "activation_compression_pamm_amd", "csrc")
    for fn in sorted(os.listdir(src)):
        if fn in ("pamm_compress.hip", "pamm_device.hpp", "pamm_kernels.hpp"):
            text = open(os.path.join(src, fn), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
            h.update(code.encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
