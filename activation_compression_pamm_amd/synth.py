"""Seeded synthetic inputs for PAMM: clustered activations X and gradients dY.

This module only makes inputs.  It holds none of the method's arithmetic and
is the one piece of code that both the HIP path's tests/benchmark and the CPU
oracle's tests use.

The activations stand in for the saved inputs of a transformer QKV projection
(the page "QKV Projections Require a Fraction of Their Memory", section 1 "Il
Problema", and section 2, sub-part "Concetto Fondamentale": many tokens, rows
close to a few directions).  Recipe, in this order, with numpy PCG64:

1. cluster centres ~ N(0, 1)^(clusters x d)
2. a cluster id per row ~ uniform over the clusters
3. a positive scale per row ~ lognormal(mean 0, sigma 0.5)
4. X = scale * centre[id] + N(0, 0.05) noise (0.05 is the standard deviation)
5. optional: a few outlier channels (distinct columns) multiplied by 20
6. optional: a fraction of rows replaced by U(-1, 1)^d (rows of no cluster)
7. dY ~ N(0, 1e-2) (1e-2 is the standard deviation), from its own stream.

Values are drawn in fp32 and rounded once to the storage dtype (bf16 with
round-to-nearest-even, kept as uint16 bit patterns, or fp32).
"""
from __future__ import annotations

import numpy as np

# name -> shape/parameters.  Seeds: data seed 1000 + index, generator seed
# 2000 + index, in the order below.
CONFIGS = {
    "tiny_fp32": dict(index=0, n=1024, d=256, d_out=768, k=8, eps=0.0, clusters=8, dtype="f32"),
    "gpt2_small_qkv": dict(index=1, n=8 * 1024, d=768, d_out=2304, k=16, eps=0.1, clusters=64,
                           outlier_channels=4, dtype="bf16"),
    "llama7b_qkv": dict(index=2, n=16 * 2048, d=4096, d_out=12288, k=64, eps=0.1, clusters=256, dtype="bf16"),
    "llama1b_sweep": dict(index=3, n=32768, d=2048, d_out=6144, k=64, k_sweep=(1024, 256, 128, 64), eps=0.1,
                          clusters=512, dtype="bf16"),
    "longseq_gqa": dict(index=4, n=131072, d=4096, d_out=6144, k=256, eps=0.2, clusters=1024,
                        random_row_frac=0.01, dtype="bf16"),
}


def data_seed(name: str) -> int:
    return 1000 + CONFIGS[name]["index"]


def generator_seed(name: str) -> int:
    return 2000 + CONFIGS[name]["index"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even), returning the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = np.isnan(a)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(dtype)


def clustered_activations(n: int, d: int, clusters: int, seed: int, dtype: str = "bf16",
                          outlier_channels: int = 0, outlier_scale: float = 20.0,
                          random_row_frac: float = 0.0, noise_std: float = 0.05,
                          scale_sigma: float = 0.5, block_rows: int = 8192) -> np.ndarray:
    """Clustered rows as described in the module docstring (steps 1-6)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0]))
    centres = rng.standard_normal((clusters, d), dtype=np.float32)
    ids = rng.integers(0, clusters, size=n)
    scales = rng.lognormal(0.0, scale_sigma, size=n).astype(np.float32)
    out_cols = rng.choice(d, size=outlier_channels, replace=False) if outlier_channels else None
    n_rand = int(round(random_row_frac * n))
    rand_rows = np.sort(rng.choice(n, size=n_rand, replace=False)) if n_rand else np.zeros(0, dtype=np.int64)
    out = np.empty((n, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    noise_rng = np.random.default_rng(np.random.SeedSequence([seed, 1]))
    rand_rng = np.random.default_rng(np.random.SeedSequence([seed, 2]))
    rand_set = np.zeros(n, dtype=bool)
    rand_set[rand_rows] = True
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        blk = centres[ids[r0:r1]] * scales[r0:r1, None]
        blk += noise_std * noise_rng.standard_normal((r1 - r0, d), dtype=np.float32)
        if out_cols is not None:
            blk[:, out_cols] *= np.float32(outlier_scale)
        sel = np.nonzero(rand_set[r0:r1])[0]
        if sel.size:
            blk[sel] = rand_rng.uniform(-1.0, 1.0, size=(sel.size, d)).astype(np.float32)
        out[r0:r1] = _store(blk, dtype)
    return out


def gradients(n: int, d_out: int, seed: int, dtype: str = "bf16", std: float = 1e-2,
              block_rows: int = 8192) -> np.ndarray:
    """Output gradient dY ~ N(0, std) (step 7), from its own random stream."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 3]))
    out = np.empty((n, d_out), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        out[r0:r1] = _store(std * rng.standard_normal((r1 - r0, d_out), dtype=np.float32), dtype)
    return out


def random_matrix(rows: int, cols: int, seed: int, dtype: str = "f32", std: float = 1.0) -> np.ndarray:
    """Unstructured N(0, std) matrix, for small edge-case tests."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4]))
    return _store(std * rng.standard_normal((rows, cols), dtype=np.float32), dtype)


def make_config(name: str, k: int | None = None, rows: int | None = None):
    """Return (X, dY, params) for a named workload.  ``rows`` truncates n
    (used to build a bounded sample of the same distribution)."""
    p = dict(CONFIGS[name])
    if k is not None:
        p["k"] = k
    n = p["n"] if rows is None else rows
    seed = data_seed(name)
    X = clustered_activations(n, p["d"], p["clusters"], seed, p["dtype"],
                              outlier_channels=p.get("outlier_channels", 0),
                              random_row_frac=p.get("random_row_frac", 0.0))
    dY = gradients(n, p["d_out"], seed, p["dtype"])
    p["n"] = n
    return X, dY, p
