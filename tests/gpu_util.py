"""Helpers for the GPU parity tests: move arrays to and from the device, run
the HIP path through the binding, and apply the parity rules against the CPU
oracle.

Parity rules
------------
Indices.  The GPU accumulates each dot product in fp32 (MFMA) and decides in
fp32; the oracle computes in fp64 and decides on the fp64 values rounded to
fp32.  For a sum of d exact products the fp32 error is at most
gamma_d * sum|x_l c_l| <= gamma_d |x||c| (gamma_d = d u / (1 - d u), u = 2^-24,
Higham, Accuracy and Stability of Numerical Algorithms, section 3.1), i.e. at
most gamma_d in cosine units, plus a few roundings of the scaling.  So every
row whose best-vs-runner-up gap and whose distance from eps both exceed
band(d) = 2 gamma_d + 8u must get bit-identical indices.  Inside the band
several answers are correct; the GPU's must then be one of them: its
generator's cosine within the band of the best, and kept/dropped consistently
with eps up to the band.

alpha.  Relative Frobenius error <= 1e-2 (bf16) / 1e-5 (fp32) over rows with
the same index, and per row |da| <= 2 gamma_d |x|/|c| + 8u|alpha|.

dW.  Relative Frobenius error <= 1e-2 (bf16) / 1e-5 (fp32); additionally
<= 1e-4 for bf16, the bound the arithmetic gives (fp32 sums, generator
product with B~ split into two bf16 terms, about 2^-17 relative).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import activation_compression_pamm_amd as pamm
from oracle import oracle as orc

U = 2.0 ** -24
TOL = {"bf16": 1e-2, "f32": 1e-5}
TIGHT = {"bf16": 1e-4, "f32": 1e-5}


# host threads for the oracle: its C calls release the GIL, so row or column
# chunks run in parallel on up to 16 host threads
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_compress(X: np.ndarray, gen_idx: np.ndarray, eps: float, rows: np.ndarray | None = None) -> dict:
    """orc.compress(..., want_scores=True) over `rows` (all rows if None),
    split into row chunks computed by a thread pool."""
    sel = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    if sel.size < 4096 or ORACLE_THREADS == 1:
        return orc.compress(X, gen_idx, eps, rows=sel, want_scores=True)
    parts = np.array_split(sel, 4 * ORACLE_THREADS)
    with cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        outs = list(ex.map(lambda r: orc.compress(X, gen_idx, eps, rows=r, want_scores=True), parts))
    res = {key: np.concatenate([o[key] for o in outs]) for key in ("f", "alpha", "cos", "margin", "scores")}
    res["C"] = outs[0]["C"]
    return res


def oracle_wgrad(C: np.ndarray, f: np.ndarray, a: np.ndarray, dY: np.ndarray,
                 cols: np.ndarray | None = None) -> np.ndarray:
    """orc.wgrad over output columns `cols` (all if None), split into column
    chunks computed by a thread pool."""
    sel = np.arange(dY.shape[1]) if cols is None else np.asarray(cols, dtype=np.int64)
    if sel.size < 256 or ORACLE_THREADS == 1:
        return orc.wgrad(C, f, a, dY, cols=sel)
    parts = np.array_split(sel, 2 * ORACLE_THREADS)
    with cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        outs = list(ex.map(lambda c: orc.wgrad(C, f, a, dY, cols=c), parts))
    return np.concatenate(outs, axis=1)


def band(d: int) -> float:
    g = d * U / (1 - d * U)
    return 2 * g + 8 * U


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return 0.0 if np.linalg.norm(a) == 0 else np.inf
    return float(np.linalg.norm(a - b) / nb)


def dtype_name(a: np.ndarray) -> str:
    return "bf16" if a.dtype == np.uint16 else "f32"


def run_gpu(X: np.ndarray, dY: np.ndarray | None, gen_idx: np.ndarray, eps: float):
    """Compress (and, with dY, wgrad and decompress) on the GPU."""
    Xd = to_dev(X)
    g = torch.from_numpy(np.ascontiguousarray(gen_idx, dtype=np.int32)).cuda()
    C, f, a = pamm.compress(Xd, g, eps)
    out = {"C": C, "f": f, "alpha": a, "X": Xd}
    if dY is not None:
        dYd = to_dev(dY)
        out["dY"] = dYd
        out["dW"] = pamm.wgrad(C, f, a, dYd)
    torch.cuda.synchronize()
    return out


def check_compress(X: np.ndarray, gen_idx: np.ndarray, eps: float, C_g: np.ndarray, f_g: np.ndarray,
                   a_g: np.ndarray, rows: np.ndarray | None = None, return_oracle: bool = False):
    """Apply the index and alpha rules on `rows` (all rows if None).  Returns
    summary statistics (and, with return_oracle, the oracle's f and alpha)."""
    dt = dtype_name(X)
    n, d = X.shape
    k = gen_idx.size
    # C is an exact copy of the generator rows
    assert np.array_equal(C_g, X[gen_idx]), "C differs from X[gen_idx]"
    r = oracle_compress(X, gen_idx, eps, rows=rows)
    sel = np.arange(n) if rows is None else np.asarray(rows)
    fg, ag = f_g[sel], a_g[sel]
    fo, ao = r["f"], r["alpha"]
    cos, margin, scores = r["cos"], r["margin"], r["scores"]
    b = band(d)
    with np.errstate(invalid="ignore"):
        clear = (margin > b) & (np.abs(cos - eps) > b)
    bad_clear = np.nonzero(clear & (fg != fo))[0]
    assert bad_clear.size == 0, (
        f"{bad_clear.size} index mismatches outside the rounding band, e.g. row {sel[bad_clear[0]]}: "
        f"gpu {fg[bad_clear[0]]} oracle {fo[bad_clear[0]]} margin {margin[bad_clear[0]]:.3e}")
    inband = np.nonzero(~clear & (fg != fo))[0]
    for p in inband:
        best = np.nanmax(scores[p]) if k and not np.all(np.isnan(scores[p])) else np.nan
        if fg[p] >= 0:
            assert 0 <= fg[p] < k
            s = scores[p, fg[p]]
            assert s >= best - b, f"row {sel[p]}: gpu pick {fg[p]} cos {s} vs best {best}"
            assert s >= eps - b, f"row {sel[p]}: gpu keeps at cos {s} < eps {eps}"
        else:
            assert not (cos[p] >= eps + b), f"row {sel[p]}: gpu drops a row of cos {cos[p]}"
    same = (fg == fo) & (fo >= 0)
    assert np.all(ag[fg < 0] == 0.0) and np.all(ao[fo < 0] == 0.0)
    Xf = orc.to_f64(X[sel])
    xn = np.linalg.norm(Xf, axis=1)
    Cf = orc.to_f64(X[gen_idx])
    cn = np.linalg.norm(Cf, axis=1) if k else np.zeros(0)
    err_alpha = rel(ag[same], ao[same]) if same.any() else 0.0
    assert err_alpha <= TOL[dt], f"alpha relative error {err_alpha}"
    if same.any():
        fs = fo[same]
        lim = 2 * (b / 2) * xn[same] / np.where(cn[fs] > 0, cn[fs], np.inf) + 8 * U * np.abs(ao[same]) + 1e-37
        da = np.abs(ag[same].astype(np.float64) - ao[same])
        worst = np.argmax(da / lim)
        assert np.all(da <= lim), f"alpha row {sel[same][worst]}: |da| {da[worst]:.3e} > {lim[worst]:.3e}"
    stats = {"inband_mismatches": int(inband.size), "rows": int(sel.size), "kept": float((fg >= 0).mean()),
             "alpha_rel": err_alpha}
    return (stats, fo, ao) if return_oracle else stats


def check_wgrad(C_g: np.ndarray, f_g: np.ndarray, a_g: np.ndarray, dY: np.ndarray, dW_g: np.ndarray,
                cols: np.ndarray | None = None) -> float:
    """dW from the GPU against the oracle's wgrad fed the GPU's triple."""
    dt = dtype_name(dY)
    ref = oracle_wgrad(C_g, f_g, a_g, dY, cols=cols)
    got = dW_g if cols is None else dW_g[:, cols]
    if np.linalg.norm(ref) == 0:
        assert np.all(got == 0)
        return 0.0
    e = rel(got, ref)
    assert e <= TOL[dt], f"dW relative error {e} > {TOL[dt]}"
    assert e <= TIGHT[dt], f"dW relative error {e} above the arithmetic bound {TIGHT[dt]}"
    return e
