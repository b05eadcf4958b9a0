"""CPU oracle for PAMM: a thin numpy/ctypes wrapper over ``pamm_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its binding) never touches it, and the two share no
code.  Every function here forwards to the plain fp64 C reference, which
follows the page "QKV Projections Require a Fraction of Their Memory",
section 2 "Metodologia", sub-part "Algoritmo in Due Fasi" (compression in the
forward pass, compressed gradient and generator product in the backward pass).

Dtype codes: 0 = fp32 (numpy float32 arrays), 1 = bf16 (numpy uint16 arrays
holding the raw bf16 bit patterns).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pamm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.orc_splitmix64_stream.argtypes = [ctypes.c_uint64, i64, p]
    lib.orc_sample_generators.argtypes = [i64, i64, ctypes.c_uint64, p]
    lib.orc_gather.argtypes = [p, i64, i64, i64, ctypes.c_int, p, i64, p]
    lib.orc_compress.argtypes = [p, i64, i64, i64, ctypes.c_int, p, i64, ctypes.c_double,
                                 p, i64, p, p, p, p, p]
    lib.orc_wgrad.argtypes = [p, ctypes.c_int, p, p, i64, i64, i64, p, i64, i64, p, i64, p]
    lib.orc_decompress.argtypes = [p, ctypes.c_int, p, p, i64, i64, i64, p, p]
    lib.orc_footprint_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.orc_footprint_bytes.restype = i64
    for name in ("orc_splitmix64_stream", "orc_sample_generators", "orc_gather", "orc_compress",
                 "orc_wgrad", "orc_decompress"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are float32 or bf16-as-uint16, got {a.dtype}")


def _rows_view(a: np.ndarray) -> tuple[np.ndarray, int]:
    """(array, leading dimension in elements) for a row-major 2-D matrix.  A
    view whose rows are contiguous but lie further apart than their length
    (a column slice of a wider matrix) is passed as it is, with its row
    stride as the leading dimension; anything else is copied densely."""
    es = a.itemsize
    if (a.ndim == 2 and a.shape[0] > 0 and a.shape[1] > 0 and a.strides[1] == es
            and a.strides[0] % es == 0 and a.strides[0] // es >= a.shape[1]):
        return a, a.strides[0] // es
    a = np.ascontiguousarray(a)
    return a, (a.shape[1] if a.ndim == 2 else 0)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def splitmix64_stream(seed: int, count: int) -> np.ndarray:
    out = np.zeros(count, dtype=np.uint64)
    _check(_load().orc_splitmix64_stream(seed, count, _ptr(out)), "splitmix64_stream")
    return out


def sample_generators(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct row ids in [0, n), ascending (Floyd + SplitMix64)."""
    out = np.zeros(max(k, 0), dtype=np.int32)
    _check(_load().orc_sample_generators(n, k, seed, _ptr(out)), "sample_generators")
    return out


def gather(X: np.ndarray, gen_idx: np.ndarray) -> np.ndarray:
    X, ldx = _rows_view(X)
    gen_idx = np.ascontiguousarray(gen_idx, dtype=np.int32)
    n, d = X.shape
    C = np.zeros((gen_idx.size, d), dtype=X.dtype)
    _check(_load().orc_gather(_ptr(X), n, d, ldx, _dtype_code(X), _ptr(gen_idx), gen_idx.size, _ptr(C)), "gather")
    return C


def compress(X: np.ndarray, gen_idx: np.ndarray, eps: float, rows: np.ndarray | None = None,
             want_scores: bool = False) -> dict:
    """Assign rows to generators.  Returns dict with C, f, alpha, cos, margin
    (and scores, nrows x k cosines, when ``want_scores``).  With ``rows`` only
    those rows are processed; outputs follow the order of ``rows``.  X may be
    a view with contiguous rows and a larger row stride."""
    X, ldx = _rows_view(X)
    gen_idx = np.ascontiguousarray(gen_idx, dtype=np.int32)
    n, d = X.shape
    k = gen_idx.size
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        m = rows.size
    else:
        m = n
    f = np.zeros(m, dtype=np.int32)
    alpha = np.zeros(m, dtype=np.float32)
    cos = np.zeros(m, dtype=np.float64)
    margin = np.zeros(m, dtype=np.float64)
    scores = np.zeros((m, k), dtype=np.float64) if want_scores else None
    rc = _load().orc_compress(_ptr(X), n, d, ldx, _dtype_code(X), _ptr(gen_idx), k, float(eps),
                              _ptr(rows), m, _ptr(f), _ptr(alpha), _ptr(cos), _ptr(margin), _ptr(scores))
    _check(rc, "compress")
    out = {"C": gather(X, gen_idx), "f": f, "alpha": alpha, "cos": cos, "margin": margin}
    if want_scores:
        out["scores"] = scores
    return out


def wgrad(C: np.ndarray, f: np.ndarray, alpha: np.ndarray, dY: np.ndarray,
          cols: np.ndarray | None = None) -> np.ndarray:
    """Approximate weight gradient dW = C^T B~ (d x d_out, or d x len(cols)), fp64.
    dY may be a view with contiguous rows and a larger row stride."""
    C = np.ascontiguousarray(C)
    dY, lddy = _rows_view(dY)
    if C.dtype != dY.dtype:
        raise TypeError("C and dY must share a dtype")
    f = np.ascontiguousarray(f, dtype=np.int32)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    k, d = C.shape
    n, d_out = dY.shape
    if cols is not None:
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        nc = cols.size
    else:
        nc = d_out
    dW = np.zeros((d, nc), dtype=np.float64)
    rc = _load().orc_wgrad(_ptr(C), _dtype_code(C), _ptr(f), _ptr(alpha), n, k, d, _ptr(dY), d_out, lddy,
                           _ptr(cols), nc, _ptr(dW))
    _check(rc, "wgrad")
    return dW


def decompress(C: np.ndarray, f: np.ndarray, alpha: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Return (exact fp64 reconstruction, reconstruction in C's dtype)."""
    C = np.ascontiguousarray(C)
    f = np.ascontiguousarray(f, dtype=np.int32)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    k, d = C.shape
    n = f.size
    x64 = np.zeros((n, d), dtype=np.float64)
    xt = np.zeros((n, d), dtype=C.dtype)
    _check(_load().orc_decompress(_ptr(C), _dtype_code(C), _ptr(f), _ptr(alpha), n, k, d, _ptr(x64), _ptr(xt)),
           "decompress")
    return x64, xt


def footprint_bytes(n: int, k: int, d: int, dtype: int) -> int:
    return int(_load().orc_footprint_bytes(n, k, d, dtype))


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
