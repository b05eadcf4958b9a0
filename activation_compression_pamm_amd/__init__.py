"""PAMM (Point-Approximate Matrix Multiplication) for AMD Instinct MI355X.

Thin Python binding over the C ABI of ``libpamm.so`` (see ``include/pamm.h``).
It only marshals arguments: PyTorch supplies device memory and the current
HIP stream, and every step of the computation runs in the library's HIP
kernels.  There is no CPU fallback; if the library is missing the calls
raise.

Method: "QKV Projections Require a Fraction of Their Memory", section 2
"Metodologia", sub-part "Algoritmo in Due Fasi" -- compress the saved inputs
X of a QKV projection into generator rows C plus an (index, scale) pair per
token, then approximate the weight gradient C^T B~ from that compressed form.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PammError", "F32", "BF16", "MAX_K", "load_library", "library_path", "abi_version",
    "sample_generators", "compress", "forward_compress", "wgrad", "wgrad_noalloc", "decompress",
    "NOALLOC_SCRATCH_BYTES", "forward_compress_workspace_size",
    "compress_workspace_size", "wgrad_workspace_size", "compressed_nbytes",
]

F32 = 0
BF16 = 1
MAX_K = 4096
# size of the fixed device array pamm_wgrad_noalloc uses as its workspace
NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpamm.so")
_lib = None

_EXPORTS = {
    # name: (restype, argtypes)
    "pamm_abi_version": (ctypes.c_int, []),
    "pamm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pamm_sample_generators": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p]),
    "pamm_compress_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "pamm_compress": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]),
    "pamm_wgrad_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                    ctypes.c_int]),
    "pamm_wgrad": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]),
    "pamm_wgrad_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]),
    "pamm_forward_compress_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                               ctypes.c_int]),
    "pamm_forward_compress": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pamm_decompress": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]),
}


class PammError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load_library().pamm_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libpamm.so (built by ``activation_compression_pamm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"PAMM HIP library not built: {_LIB_PATH} is missing "
                               "(run `python -m activation_compression_pamm_amd.build`)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def abi_version() -> int:
    return load_library().pamm_abi_version()


def _check(status: int, where: str):
    if status != 0:
        raise PammError(status, where)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"PAMM supports float32 and bfloat16 tensors, got {t.dtype}")


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return t.shape[0], t.shape[1], t.stride(0)


def _empty_rows(rows, cols, dtype, device):
    """An uninitialised [rows x cols] tensor whose rows start a multiple of
    16 bytes apart, as the C ABI's leading-dimension rule asks: a view of a
    buffer with padded rows when cols elements do not fill whole 16 bytes."""
    torch = _torch()
    per = 16 // torch.empty(0, dtype=dtype).element_size()
    ld = (cols + per - 1) // per * per
    buf = torch.empty((rows, ld), dtype=dtype, device=device)
    return buf if ld == cols else buf[:, :cols]


def _on_gpu(where, **tensors):
    """Every tensor argument must live on one GPU: the kernels read and write
    them in place."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{where}: {name} must be on the GPU, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{where}: {name} is on {t.device}, expected {dev}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def sample_generators(n: int, k: int, seed: int, *, pin: bool = False):
    """k distinct row ids of [0, n), ascending, drawn on the host (int32 CPU
    tensor; in page-locked memory with ``pin``, so that its upload can be
    asynchronous)."""
    torch = _torch()
    out = torch.empty(max(k, 0), dtype=torch.int32, pin_memory=pin)
    _check(load_library().pamm_sample_generators(n, k, seed & (2**64 - 1), _ptr(out)), "pamm_sample_generators")
    return out


def compress_workspace_size(n: int, d: int, k: int, dtype: int) -> int:
    return int(load_library().pamm_compress_workspace_size(n, d, k, dtype))


def wgrad_workspace_size(n: int, k: int, d: int, d_out: int, dtype: int) -> int:
    return int(load_library().pamm_wgrad_workspace_size(n, k, d, d_out, dtype))


def compressed_nbytes(n: int, k: int, d: int, dtype: int) -> int:
    """Bytes of the saved triple (C, f, alpha)."""
    return k * d * (2 if dtype == BF16 else 4) + 8 * n


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _need(where, name, t, shape, dtype):
    """A caller-supplied tensor must have exactly this shape and dtype and be
    contiguous: the kernels read and write it as a dense array."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{where}: {name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{where}: {name} must be contiguous")


def _check_triple(where, C, f, alpha, n, k, d, dtype):
    torch = _torch()
    if C is not None:
        _need(where, "C", C, (k, d), dtype)
    if f is not None:
        _need(where, "f", f, (n,), torch.int32)
    if alpha is not None:
        _need(where, "alpha", alpha, (n,), torch.float32)


def _check_workspace(where, workspace):
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError(f"{where}: workspace must be contiguous")


def compress(X, gen_idx, eps: float, *, C=None, f=None, alpha=None, workspace=None, stream=None):
    """Compress activations X [n x d] (CUDA/HIP tensor, bf16 or fp32).

    gen_idx: int32 device tensor of k generator row ids (see sample_generators).
    Returns (C [k x d], f [n] int32, alpha [n] fp32)."""
    torch = _torch()
    n, d, ldx = _rows(X, "X")
    dt = _dtype_code(X)
    if gen_idx.dim() != 1:
        raise ValueError(f"compress: gen_idx must be 1-D, got shape {tuple(gen_idx.shape)}")
    k = gen_idx.numel()
    _check_triple("compress", C, f, alpha, n, k, d, X.dtype)
    _check_workspace("compress", workspace)
    _on_gpu("compress", X=X, C=C, f=f, alpha=alpha, workspace=workspace)
    gen_idx = gen_idx.to(device=X.device, dtype=torch.int32).contiguous()
    if C is None:
        C = torch.empty((k, d), dtype=X.dtype, device=X.device)
    if f is None:
        f = torch.empty(n, dtype=torch.int32, device=X.device)
    if alpha is None:
        alpha = torch.empty(n, dtype=torch.float32, device=X.device)
    ws = _workspace(compress_workspace_size(n, d, k, dt), X.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().pamm_compress(_ptr(X), n, d, ldx, dt, _ptr(gen_idx), k, float(eps), _ptr(C), _ptr(f),
                                      _ptr(alpha), _ptr(ws), nbytes, _stream_ptr(stream))
    _check(st, "pamm_compress")
    return C, f, alpha


def forward_compress_workspace_size(n: int, d: int, k: int, dtype: int = BF16) -> int:
    return int(load_library().pamm_forward_compress_workspace_size(n, d, k, dtype))


def forward_compress(X, W, gen_idx, eps: float, *, bias=None, Y=None, C=None, f=None, alpha=None, workspace=None,
                     stream=None):
    """The projection Y = X W^T (+ bias) and the compression of X in one pass
    over X (bf16 only).  X [n x d], W [d_out x d] (the layout of a linear
    layer's weight), bias [d_out] or None, gen_idx int32 [k] on the device.
    Returns (Y [n x d_out] bf16, C [k x d], f [n] int32, alpha [n] fp32).
    A Y allocated here has its rows padded to a multiple of 16 bytes (the
    returned tensor is a view of the exact shape)."""
    torch = _torch()
    n, d, ldx = _rows(X, "X")
    dt = _dtype_code(X)
    d_out, dw, ldw = _rows(W, "W")
    if dw != d:
        raise ValueError(f"forward_compress: W must be [d_out x {d}], got {tuple(W.shape)}")
    if W.dtype != X.dtype:
        raise TypeError("forward_compress: X and W must share a dtype")
    if bias is not None:
        _need("forward_compress", "bias", bias, (d_out,), X.dtype)
    if gen_idx.dim() != 1:
        raise ValueError(f"forward_compress: gen_idx must be 1-D, got shape {tuple(gen_idx.shape)}")
    k = gen_idx.numel()
    _check_triple("forward_compress", C, f, alpha, n, k, d, X.dtype)
    _check_workspace("forward_compress", workspace)
    if Y is not None and (tuple(Y.shape) != (n, d_out) or Y.dtype != X.dtype):
        raise ValueError(f"Y must be {X.dtype} of shape {(n, d_out)}, got {tuple(Y.shape)} {Y.dtype}")
    _on_gpu("forward_compress", X=X, W=W, bias=bias, Y=Y, C=C, f=f, alpha=alpha, workspace=workspace)
    gen_idx = gen_idx.to(device=X.device, dtype=torch.int32).contiguous()
    if Y is None:
        Y = _empty_rows(n, d_out, X.dtype, X.device)
    _, _, ldy = _rows(Y, "Y")
    if C is None:
        C = torch.empty((k, d), dtype=X.dtype, device=X.device)
    if f is None:
        f = torch.empty(n, dtype=torch.int32, device=X.device)
    if alpha is None:
        alpha = torch.empty(n, dtype=torch.float32, device=X.device)
    ws = _workspace(forward_compress_workspace_size(n, d, k, dt), X.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().pamm_forward_compress(_ptr(X), n, d, ldx, dt, _ptr(W), d_out, ldw, _ptr(bias), _ptr(Y), ldy,
                                              _ptr(gen_idx), k, float(eps), _ptr(C), _ptr(f), _ptr(alpha), _ptr(ws),
                                              nbytes, _stream_ptr(stream))
    _check(st, "pamm_forward_compress")
    return Y, C, f, alpha


def wgrad(C, f, alpha, dY, *, dW=None, accumulate: bool = False, transpose_out: bool = False, workspace=None,
          stream=None):
    """Approximate weight gradient dW = C^T B~ [d x d_out] (fp32) from the
    compressed triple and the output gradient dY [n x d_out].  With
    transpose_out the result is dW^T [d_out x d], the layout of the weight
    gradient of a layer Y = X W^T.  A dW allocated here has its rows padded
    to a multiple of 16 bytes (the returned tensor is a view of the exact
    shape)."""
    torch = _torch()
    n, d_out, lddy = _rows(dY, "dY")
    dt = _dtype_code(dY)
    if C.dim() != 2:
        raise ValueError(f"wgrad: C must be 2-D [k x d], got shape {tuple(C.shape)}")
    if C.dtype != dY.dtype:
        raise TypeError("C and dY must share a dtype")
    k, d = C.shape
    _check_triple("wgrad", C, f, alpha, n, k, d, dY.dtype)
    _check_workspace("wgrad", workspace)
    shape = (d_out, d) if transpose_out else (d, d_out)
    if dW is not None and (tuple(dW.shape) != shape or dW.dtype != torch.float32):
        raise ValueError(f"dW must be float32 of shape {shape}, got {tuple(dW.shape)} {dW.dtype}")
    _on_gpu("wgrad", C=C, f=f, alpha=alpha, dY=dY, dW=dW, workspace=workspace)
    if dW is None:
        dW = _empty_rows(shape[0], shape[1], torch.float32, dY.device)
    _, _, lddw = _rows(dW, "dW")
    ws = _workspace(wgrad_workspace_size(n, k, d, d_out, dt), dY.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().pamm_wgrad(_ptr(C), _ptr(f), _ptr(alpha), n, k, d, _ptr(dY), d_out, lddy, dt, _ptr(dW), lddw,
                                   1 if accumulate else 0, 1 if transpose_out else 0, _ptr(ws), nbytes,
                                   _stream_ptr(stream))
    _check(st, "pamm_wgrad")
    return dW


def wgrad_noalloc(C, f, alpha, dY, dW, *, accumulate: bool = False, transpose_out: bool = False, stream=None):
    """wgrad through pamm_wgrad_noalloc: the library uses its fixed per-GPU
    scratch array instead of a workspace and allocates nothing.  dW (fp32,
    [d x d_out], or [d_out x d] with transpose_out) is supplied by the
    caller.  Calls that may overlap on one GPU race on the shared array."""
    torch = _torch()
    n, d_out, lddy = _rows(dY, "dY")
    dt = _dtype_code(dY)
    if C.dim() != 2:
        raise ValueError(f"wgrad_noalloc: C must be 2-D [k x d], got shape {tuple(C.shape)}")
    if C.dtype != dY.dtype:
        raise TypeError("C and dY must share a dtype")
    k, d = C.shape
    _check_triple("wgrad_noalloc", C, f, alpha, n, k, d, dY.dtype)
    shape = (d_out, d) if transpose_out else (d, d_out)
    if tuple(dW.shape) != shape or dW.dtype != torch.float32:
        raise ValueError(f"dW must be float32 of shape {shape}, got {tuple(dW.shape)} {dW.dtype}")
    _on_gpu("wgrad_noalloc", C=C, f=f, alpha=alpha, dY=dY, dW=dW)
    _, _, lddw = _rows(dW, "dW")
    st = load_library().pamm_wgrad_noalloc(_ptr(C), _ptr(f), _ptr(alpha), n, k, d, _ptr(dY), d_out, lddy, dt,
                                           _ptr(dW), lddw, 1 if accumulate else 0, 1 if transpose_out else 0,
                                           _stream_ptr(stream))
    _check(st, "pamm_wgrad_noalloc")
    return dW


def decompress(C, f, alpha, *, out=None, stream=None):
    """Reconstruction X~_i = alpha_i C_f(i) (zero rows where f = -1).  An out
    allocated here has its rows padded to a multiple of 16 bytes (the returned
    tensor is a view of the exact shape)."""
    torch = _torch()
    if C.dim() != 2:
        raise ValueError(f"decompress: C must be 2-D [k x d], got shape {tuple(C.shape)}")
    k, d = C.shape
    if f.dim() != 1:
        raise ValueError(f"decompress: f must be 1-D, got shape {tuple(f.shape)}")
    n = f.numel()
    dt = _dtype_code(C)
    _check_triple("decompress", C, f, alpha, n, k, d, C.dtype)
    if out is not None and (tuple(out.shape) != (n, d) or out.dtype != C.dtype):
        raise ValueError(f"out must be {C.dtype} of shape {(n, d)}, got {tuple(out.shape)} {out.dtype}")
    _on_gpu("decompress", C=C, f=f, alpha=alpha, out=out)
    if out is None:
        out = _empty_rows(n, d, C.dtype, f.device)
    _, _, ldxt = _rows(out, "out")
    st = load_library().pamm_decompress(_ptr(C), _ptr(f), _ptr(alpha), n, k, d, dt, _ptr(out), ldxt,
                                        _stream_ptr(stream))
    _check(st, "pamm_decompress")
    return out
