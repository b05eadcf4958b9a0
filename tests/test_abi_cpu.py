"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* libpamm.so loads and exports every function include/pamm.h declares;
* the library's generator sampler and the oracle's (two independent
  implementations of the same published SplitMix64 + Floyd procedure) agree;
* invalid arguments are rejected with the documented status before anything
  is enqueued (these calls never reach the HIP runtime).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import activation_compression_pamm_amd as pamm
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pamm.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EUNSUP, EHIP, EVALUE, ETOOLARGE = range(10)
FAKE = 0x10000  # an aligned, never-dereferenced address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pamm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return pamm.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 11
    for name in names:
        assert hasattr(lib, name), name
        assert name in pamm._EXPORTS, f"binding does not wrap {name}"


def test_version_and_status_strings(lib):
    assert lib.pamm_abi_version() == 3
    for s in range(10):
        assert lib.pamm_status_string(s)
    assert lib.pamm_status_string(12345) == b"unknown status"


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (100, 100), (32768, 64), (131072, 256), (1000, 0), (2048, 1024),
                                 (64, 17), (65, 65), (2**31 - 1, 5)])  # bitmap word edges, the largest n
def test_sampler_matches_oracle(n, k):
    for seed in (0, 1, 2002, 2**63 + 5):
        lib_idx = pamm.sample_generators(n, k, seed).numpy()
        assert np.array_equal(lib_idx, orc.sample_generators(n, k, seed))


def test_sampler_errors(lib):
    out = (ctypes.c_int32 * 4)()
    assert lib.pamm_sample_generators(3, 4, 0, out) == ESHAPE
    assert lib.pamm_sample_generators(3, -1, 0, out) == ESHAPE
    assert lib.pamm_sample_generators(3, 2, 0, None) == ENULL
    assert lib.pamm_sample_generators(3, 0, 0, None) == OK


def test_workspace_sizes(lib):
    assert lib.pamm_compress_workspace_size(32768, 4096, 64, 1) == 0
    assert lib.pamm_compress_workspace_size(32768, 2048, 1024, 1) >= 12 * 4 * 32768 + 4 * 32768
    w = lib.pamm_wgrad_workspace_size(32768, 64, 4096, 12288, 1)
    # chunk partial rows (n/256 + k) x d_out fp32 dominate
    assert w >= (32768 // 256 + 64) * 12288 * 4
    assert w % 256 == 0
    # a small problem (n = 8192, 16 generators, 36 column slabs) is cut into
    # 64-row chunks so that its items fill the device: room for n/64 + k rows
    w = lib.pamm_wgrad_workspace_size(8192, 16, 768, 2304, 1)
    assert w >= (8192 // 64 + 16) * 2304 * 4
    assert w < (8192 // 32 + 16) * 2304 * 4
    # in between (n = 20000, 64 slabs): 128-row chunks
    w = lib.pamm_wgrad_workspace_size(20000, 16, 32, 4096, 1)
    assert (20000 // 128 + 16) * 4096 * 4 <= w < (20000 // 64 + 16) * 4096 * 4


def call_compress(lib, X=FAKE, n=64, d=32, ldx=32, dt=1, gen=FAKE, k=4, eps=0.1, C=FAKE, f=FAKE, a=FAKE,
                  ws=None, wsb=0):
    return lib.pamm_compress(X, n, d, ldx, dt, gen, k, eps, C, f, a, ws, wsb, None)


def test_compress_validation(lib):
    assert call_compress(lib, dt=7) == EDTYPE
    assert call_compress(lib, k=65) == ESHAPE
    assert call_compress(lib, k=-1) == ESHAPE
    assert call_compress(lib, ldx=31) == ESHAPE
    assert call_compress(lib, d=0, ldx=0) == ESHAPE
    assert call_compress(lib, n=10000, k=5000) == ESHAPE  # k above PAMM_MAX_K
    # a matrix spanning more than 2^40 elements
    assert call_compress(lib, n=1 << 21, ldx=1 << 20) == ESHAPE
    assert call_compress(lib, n=1, ldx=1 << 41) == ESHAPE
    assert call_compress(lib, eps=-0.5) == EVALUE
    assert call_compress(lib, eps=float("nan")) == EVALUE
    assert call_compress(lib, eps=float("inf")) == EVALUE
    assert call_compress(lib, X=None) == ENULL
    assert call_compress(lib, gen=None) == ENULL
    assert call_compress(lib, C=None) == ENULL
    assert call_compress(lib, f=None) == ENULL
    assert call_compress(lib, X=FAKE + 8) == EALIGN
    assert call_compress(lib, ldx=36) == EALIGN      # bf16 rows must start on 16 bytes
    assert call_compress(lib, dt=0, ldx=34) == EALIGN
    assert call_compress(lib, a=FAKE + 2) == EALIGN
    # k > 256 needs a workspace
    assert call_compress(lib, n=1024, k=300, ws=None, wsb=0) == EWS
    need = lib.pamm_compress_workspace_size(1024, 32, 300, 1)
    assert call_compress(lib, n=1024, k=300, ws=FAKE, wsb=need - 1) == EWS
    assert call_compress(lib, n=1024, k=300, ws=FAKE + 16, wsb=need) == EALIGN
    # n = 0 is a no-op
    assert call_compress(lib, n=0, k=0, X=None, gen=None, C=None, f=None, a=None) == OK


def call_wgrad(lib, C=FAKE, f=FAKE, a=FAKE, n=64, k=4, d=32, dY=FAKE, dout=48, lddy=48, dt=1, dW=FAKE, lddw=48,
               acc=0, tr=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.pamm_wgrad_workspace_size(n, k, d, dout, dt)
    return lib.pamm_wgrad(C, f, a, n, k, d, dY, dout, lddy, dt, dW, lddw, acc, tr, ws, wsb, None)


def test_wgrad_validation(lib):
    assert call_wgrad(lib, dt=2) == EDTYPE
    assert call_wgrad(lib, k=65) == ESHAPE
    assert call_wgrad(lib, lddy=40) == ESHAPE
    assert call_wgrad(lib, lddw=40) == ESHAPE
    assert call_wgrad(lib, dout=0, lddy=0, lddw=0) == ESHAPE
    assert call_wgrad(lib, n=1 << 21, lddy=1 << 20) == ESHAPE     # dY spans more than 2^40 elements
    assert call_wgrad(lib, d=1 << 21, lddw=1 << 20) == ESHAPE     # so does dW
    assert call_wgrad(lib, dW=None) == ENULL
    assert call_wgrad(lib, dY=None) == ENULL
    assert call_wgrad(lib, C=None) == ENULL
    assert call_wgrad(lib, dW=FAKE + 4) == EALIGN
    assert call_wgrad(lib, lddw=50) == EALIGN
    assert call_wgrad(lib, lddy=52) == EALIGN
    assert call_wgrad(lib, ws=None) == EWS
    assert call_wgrad(lib, wsb=1024) == EWS
    assert call_wgrad(lib, ws=FAKE + 64) == EALIGN
    # transposed output: dW^T [d_out x d] needs lddw >= d
    assert call_wgrad(lib, tr=1, d=64, lddw=48) == ESHAPE
    assert call_wgrad(lib, tr=1, d=32, lddw=30) == ESHAPE
    assert call_wgrad(lib, tr=1, d=32, lddw=34) == EALIGN


def test_wgrad_noalloc_validation(lib):
    # the no-allocation call checks every argument, then the size against its
    # fixed scratch array, before it looks up any device
    def call(C=FAKE, f=FAKE, a=FAKE, n=64, k=4, d=32, dY=FAKE, dout=48, lddy=48, dt=1, dW=FAKE, lddw=48, tr=0):
        return lib.pamm_wgrad_noalloc(C, f, a, n, k, d, dY, dout, lddy, dt, dW, lddw, 0, tr, None)
    assert call(dt=2) == EDTYPE
    assert call(k=65) == ESHAPE
    assert call(lddw=40) == ESHAPE
    assert call(dW=None) == ENULL
    assert call(dY=FAKE + 2) == EALIGN
    assert call(tr=1, d=64, lddw=48) == ESHAPE
    # 65536 tokens x 12288 outputs with 4096 generators needs ~274 MiB
    big = dict(n=65536, k=4096, d=4096, dout=12288, lddy=12288, lddw=12288)
    assert lib.pamm_wgrad_workspace_size(65536, 4096, 4096, 12288, 1) > pamm.NOALLOC_SCRATCH_BYTES
    assert call(**big) == ETOOLARGE
    assert lib.pamm_status_string(ETOOLARGE).startswith(b"the problem needs more memory")
    # the largest workloads of the benchmark configurations fit
    for n, k, d, dout in ((32768, 1024, 2048, 6144), (131072, 256, 4096, 6144), (32768, 64, 4096, 12288)):
        assert lib.pamm_wgrad_workspace_size(n, k, d, dout, 1) <= pamm.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PAMM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pamm.NOALLOC_SCRATCH_BYTES


def test_forward_compress_validation(lib):
    def call(X=FAKE, n=64, d=32, ldx=32, dt=1, W=FAKE, dout=48, ldw=32, bias=None, Y=FAKE, ldy=48, gen=FAKE, k=4,
             eps=0.1, C=FAKE, f=FAKE, a=FAKE, ws=FAKE, wsb=None):
        if wsb is None:
            wsb = lib.pamm_forward_compress_workspace_size(n, d, k, dt)
        return lib.pamm_forward_compress(X, n, d, ldx, dt, W, dout, ldw, bias, Y, ldy, gen, k, eps, C, f, a, ws, wsb,
                                         None)
    assert call(dt=4) == EDTYPE
    assert call(dt=0, ldx=32) == EUNSUP          # fp32 is not offered by the fused pass
    assert call(ldw=16) == ESHAPE
    assert call(ldy=40) == ESHAPE
    assert call(dout=0, ldy=0) == ESHAPE
    assert call(n=1 << 21, ldx=1 << 20, ldy=1 << 20) == ESHAPE     # X and Y span more than 2^40 elements
    assert call(k=65) == ESHAPE
    assert call(eps=-0.5) == EVALUE
    assert call(W=None) == ENULL
    assert call(Y=None) == ENULL
    assert call(W=FAKE + 8) == EALIGN
    assert call(ldw=36) == EALIGN
    assert call(Y=FAKE + 4) == EALIGN
    assert call(bias=FAKE + 1) == EALIGN
    assert call(ws=None) == EWS
    assert call(wsb=0) == EWS
    assert call(ws=FAKE + 32) == EALIGN
    # 32-bit addressing of X and W: a W spanning 4 GiB is refused
    assert call(dout=300000, ldw=8192, d=8192, ldx=8192, ldy=300000) == EUNSUP
    assert call(n=0, k=0, X=None, gen=None, C=None, f=None, a=None, Y=None, W=None) == OK
    assert lib.pamm_forward_compress_workspace_size(1024, 32, 300, 1) > lib.pamm_forward_compress_workspace_size(
        1024, 32, 200, 1) > 0


def test_decompress_validation(lib):
    def call(C=FAKE, f=FAKE, a=FAKE, n=64, k=4, d=32, dt=1, Xt=FAKE, ld=32):
        return lib.pamm_decompress(C, f, a, n, k, d, dt, Xt, ld, None)
    assert call(dt=3) == EDTYPE
    assert call(k=65) == ESHAPE
    assert call(ld=16) == ESHAPE
    assert call(n=1 << 21, ld=1 << 20) == ESHAPE
    assert call(Xt=None) == ENULL
    assert call(Xt=FAKE + 8) == EALIGN
    assert call(n=0, k=0, C=None, f=None, a=None, Xt=None) == OK


def test_binding_refuses_without_library(monkeypatch):
    monkeypatch.setattr(pamm, "_lib", None)
    monkeypatch.setattr(pamm, "_LIB_PATH", "/nonexistent/libpamm.so")
    with pytest.raises(RuntimeError, match="not built"):
        pamm.load_library()


def test_binding_checks_arrays_before_any_launch():
    # Every caller-supplied array is checked for shape, dtype and contiguity
    # before the device check and before the library is called: a short f or
    # alpha would otherwise be read or written past its end by the kernels.
    torch = pytest.importorskip("torch")
    n, d, k, dout = 8, 16, 2, 24
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    X = torch.zeros(n, d, dtype=bf)
    g = torch.zeros(k, dtype=i32)
    C = torch.zeros(k, d, dtype=bf)
    f = torch.zeros(n, dtype=i32)
    a = torch.zeros(n, dtype=f32)
    dY = torch.zeros(n, dout, dtype=bf)
    bad = [
        ("compress", lambda: pamm.compress(X, g, 0.0, f=torch.zeros(n - 1, dtype=i32)), ValueError, "f must have shape"),
        ("compress", lambda: pamm.compress(X, g, 0.0, alpha=torch.zeros(n + 1, dtype=f32)), ValueError, "alpha must"),
        ("compress", lambda: pamm.compress(X, g, 0.0, f=torch.zeros(n, dtype=torch.int64)), TypeError, "f must be"),
        ("compress", lambda: pamm.compress(X, g, 0.0, alpha=torch.zeros(n, dtype=bf)), TypeError, "alpha must be"),
        ("compress", lambda: pamm.compress(X, g, 0.0, C=torch.zeros(k, d + 1, dtype=bf)), ValueError, "C must have"),
        ("compress", lambda: pamm.compress(X, g, 0.0, C=torch.zeros(k, d, dtype=f32)), TypeError, "C must be"),
        ("compress", lambda: pamm.compress(X, g, 0.0, C=torch.zeros(d, k, dtype=bf).t()), ValueError, "contiguous"),
        ("compress", lambda: pamm.compress(X, g.view(1, k), 0.0), ValueError, "gen_idx must be 1-D"),
        ("compress", lambda: pamm.compress(X, g, 0.0, f=torch.zeros(2 * n, dtype=i32)[::2]), ValueError, "contiguous"),
        ("wgrad", lambda: pamm.wgrad(C, f[:-1], a, dY), ValueError, "f must have shape"),
        ("wgrad", lambda: pamm.wgrad(C, f, a[:-1], dY), ValueError, "alpha must have shape"),
        ("wgrad", lambda: pamm.wgrad(C, f.to(torch.int64), a, dY), TypeError, "f must be"),
        ("wgrad", lambda: pamm.wgrad(C, f, a.to(torch.float64), dY), TypeError, "alpha must be"),
        ("wgrad", lambda: pamm.wgrad(torch.zeros(d, k, dtype=bf).t(), f, a, dY), ValueError, "contiguous"),
        ("wgrad", lambda: pamm.wgrad(C.view(-1), f, a, dY), ValueError, "C must be 2-D"),
        ("wgrad", lambda: pamm.wgrad(C.float(), f, a, dY), TypeError, "share a dtype"),
        ("wgrad", lambda: pamm.wgrad(C, f, a, dY, dW=torch.zeros(d, dout + 1)), ValueError, "dW must be"),
        ("wgrad", lambda: pamm.wgrad(C, f, a, dY, dW=torch.zeros(d, dout, dtype=torch.float64)), ValueError,
         "dW must be"),
        ("decompress", lambda: pamm.decompress(C, f, a[:-1]), ValueError, "alpha must have shape"),
        ("decompress", lambda: pamm.decompress(C, f.to(torch.int64), a), TypeError, "f must be"),
        ("decompress", lambda: pamm.decompress(torch.zeros(d, k, dtype=bf).t(), f, a), ValueError, "contiguous"),
        ("decompress", lambda: pamm.decompress(C, f.view(2, -1), a), ValueError, "f must be 1-D"),
        ("decompress", lambda: pamm.decompress(C, f, a, out=torch.zeros(n, d, dtype=f32)), ValueError, "out must be"),
    ]
    for where, call, exc, msg in bad:
        with pytest.raises(exc, match=msg):
            call()
    # well-formed host arrays pass these checks and stop at the device check
    for call in (lambda: pamm.compress(X, g, 0.0, C=C, f=f, alpha=a),
                 lambda: pamm.wgrad(C, f, a, dY),
                 lambda: pamm.decompress(C, f, a)):
        with pytest.raises(ValueError, match="must be on the GPU"):
            call()
