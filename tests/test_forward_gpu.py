"""GPU: the projection and the compression in one pass (pamm_forward_compress)
through the C ABI.  Y against an fp64 product of the same bf16 inputs within
the bf16 rounding plus the fp32 accumulation bound; (C, f, alpha) against the
oracle under the parity rules of the other compress tests."""
import sys

import numpy as np
import pytest
import torch

import activation_compression_pamm_amd as pamm
from activation_compression_pamm_amd import synth
from oracle import oracle as orc

from gpu_util import ORACLE_THREADS, U, check_compress, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check_y(X, W, b, Y_g, rows):
    """|Y - (X W^T + b)| <= 2^-8 |y| + 2 gamma_d sum|x w| + 2u|y|: the bf16
    rounding (8 significant bits, unit roundoff 2^-8) of an fp32 sum of exact
    bf16 products (Higham, Accuracy and Stability, section 3.1) plus the fp32
    bias addition."""
    d = X.shape[1]
    g = d * U / (1 - d * U)
    Xr = orc.to_f64(X[rows])
    Wf = orc.to_f64(W)
    ref = Xr @ Wf.T
    if b is not None:
        ref = ref + orc.to_f64(b)[None, :]
    absum = np.abs(Xr) @ np.abs(Wf).T
    got = orc.to_f64(Y_g[rows])
    lim = 2.0 ** -8 * np.abs(ref) + 2 * g * absum + 2 * U * np.abs(ref) + 1e-37
    bad = np.abs(got - ref) > lim
    assert not bad.any(), f"{bad.sum()} Y entries off, e.g. {np.argwhere(bad)[0]}"
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))


def run_case(n, d, d_out, k, eps, bias=True, seed=0, ldx=None, ldw=None, rows=None):
    say("forward", f"n={n} d={d} d_out={d_out} k={k} eps={eps} bias={bias} ldx={ldx} ldw={ldw}")
    ldx = ldx or d
    ldw = ldw or d
    Xbig = synth.clustered_activations(n, ldx, max(2, min(64, k or 2)), seed=seed + 1, dtype="bf16")
    Wbig = synth.random_matrix(d_out, ldw, seed + 2, "bf16")
    X = np.ascontiguousarray(Xbig[:, :d])
    W = np.ascontiguousarray(Wbig[:, :d])
    b = synth.random_matrix(1, d_out, seed + 3, "bf16")[0] if bias else None
    g = pamm.sample_generators(n, k, seed + 4).numpy()
    Y, C, f, a = pamm.forward_compress(to_dev(Xbig)[:, :d], to_dev(Wbig)[:, :d], torch.from_numpy(g).cuda(), eps,
                                       bias=None if b is None else to_dev(b))
    torch.cuda.synchronize()
    Y_g = to_host(Y)
    rows = np.arange(n) if rows is None else rows
    err = check_y(X, W, b, Y_g, rows)
    stats = check_compress(X, g, eps, to_host(C), to_host(f), to_host(a))
    say("forward", "ok", stats, f"Y max rel {err:.2e}")
    return Y, C, f, a


@pytest.mark.parametrize("n,d,d_out,k,eps,bias", [
    (3000, 200, 296, 24, 0.1, True),     # ragged rows, tail stage, partial Y tile, narrow generator tile
    (2048, 256, 768, 16, 0.1, False),    # no bias
    (4096, 128, 512, 256, 0.0, True),    # one full generator tile
    (2600, 136, 264, 300, 0.05, True),   # two generator tiles and the merge; odd stage count
    (1000, 64, 8, 5, 0.2, True),         # one stage, a single 8-column Y tile
    (777, 72, 1000, 1, 0.0, True),       # one generator; a partial last Y tile of 232 columns
])
def test_forward_compress_shapes(n, d, d_out, k, eps, bias):
    run_case(n, d, d_out, k, eps, bias=bias)


def test_forward_compress_strided_and_no_generators():
    run_case(1500, 120, 392, 40, 0.1, ldx=144, ldw=128)
    say("forward", "k=0")
    n, d, d_out = 500, 64, 128
    X = synth.clustered_activations(n, d, 4, seed=9, dtype="bf16")
    W = synth.random_matrix(d_out, d, 10, "bf16")
    Y, C, f, a = pamm.forward_compress(to_dev(X), to_dev(W), torch.zeros(0, dtype=torch.int32).cuda(), 0.0)
    torch.cuda.synchronize()
    assert np.all(to_host(f) == -1) and np.all(to_host(a) == 0)
    check_y(X, W, None, to_host(Y), np.arange(n))


def test_forward_compress_llama7b_shape():
    # the 7B QKV projection: every row of (f, alpha), Y on 512 sampled rows
    X, dY, p = synth.make_config("llama7b_qkv")
    del dY
    n, d, d_out, k, eps = p["n"], p["d"], p["d_out"], p["k"], p["eps"]
    say("forward-7B", f"n={n} d={d} d_out={d_out} k={k} ({ORACLE_THREADS} oracle threads)")
    W = synth.random_matrix(d_out, d, 77, "bf16")
    b = synth.random_matrix(1, d_out, 78, "bf16")[0]
    g = pamm.sample_generators(n, k, synth.generator_seed("llama7b_qkv")).numpy()
    Y, C, f, a = pamm.forward_compress(to_dev(X), to_dev(W), torch.from_numpy(g).cuda(), eps, bias=to_dev(b))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(5).choice(n, 510, replace=False)]))
    err = check_y(X, W, b, to_host(Y), rows)
    stats = check_compress(X, g, eps, to_host(C), to_host(f), to_host(a))
    # the same compression as pamm_compress up to in-band choices
    C2, f2, a2 = pamm.compress(to_dev(X), torch.from_numpy(g).cuda(), eps)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    agree = (to_host(f) == to_host(f2)).mean()
    assert agree > 0.9999, agree
    say("forward-7B", "ok", stats, f"Y max rel {err:.2e}", f"index agreement with pamm_compress {agree:.6f}")
