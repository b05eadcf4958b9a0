"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Each case prints its name, shapes and seeds before touching the GPU.  Every
case compares every output, the full-size workloads included (the oracle's
row and column chunks run on a pool of host threads).
"""
import sys
import time

import numpy as np
import pytest
import torch

import activation_compression_pamm_amd as pamm
from activation_compression_pamm_amd import synth
from oracle import oracle as orc

from gpu_util import ORACLE_THREADS, TIGHT, TOL, check_compress, check_wgrad, oracle_wgrad, rel, run_gpu, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def full_case(X, dY, gen_idx, eps, label):
    n, d = X.shape
    say(label, f"n={n} d={d} d_out={dY.shape[1]} k={gen_idx.size} eps={eps} dtype={X.dtype}")
    out = run_gpu(X, dY, gen_idx, eps)
    C_g, f_g, a_g = to_host(out["C"]), to_host(out["f"]), to_host(out["alpha"])
    stats = check_compress(X, gen_idx, eps, C_g, f_g, a_g)
    e_iso = check_wgrad(C_g, f_g, a_g, dY, to_host(out["dW"]))
    # end to end: oracle compress + oracle wgrad, independent of the GPU
    r = orc.compress(X, gen_idx, eps)
    dW_o = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    e_e2e = rel(to_host(out["dW"]), dW_o)
    dt = "bf16" if X.dtype == np.uint16 else "f32"
    if stats["inband_mismatches"] == 0:
        # with identical indices the end-to-end result must meet the tolerance;
        # an in-band flip legitimately moves a whole row to another generator
        assert e_e2e <= TOL[dt], f"end-to-end dW error {e_e2e}"
    # reconstruction: bit-exact against the oracle fed the GPU's triple
    xt = to_host(pamm.decompress(out["C"], out["f"], out["alpha"]))
    _, xt_o = orc.decompress(C_g, f_g, a_g)
    assert np.array_equal(xt, xt_o)
    say(label, "ok", stats, f"dW iso {e_iso:.2e} e2e {e_e2e:.2e}")
    return out, stats


# --------------------------------------------------------------------------
# the small workloads, every output compared
# --------------------------------------------------------------------------

def test_tiny_fp32_config():
    X, dY, p = synth.make_config("tiny_fp32")
    g = pamm.sample_generators(p["n"], p["k"], synth.generator_seed("tiny_fp32")).numpy()
    full_case(X, dY, g, p["eps"], "tiny_fp32")


def test_gpt2_small_qkv_config():
    X, dY, p = synth.make_config("gpt2_small_qkv")
    g = pamm.sample_generators(p["n"], p["k"], synth.generator_seed("gpt2_small_qkv")).numpy()
    full_case(X, dY, g, p["eps"], "gpt2_small_qkv")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,d,dout,k,eps", [
    (1000, 200, 296, 24, 0.1),     # ragged rows, columns, outputs and generator tile
    (777, 72, 136, 5, 0.0),
    (2500, 384, 520, 64, 0.3),
    (1536, 256, 256, 128, 0.1),
    (1100, 136, 264, 256, 0.05),   # one full 256-generator tile
    (2048, 256, 384, 300, 0.1),    # two generator tiles + merge
    (3000, 128, 200, 1024, 0.1),   # four tiles, many small segments
])
def test_ragged_shapes(dtype, n, d, dout, k, eps):
    X = synth.clustered_activations(n, d, max(4, k // 2), seed=n + d, dtype=dtype)
    dY = synth.gradients(n, dout, seed=n + dout, dtype=dtype)
    g = pamm.sample_generators(n, k, seed=k + 7).numpy()
    full_case(X, dY, g, eps, f"ragged-{dtype}")


def test_long_segments_split_into_chunks():
    # one generator collects thousands of rows: its row list is cut into
    # several chunks whose partial sums the generator product adds up
    n, d, dout = 6000, 128, 192
    X = synth.clustered_activations(n, d, 2, seed=3, dtype="bf16")
    dY = synth.gradients(n, dout, seed=4, dtype="bf16")
    g = np.array([0, 1, 2], dtype=np.int32)
    full_case(X, dY, g, 0.0, "long-segments")


@pytest.mark.parametrize("n,d,dout,k", [
    (65536, 32, 64, 1024),   # 64 sort blocks, 1024 generators: histogram prefixed once
    (65537, 32, 64, 40),     # a last sort block of one row
    (6000, 64, 96, 4096),    # the largest k (LDS beyond 64 KB in the sort)
    (300000, 16, 16, 16),    # 293 sort blocks summing a small histogram
    (20000, 32, 4096, 16),   # 128-row chunks (the layout halves 256 once)
])
def test_sort_block_edges_and_largest_k(n, d, dout, k):
    X = synth.clustered_activations(n, d, 64, seed=n + k, dtype="bf16")
    dY = synth.gradients(n, dout, seed=n + dout, dtype="bf16")
    g = pamm.sample_generators(n, k, seed=k + 3).numpy()
    full_case(X, dY, g, 0.05, "sort-path")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k", [33, 64, 100])
def test_full_row_blocks_with_a_ragged_stage(dtype, k):
    # enough rows for the 8-wave small-k compress (a 128-row block per
    # compute unit) and a row length that ends in a partial stage, which
    # the rotated stage order places in the middle of most workgroups' walks
    n, d, dout = 40000, 200, 96
    X = synth.clustered_activations(n, d, 48, seed=n + k, dtype=dtype)
    dY = synth.gradients(n, dout, seed=n + dout + k, dtype=dtype)
    g = pamm.sample_generators(n, k, seed=k + 5).numpy()
    full_case(X, dY, g, 0.1, f"ragged-stage-{dtype}")


@pytest.mark.parametrize("n,d,dout,k,dtype", [
    (20000, 64, 1024, 512, "f32"),
    (30001, 72, 1544, 300, "bf16"),   # ragged rows and output columns
])
def test_paired_reduction_items(n, d, dout, k, dtype):
    # full-length (256-row) chunks with few rows per generator: each
    # reduction item walks two chunks, one per half of the wave's row groups
    X = synth.clustered_activations(n, d, k // 2, seed=n + k, dtype=dtype)
    dY = synth.gradients(n, dout, seed=n + dout, dtype=dtype)
    g = pamm.sample_generators(n, k, seed=k + 11).numpy()
    full_case(X, dY, g, 0.1, f"paired-{dtype}")


def _random_case(i):
    # shapes, generator counts and thresholds drawn from one seeded stream;
    # row lengths a multiple of 16 bytes (the ABI's leading-dimension rule)
    rng = np.random.default_rng(9000 + i)
    dtype = "bf16" if i % 3 else "f32"
    per = 8 if dtype == "bf16" else 4
    n = int(rng.integers(1, 5000))
    d = per * int(rng.integers(1, 512 // per + 1))
    dout = per * int(rng.integers(1, 640 // per + 1))
    k = int(rng.integers(1, min(n, 600) + 1))
    eps = float(rng.choice([0.0, 0.05, 0.2, 0.5]))
    return dtype, n, d, dout, k, eps


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(i):
    dtype, n, d, dout, k, eps = _random_case(i)
    X = synth.clustered_activations(n, d, max(2, min(64, k)), seed=100 + i, dtype=dtype)
    dY = synth.gradients(n, dout, seed=200 + i, dtype=dtype)
    g = pamm.sample_generators(n, k, seed=300 + i).numpy()
    full_case(X, dY, g, eps, f"random-{i}")


# --------------------------------------------------------------------------
# degenerate cases the method has
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_k_equals_n_gives_exact_product(dtype):
    n, d, dout = 512, 64, 96
    X = synth.random_matrix(n, d, 11, dtype)
    dY = synth.random_matrix(n, dout, 12, dtype)
    g = np.arange(n, dtype=np.int32)
    say("k=n", dtype)
    out = run_gpu(X, dY, g, 0.0)
    f_g, a_g = to_host(out["f"]), to_host(out["alpha"])
    assert np.array_equal(f_g, np.arange(n))
    assert np.all(a_g == 1.0)   # |c|^2 uses the same MFMA arithmetic as the dot products
    exact = orc.to_f64(X).T @ orc.to_f64(dY)
    e = rel(to_host(out["dW"]), exact)
    assert e <= (1e-4 if dtype == "bf16" else 1e-5), e


# bf16 with 128- or 256-generator tiles and at least one (row block, tile)
# pair per compute unit: the GEMM-shaped compress kernel.  Ragged rows, a tail stage,
# a padding stage position, a partial last tile and a strided view.
GEMM_CASES = [
    (65573, 136, 136, 256, 0.05),   # ragged n; tail stage of 8; odd stage count
    (33000, 200, 200, 300, 0.1),    # two tiles, the last one 44 generators
    (65536, 64, 64, 256, 0.0),      # a single stage (and one padding position)
    (32768, 256, 256, 512, 0.0),    # two full tiles
    (65536, 120, 144, 256, 0.1),    # strided view: ldx > d
    # 128-row blocks (the 256-row blocks would leave compute units idle)
    (32845, 136, 136, 256, 0.05),   # ragged n; tail stage; odd stage count
    (20000, 200, 200, 300, 0.1),    # two tiles, the last one 44 generators
    (32768, 128, 128, 256, 0.0),    # no tail, even stage count
    (32768, 120, 144, 256, 0.1),    # strided view
    # 64 < k <= 128 at the same sizes (the 128-row kernel)
    (32868, 136, 136, 128, 0.05),   # ragged n; tail stage; odd stage count
    (32768, 128, 128, 100, 0.1),    # a partial tile of 100 generators; no tail
    (32768, 120, 144, 96, 0.0),     # strided view
]


@pytest.mark.parametrize("n,d,ldx,k,eps", GEMM_CASES)
def test_gemm_tiles(n, d, ldx, k, eps):
    Xbig = synth.clustered_activations(n, ldx, 64, seed=61 + d, dtype="bf16")
    X = np.ascontiguousarray(Xbig[:, :d])
    g = pamm.sample_generators(n, k, 62).numpy()
    say("gemm-tiles", f"n={n} d={d} ldx={ldx} k={k} eps={eps}")
    C, f, a = pamm.compress(to_dev(Xbig)[:, :d], torch.from_numpy(g).cuda(), eps)
    torch.cuda.synchronize()
    C_g, f_g, a_g = to_host(C), to_host(f), to_host(a)
    stats = check_compress(X, g, eps, C_g, f_g, a_g)
    # a generator's own row: itself (unless a duplicate row ties lower), alpha
    # 1 to a few ulps (|c|^2 from fp32 dot2 sums, the dot from the MFMA)
    own = f_g[g]
    mine = own == np.arange(k)
    assert np.all(own <= np.arange(k)) and np.mean(mine) > 0.99
    assert np.all(np.abs(a_g[g][mine] - 1.0) <= 1e-5), np.abs(a_g[g][mine] - 1.0).max()
    say("gemm-tiles", "ok", stats)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scaled_copies_and_self_rows_exact(dtype):
    n, d = 700, 96
    X32 = synth.bf16_bits_to_f32(synth.random_matrix(n, d, 21, "bf16")) if dtype == "bf16" else \
        synth.random_matrix(n, d, 21, "f32").copy()
    g = np.array([3, 50, 99, 400, 650], dtype=np.int32)
    plan = {10: (0, 2.0), 11: (1, -4.0), 12: (2, 0.5), 13: (3, -0.25), 600: (4, 8.0), 699: (0, -1.0)}
    for row, (j, s) in plan.items():
        X32[row] = np.float32(s) * X32[g[j]]
    X = synth.f32_to_bf16_bits(X32) if dtype == "bf16" else X32
    say("scaled-copies", dtype)
    out = run_gpu(X, None, g, 0.0)
    f_g, a_g = to_host(out["f"]), to_host(out["alpha"])
    for row, (j, s) in plan.items():
        assert f_g[row] == j and a_g[row] == s, (row, f_g[row], a_g[row])
    assert np.array_equal(f_g[g], np.arange(5)) and np.all(a_g[g] == 1.0)
    xt = to_host(pamm.decompress(out["C"], out["f"], out["alpha"]))
    for row in list(plan) + list(g):
        assert np.array_equal(xt[row], X[row])


def test_duplicate_generators_and_zero_and_nan_rows():
    n, d, dout = 300, 64, 80
    X = synth.random_matrix(n, d, 31, "f32").copy()
    X[40] = X[7]            # duplicate rows, both generators
    X[41] = 4 * X[7]        # collinear with both
    X[100] = 0.0            # zero generator
    X[101] = 0.0            # zero row
    X[102, 5] = np.nan      # NaN row
    g = np.array([7, 40, 100, 200], dtype=np.int32)
    dY = synth.random_matrix(n, dout, 32, "f32")
    for eps in (0.0, 0.2):
        say("degenerate", eps)
        out = run_gpu(X, dY, g, eps)
        f_g, a_g = to_host(out["f"]), to_host(out["alpha"])
        assert f_g[7] == 0 and f_g[40] == 0 and f_g[41] == 0 and a_g[41] == 4.0
        assert f_g[102] == -1 and a_g[102] == 0.0
        if eps == 0.0:
            assert f_g[101] == 0 and a_g[101] == 0.0
        else:
            assert f_g[101] == -1 and f_g[100] == -1
        assert not np.any(f_g == 2)   # the zero generator never wins a nonzero row
        check_compress(X, g, eps, to_host(out["C"]), f_g, a_g)
        check_wgrad(to_host(out["C"]), f_g, a_g, dY, to_host(out["dW"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_infinite_generator_never_wins(dtype):
    # A generator holding +inf scores NaN (inf / inf) against every row, so it
    # never wins; the row itself has a NaN cosine and is dropped.  Checked with
    # that generator in the first slot and in a middle one (small-k kernel).
    n, d = 300, 64
    X32 = synth.random_matrix(n, d, 37, "f32").copy()
    X32[150, 3] = np.inf
    X = synth.f32_to_bf16_bits(X32) if dtype == "bf16" else X32
    finite = np.arange(n) != 150
    for g in (np.array([150, 160, 170, 180], dtype=np.int32), np.array([7, 150, 200, 250], dtype=np.int32)):
        slot = int(np.nonzero(g == 150)[0][0])
        for eps in (0.0, 0.2):
            say("inf-generator", f"{dtype} slot={slot} eps={eps}")
            out = run_gpu(X, None, g, eps)
            f_g, a_g = to_host(out["f"]), to_host(out["alpha"])
            assert f_g[150] == -1 and a_g[150] == 0.0
            assert not np.any(f_g[finite] == slot)
            check_compress(X, g, eps, to_host(out["C"]), f_g, a_g)


@pytest.mark.parametrize("n,k", [
    (65536, 256),   # 256-row blocks, one generator tile: 4 waves of 128 x 128
    (32768, 256),   # 128-row blocks
    (65536, 300),   # several generator tiles: 8 waves of 128 x 64, then the merge
])
def test_gemm_tiles_degenerate_rows(n, k):
    # the same degenerate cases on the GEMM-shaped kernel (bf16, 256-generator
    # tiles): duplicate and collinear generators, a zero generator, a zero
    # row, a NaN row, and a generator holding +inf
    d = 128
    X32 = synth.bf16_bits_to_f32(synth.random_matrix(n, d, 33, "bf16")).copy()
    X32[40] = X32[7]
    X32[41] = -4 * X32[7]
    X32[100] = 0.0
    X32[101] = 0.0
    X32[102, 5] = np.nan
    X32[150, 3] = np.inf    # a generator holding +inf: scores NaN, never wins
    X = synth.f32_to_bf16_bits(X32)
    rng = np.random.default_rng(34)
    others = rng.choice(np.setdiff1d(np.arange(n), [7, 40, 41, 100, 101, 102, 150, 200]), k - 5, replace=False)
    g = np.sort(np.concatenate([[7, 40, 100, 150, 200], others])).astype(np.int32)
    s7, s100, s150 = (int(np.searchsorted(g, r)) for r in (7, 100, 150))
    gd = torch.from_numpy(g).cuda()
    for eps in (0.0, 0.2):
        say("gemm-degenerate", f"n={n} k={k} eps={eps}")
        C, f, a = pamm.compress(to_dev(X), gd, eps)
        torch.cuda.synchronize()
        f_g, a_g = to_host(f), to_host(a)
        assert f_g[7] == s7 and f_g[40] == s7 and f_g[41] == s7
        assert abs(a_g[41] + 4.0) <= 4.0 * 1e-5 and a_g[7] == a_g[40]
        assert f_g[102] == -1 and a_g[102] == 0.0
        if eps == 0.0:
            assert f_g[101] == 0 and a_g[101] == 0.0   # all scores 0: the lowest slot
        else:
            assert f_g[101] == -1 and f_g[100] == -1
        nonzero = np.ones(n, bool)
        nonzero[[100, 101, 102, 150]] = False
        assert not np.any(f_g[nonzero] == s100)   # the zero generator never wins a nonzero row
        assert f_g[150] == -1 and not np.any(f_g == s150)
        check_compress(X, g, eps, to_host(C), f_g, a_g)


@pytest.mark.parametrize("n,k", [(65536, 256), (32768, 256), (65536, 512)])
def test_gemm_tiles_degenerate_rows_plain_generators(n, k):
    # the same rows with every generator of finite, positive norm (no zero
    # generator, no padding): the epilogue's shorter scan
    d = 128
    X32 = synth.bf16_bits_to_f32(synth.random_matrix(n, d, 35, "bf16")).copy()
    X32[40] = X32[7]
    X32[41] = -4 * X32[7]
    X32[101] = 0.0
    X32[102, 5] = np.nan
    X = synth.f32_to_bf16_bits(X32)
    rng = np.random.default_rng(36)
    others = rng.choice(np.setdiff1d(np.arange(n), [7, 40, 41, 101, 102]), k - 2, replace=False)
    g = np.sort(np.concatenate([[7, 40], others])).astype(np.int32)
    s7 = int(np.searchsorted(g, 7))
    gd = torch.from_numpy(g).cuda()
    for eps in (0.0, 0.2):
        say("gemm-degenerate-plain", f"n={n} k={k} eps={eps}")
        C, f, a = pamm.compress(to_dev(X), gd, eps)
        torch.cuda.synchronize()
        f_g, a_g = to_host(f), to_host(a)
        assert f_g[7] == s7 and f_g[40] == s7 and f_g[41] == s7
        assert abs(a_g[41] + 4.0) <= 4.0 * 1e-5 and a_g[7] == a_g[40]
        assert f_g[102] == -1 and a_g[102] == 0.0
        if eps == 0.0:
            assert f_g[101] == 0 and a_g[101] == 0.0   # all scores 0: the lowest slot
        else:
            assert f_g[101] == -1
        check_compress(X, g, eps, to_host(C), f_g, a_g)


def test_no_generators_and_single_row():
    X = synth.random_matrix(50, 16, 41, "bf16")
    dY = synth.random_matrix(50, 24, 42, "bf16")
    say("k=0")
    out = run_gpu(X, dY, np.zeros(0, dtype=np.int32), 0.0)
    assert np.all(to_host(out["f"]) == -1) and np.all(to_host(out["alpha"]) == 0)
    assert np.all(to_host(out["dW"]) == 0)
    say("n=1")
    X1, dY1 = X[:1], dY[:1]
    out = run_gpu(X1, dY1, np.array([0], dtype=np.int32), 0.5)
    assert to_host(out["f"])[0] == 0 and to_host(out["alpha"])[0] == 1.0
    e = rel(to_host(out["dW"]), orc.to_f64(X1).T @ orc.to_f64(dY1))
    assert e < 1e-4


def test_eps_above_one_drops_everything():
    X, dY, p = synth.make_config("gpt2_small_qkv", rows=2048)
    g = pamm.sample_generators(2048, 16, 5).numpy()
    say("eps>1")
    out = run_gpu(X, dY, g, 1.5)
    assert np.all(to_host(out["f"]) == -1)
    assert np.all(to_host(out["dW"]) == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,dout", [(128, 160), (123, 157), (5, 3)])
def test_accumulate_and_strided_views(dtype, d, dout):
    # strided views whose row lengths need not be multiples of 16 bytes: the
    # leading dimensions are, as the C ABI requires
    n, k = 900, 12
    ldx = (d + 7) // 8 * 8 + 16      # multiples of 16 bytes for both dtypes
    lddy = (dout + 7) // 8 * 8 + 16
    Xbig = synth.clustered_activations(n, ldx, 8, seed=51 + d, dtype=dtype)
    dYbig = synth.gradients(n, lddy, seed=52, dtype=dtype)
    X = np.ascontiguousarray(Xbig[:, :d])
    dY = np.ascontiguousarray(dYbig[:, :dout])
    g = pamm.sample_generators(n, k, 53).numpy()
    say("strided", dtype, f"d={d} ldx={ldx} d_out={dout} lddy={lddy}")
    Xd = to_dev(Xbig)[:, :d]
    dYd = to_dev(dYbig)[:, :dout]
    gd = torch.from_numpy(g).cuda()
    C, f, a = pamm.compress(Xd, gd, 0.1)
    lddw = dout + 8 - dout % 4
    dW0 = torch.full((d, lddw), 3.0, device="cuda")[:, :dout]
    pamm.wgrad(C, f, a, dYd, dW=dW0, accumulate=True)
    xt_big = torch.full((n, ldx), 7.0, device="cuda", dtype=Xd.dtype)
    pamm.decompress(C, f, a, out=xt_big[:, :d])
    torch.cuda.synchronize()
    C_g, f_g, a_g = to_host(C), to_host(f), to_host(a)
    check_compress(X, g, 0.1, C_g, f_g, a_g)
    ref = orc.wgrad(C_g, f_g, a_g, dY) + 3.0
    assert rel(to_host(dW0), ref) < 1e-4
    xt = to_host(xt_big)
    _, xt_o = orc.decompress(C_g, f_g, a_g)
    assert np.array_equal(xt[:, :d], xt_o)
    # nothing written past the row length
    assert np.all(orc.to_f64(xt[:, d:]) == 7.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_default_outputs_with_ragged_rows(dtype):
    # widths whose rows do not fill whole 16 bytes: outputs the binding
    # allocates get padded rows (the leading-dimension rule of the C ABI) and
    # hold the same bits as outputs the caller supplies; k = 300 takes the
    # wide product tile, whose last 16-byte piece of a row is partly outside
    n, d, dout, k = 3000, 123, 157, 300
    ldx = (d + 7) // 8 * 8 + 8
    lddy = (dout + 7) // 8 * 8 + 8
    Xbig = synth.clustered_activations(n, ldx, 8, seed=81, dtype=dtype)
    dYbig = synth.gradients(n, lddy, seed=82, dtype=dtype)
    Xd, dYd = to_dev(Xbig)[:, :d], to_dev(dYbig)[:, :dout]
    g = pamm.sample_generators(n, k, 83).cuda()
    say("default outputs", dtype, f"n={n} d={d} d_out={dout} k={k}")
    C, f, a = pamm.compress(Xd, g, 0.1)
    dW = pamm.wgrad(C, f, a, dYd)
    given = torch.full((d, dout + 3), 5.0, device="cuda")
    pamm.wgrad(C, f, a, dYd, dW=given[:, :dout])
    dWt = pamm.wgrad(C, f, a, dYd, transpose_out=True)
    xt = pamm.decompress(C, f, a)
    xt2 = pamm.decompress(C, f, a, out=torch.empty((n, ldx), dtype=C.dtype, device="cuda")[:, :d])
    torch.cuda.synchronize()
    assert dW.shape == (d, dout) and dWt.shape == (dout, d) and xt.shape == (n, d)
    assert torch.equal(dW, given[:, :dout]) and torch.equal(dWt, dW.t()) and torch.equal(xt, xt2)
    assert torch.all(given[:, dout:] == 5.0)
    ref = orc.wgrad(to_host(C), to_host(f), to_host(a), np.ascontiguousarray(dYbig[:, :dout]))
    assert rel(to_host(dW), ref) < 1e-4
    if dtype == "bf16":
        dy = 150                      # Y rows of 300 bytes
        Wbig = synth.random_matrix(dy, ldx, 84, "bf16")
        Wd = to_dev(Wbig)[:, :d]
        Y = pamm.forward_compress(Xd, Wd, g, 0.1)[0]
        Yg = torch.empty((n, dy + 2), dtype=torch.bfloat16, device="cuda")[:, :dy]
        pamm.forward_compress(Xd, Wd, g, 0.1, Y=Yg)
        torch.cuda.synchronize()
        assert Y.shape == (n, dy) and torch.equal(Y, Yg)


def test_deterministic_bitwise():
    X, dY, p = synth.make_config("gpt2_small_qkv")
    g = pamm.sample_generators(p["n"], p["k"], 9).numpy()
    say("determinism")
    a = run_gpu(X, dY, g, p["eps"])
    b = run_gpu(X, dY, g, p["eps"])
    for key in ("C", "f", "alpha", "dW"):
        assert torch.equal(a[key], b[key]), key


# --------------------------------------------------------------------------
# full-size workloads: every row of (f, alpha) and every dW column, the
# oracle split over host threads; plus bitwise rerun determinism
# --------------------------------------------------------------------------

def full_size_case(name, k=None):
    X, dY, p = synth.make_config(name, k=k)
    n, d, dout = p["n"], p["d"], p["d_out"]
    k = p["k"]
    g = pamm.sample_generators(n, k, synth.generator_seed(name)).numpy()
    say(name, f"n={n} d={d} d_out={dout} k={k} eps={p['eps']} (every row and column, {ORACLE_THREADS} threads)")
    t0 = time.perf_counter()
    out = run_gpu(X, dY, g, p["eps"])
    C_g, f_g, a_g = to_host(out["C"]), to_host(out["f"]), to_host(out["alpha"])
    dW_g = to_host(out["dW"])
    again = run_gpu(X, dY, g, p["eps"])
    for key in ("f", "alpha", "dW"):
        assert torch.equal(out[key], again[key]), key
    del again, out
    torch.cuda.empty_cache()
    say(name, "gpu done, oracle compress")
    stats, f_o, a_o = check_compress(X, g, p["eps"], C_g, f_g, a_g, return_oracle=True)
    say(name, "oracle wgrad")
    e = check_wgrad(C_g, f_g, a_g, dY, dW_g)
    assert np.all((f_g >= -1) & (f_g < k))
    assert np.all(a_g[f_g < 0] == 0)
    # end to end: the GPU's dW against the oracle's wgrad of the oracle's own
    # triple.  Within the tolerance always (an in-band flip moves a row to a
    # generator of equal score up to rounding); within the arithmetic bound
    # when every index agrees
    say(name, "oracle wgrad of the oracle's own triple")
    dt = "bf16" if X.dtype == np.uint16 else "f32"
    e2e = rel(dW_g, oracle_wgrad(C_g, f_o, a_o, dY))
    assert e2e <= TOL[dt], f"end-to-end dW error {e2e}"
    if stats["inband_mismatches"] == 0:
        assert e2e <= TIGHT[dt], f"end-to-end dW error {e2e} with identical indices"
    say(name, "ok", stats, f"dW {e:.2e} e2e {e2e:.2e}", f"{time.perf_counter() - t0:.1f} s")
    return stats


def test_llama7b_qkv_full_size():
    full_size_case("llama7b_qkv")


@pytest.mark.parametrize("k", [1024, 256, 128, 64])
def test_llama1b_sweep_full_size(k):
    full_size_case("llama1b_sweep", k=k)


def test_longseq_gqa_full_size():
    full_size_case("longseq_gqa")
