"""Pins for the CPU oracle: each test checks the oracle against something that
does not come from the oracle itself -- a hand-worked example, a published RNG
output, a closed form, a textbook/library routine (least squares, a dense
matrix product), an invariant of the definition, or brute force on tiny
inputs.  The method is the one on the page "QKV Projections Require a
Fraction of Their Memory", section 2 "Metodologia", sub-part "Algoritmo in Due
Fasi".
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as orc
from activation_compression_pamm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def gauss(n, d, seed, dtype="f32"):
    return synth.random_matrix(n, d, seed, dtype)


# --------------------------------------------------------------------------
# random generator selection
# --------------------------------------------------------------------------

def test_splitmix64_matches_published_vector():
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed1234567.json")))
    got = orc.splitmix64_stream(g["seed"], len(g["outputs"]))
    assert [int(v) for v in got] == [int(v) for v in g["outputs"]]


@pytest.mark.parametrize("n,k,seed", [(1, 1, 0), (10, 3, 5), (1000, 37, 9), (4096, 4096, 1), (50, 0, 2)])
def test_sample_is_sorted_distinct_in_range(n, k, seed):
    idx = orc.sample_generators(n, k, seed)
    assert idx.size == k
    assert np.all(np.diff(idx) > 0)
    if k:
        assert idx[0] >= 0 and idx[-1] < n
    if k == n:
        assert np.array_equal(idx, np.arange(n))


def test_sample_subsets_uniform():
    # Uniform sampling without replacement: for n=4, k=2 every one of the 6
    # subsets has probability 1/6.  Chi-square over 12000 seeds, 5 dof.
    from collections import Counter
    cnt = Counter(tuple(orc.sample_generators(4, 2, s)) for s in range(12000))
    assert len(cnt) == 6
    exp = 12000 / 6
    chi2 = sum((v - exp) ** 2 / exp for v in cnt.values())
    assert chi2 < 25.0  # p ~ 1.4e-4 at 5 dof


def test_sample_inclusion_uniform():
    # each index is included with probability k/n
    n, k, trials = 30, 7, 6000
    hits = np.zeros(n)
    for s in range(trials):
        hits[orc.sample_generators(n, k, 10_000 + s)] += 1
    p = k / n
    z = (hits - trials * p) / np.sqrt(trials * p * (1 - p))
    assert np.abs(z).max() < 4.5


def test_sample_rejects_bad_args():
    with pytest.raises(ValueError):
        orc.sample_generators(5, 6, 0)
    with pytest.raises(ValueError):
        orc.sample_generators(5, -1, 0)


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_example(dtype):
    g = json.load(open(os.path.join(GOLD, "hand_example.json")))
    X = np.array(g["X"], dtype=np.float32)
    dY = np.array(g["dY"], dtype=np.float32)
    if dtype == "bf16":  # every value is exact in bf16
        X, dY = synth.f32_to_bf16_bits(X), synth.f32_to_bf16_bits(dY)
    r = orc.compress(X, np.array(g["gen_idx"]), g["eps"])
    assert r["f"].tolist() == g["f"]
    assert r["alpha"].tolist() == g["alpha"]
    dW = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    assert dW.tolist() == g["dW"]
    x64, xt = orc.decompress(r["C"], r["f"], r["alpha"])
    assert x64.tolist() == g["Xt"]
    assert orc.to_f64(xt).tolist() == g["Xt"]


# --------------------------------------------------------------------------
# k = n: every row is its own generator and dW is the exact product
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_equals_n_is_exact_product(dtype):
    n, d, dout = 40, 12, 9
    X = gauss(n, d, 1, dtype)
    dY = gauss(n, dout, 2, dtype)
    r = orc.compress(X, np.arange(n), 0.0)
    assert np.array_equal(r["f"], np.arange(n))
    assert np.all(r["alpha"] == 1.0)
    dW = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    exact = orc.to_f64(X).T @ orc.to_f64(dY)
    assert rel(dW, exact) < 1e-12


# --------------------------------------------------------------------------
# brute force on tiny inputs: exhaustive generator choice by least squares
# --------------------------------------------------------------------------

def brute_force(X64, gen_idx, eps):
    """Distance of each row to the line spanned by each generator, by
    numpy.linalg.lstsq; the nearest line wins (first on ties); the row is
    kept iff 1 - residual/|x|^2 >= eps^2 (|cos| >= eps)."""
    C = X64[gen_idx]
    n = X64.shape[0]
    f = np.full(n, -1)
    a = np.zeros(n)
    tie = np.zeros(n, dtype=bool)
    for i in range(n):
        x = X64[i]
        res = np.empty(len(gen_idx))
        coef = np.empty(len(gen_idx))
        for j, c in enumerate(C):
            sol, *_ = np.linalg.lstsq(c[:, None], x, rcond=None)
            coef[j] = sol[0]
            res[j] = np.sum((x - sol[0] * c) ** 2)
        j = int(np.argmin(res))
        xx = np.sum(x * x)
        srt = np.sort(res)
        if len(srt) > 1 and srt[1] - srt[0] <= 1e-9 * max(xx, 1e-300):
            tie[i] = True
        cos2 = 1.0 - res[j] / xx if xx > 0 else 0.0
        if abs(np.sqrt(max(cos2, 0.0)) - eps) < 1e-9:
            tie[i] = True
        if np.sqrt(max(cos2, 0.0)) >= eps:
            f[i] = j
            a[i] = coef[j]
    return f, a, tie


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("eps", [0.0, 0.3, 0.7])
def test_brute_force_tiny(seed, eps):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(8, 65))
    d = int(rng.integers(2, 17))
    k = int(rng.integers(1, 9))
    dtype = "bf16" if seed % 2 else "f32"
    X = gauss(n, d, 100 + seed, dtype)
    dY = gauss(n, 5, 200 + seed, dtype)
    gen_idx = orc.sample_generators(n, k, 300 + seed)
    X64 = orc.to_f64(X)
    r = orc.compress(X, gen_idx, eps)
    f_bf, a_bf, tie = brute_force(X64, gen_idx, eps)
    ok = ~tie
    assert ok.sum() >= n - 1
    assert np.array_equal(r["f"][ok], f_bf[ok])
    # alpha: the oracle's fp32 value vs the least-squares coefficient
    keep = ok & (f_bf >= 0)
    np.testing.assert_allclose(r["alpha"][keep], a_bf[keep], rtol=2 ** -23, atol=1e-30)
    # dW through a dense one-hot coefficient matrix: (S C)^T dY
    S = np.zeros((n, k))
    S[np.nonzero(r["f"] >= 0)[0], r["f"][r["f"] >= 0]] = r["alpha"][r["f"] >= 0]
    dW_bf = (S @ orc.to_f64(r["C"])).T @ orc.to_f64(dY)
    dW = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    assert rel(dW, dW_bf) < 1e-12 or np.linalg.norm(dW_bf) == np.linalg.norm(dW) == 0


# --------------------------------------------------------------------------
# exact special cases and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scaled_copies_reproduce_exactly(dtype):
    n, d = 30, 10
    X = gauss(n, d, 7, dtype).copy()
    gen_idx = np.array([2, 5, 11, 17])
    scales = {20: (0, 2.0), 21: (1, -4.0), 22: (2, 0.5), 23: (3, -0.25), 24: (0, -1.0)}
    X32 = synth.bf16_bits_to_f32(X) if dtype == "bf16" else X.astype(np.float32)
    for row, (j, s) in scales.items():
        X32[row] = np.float32(s) * X32[gen_idx[j]]
    X = synth.f32_to_bf16_bits(X32) if dtype == "bf16" else X32
    r = orc.compress(X, gen_idx, 0.0)
    _, xt = orc.decompress(r["C"], r["f"], r["alpha"])
    for row, (j, s) in scales.items():
        assert r["f"][row] == j
        assert r["alpha"][row] == s
        assert np.array_equal(xt[row], X[row])


def test_self_assignment():
    X = gauss(50, 16, 8)
    gen_idx = orc.sample_generators(50, 9, 4)
    r = orc.compress(X, gen_idx, 0.0)
    assert np.array_equal(r["f"][gen_idx], np.arange(9))
    assert np.all(r["alpha"][gen_idx] == 1.0)


def test_footprint():
    for dtype, es in ((0, 4), (1, 2)):
        X = gauss(64, 24, 9, "bf16" if dtype else "f32")
        r = orc.compress(X, np.arange(0, 64, 8), 0.0)
        nbytes = r["C"].nbytes + r["f"].nbytes + r["alpha"].nbytes
        assert nbytes == orc.footprint_bytes(64, 8, 24, dtype) == 8 * 24 * es + 8 * 64


def test_k1_closed_form():
    # one generator, eps = 0: dW = c (c^T X^T dY) / |c|^2 up to the fp32
    # rounding of each alpha
    n, d, dout = 60, 14, 11
    X = gauss(n, d, 10)
    dY = gauss(n, dout, 11)
    r = orc.compress(X, np.array([13]), 0.0)
    assert np.all(r["f"] == 0)
    c = X[13].astype(np.float64)
    X64, dY64 = X.astype(np.float64), dY.astype(np.float64)
    closed = np.outer(c, c @ X64.T @ dY64) / (c @ c)
    dW = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    assert rel(dW, closed) < 1e-6


def test_eps_extremes():
    X = gauss(80, 12, 12)
    dY = gauss(80, 6, 13)
    gen_idx = orc.sample_generators(80, 5, 1)
    r0 = orc.compress(X, gen_idx, 0.0)
    assert np.all(r0["f"] >= 0)
    r1 = orc.compress(X, gen_idx, 1.5)
    assert np.all(r1["f"] == -1) and np.all(r1["alpha"] == 0.0)
    assert np.all(orc.wgrad(r1["C"], r1["f"], r1["alpha"], dY) == 0.0)
    # eps in between: kept iff cosine >= eps
    r = orc.compress(X, gen_idx, 0.4)
    assert np.array_equal(r["f"] >= 0, r0["cos"].astype(np.float32) >= np.float32(0.4))


def test_sign_flip_of_a_row():
    X = gauss(40, 10, 14)
    gen_idx = np.array([0, 7, 19])
    r = orc.compress(X, gen_idx, 0.2)
    Xn = X.copy()
    others = np.setdiff1d(np.arange(40), gen_idx)
    Xn[others] = -Xn[others]
    rn = orc.compress(Xn, gen_idx, 0.2)
    assert np.array_equal(rn["f"], r["f"])
    assert np.array_equal(rn["alpha"][others], -r["alpha"][others])
    assert np.array_equal(rn["cos"], r["cos"])


def test_power_of_two_scaling():
    X = gauss(40, 10, 15)
    dY = gauss(40, 7, 16)
    gen_idx = np.array([1, 9, 22, 30])
    r = orc.compress(X, gen_idx, 0.1)
    r2 = orc.compress(X * np.float32(2.0), gen_idx, 0.1)
    assert np.array_equal(r2["f"], r["f"])
    assert np.array_equal(r2["alpha"], r["alpha"])
    assert np.array_equal(r2["C"], 2 * r["C"])
    assert np.array_equal(orc.wgrad(r2["C"], r2["f"], r2["alpha"], dY),
                          2 * orc.wgrad(r["C"], r["f"], r["alpha"], dY))


def test_linearity_in_dY():
    X = gauss(50, 10, 17)
    rng = np.random.default_rng(0)
    d1 = rng.integers(-8, 9, size=(50, 6)).astype(np.float32)
    d2 = rng.integers(-8, 9, size=(50, 6)).astype(np.float32)
    r = orc.compress(X, np.array([3, 8, 40]), 0.0)
    w12 = orc.wgrad(r["C"], r["f"], r["alpha"], d1 + d2)
    w1 = orc.wgrad(r["C"], r["f"], r["alpha"], d1)
    w2 = orc.wgrad(r["C"], r["f"], r["alpha"], d2)
    assert rel(w12, w1 + w2) < 1e-12


def test_row_permutation():
    n = 45
    X = gauss(n, 9, 18)
    dY = gauss(n, 5, 19)
    gen_idx = np.array([4, 10, 33])
    r = orc.compress(X, gen_idx, 0.3)
    perm = np.random.default_rng(1).permutation(n)  # new row i = old row perm[i]
    inv = np.argsort(perm)
    gnew = np.sort(inv[gen_idx])
    rp = orc.compress(X[perm], gnew, 0.3)
    old_gen_row = np.where(r["f"] >= 0, gen_idx[np.maximum(r["f"], 0)], -1)
    new_gen_row = np.where(rp["f"] >= 0, perm[gnew[np.maximum(rp["f"], 0)]], -1)
    assert np.array_equal(new_gen_row, old_gen_row[perm])
    assert np.array_equal(rp["alpha"], r["alpha"][perm])
    assert rel(orc.wgrad(rp["C"], rp["f"], rp["alpha"], dY[perm]),
               orc.wgrad(r["C"], r["f"], r["alpha"], dY)) < 1e-12


def test_reconstruction_associativity():
    X = gauss(70, 12, 20, "bf16")
    dY = gauss(70, 8, 21, "bf16")
    r = orc.compress(X, orc.sample_generators(70, 6, 3), 0.2)
    x64, _ = orc.decompress(r["C"], r["f"], r["alpha"])
    assert rel(orc.wgrad(r["C"], r["f"], r["alpha"], dY), x64.T @ orc.to_f64(dY)) < 1e-12


# --------------------------------------------------------------------------
# the reconstruction's rounding to bf16 (reading R9: the fp32 product alpha*c
# rounded to the storage dtype, nearest-even)
# --------------------------------------------------------------------------

def _is_nan_bf16(h):
    h = np.asarray(h, dtype=np.uint16)
    return ((h & 0x7f80) == 0x7f80) & ((h & 0x007f) != 0)


def test_reconstruction_rounding_golden_table():
    # each golden fp32 value v is reconstructed as v * 1.0 (one generator equal
    # to bf16 1.0, alpha = v), so the stored bf16 is the rounding of v itself
    g = json.load(open(os.path.join(GOLD, "bf16_rounding.json")))
    cases = g["cases"]
    alpha = np.array([int(c["f32"], 16) for c in cases], dtype=np.uint32).view(np.float32)
    C = np.array([[0x3f80]], dtype=np.uint16)
    f = np.zeros(len(cases), dtype=np.int32)
    _, xt = orc.decompress(C, f, alpha)
    for c, got in zip(cases, xt[:, 0]):
        if c["bf16"] == "nan":
            assert _is_nan_bf16(got), (c, hex(int(got)))
        else:
            assert int(got) == int(c["bf16"], 16), (c, hex(int(got)))


def test_reconstruction_rounding_matches_torch():
    # random bf16 generators times random fp32 scales, many products landing
    # exactly on a rounding tie, plus overflow, subnormal and NaN products.
    # Expected: numpy's fp32 product (one IEEE rounding) converted by torch's
    # CPU float32 -> bfloat16 conversion (round to nearest even); neither shares
    # code with the oracle.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    k, d, n = 16, 64, 600
    cbits = rng.integers(0, 1 << 16, size=(k, d), dtype=np.uint32).astype(np.uint16)
    cbits[(cbits & 0x7f80) == 0x7f80] &= 0xbfff          # finite generators (exponent not all ones)
    cbits[0] = 0x3f80                                    # a generator of ones: product = alpha
    cbits[1] = np.where(np.arange(d) % 2, 0x4000, 0xc080)  # powers of two: +2, -4
    abits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    abits[(abits & 0x7f800000) == 0x7f800000] ^= 0x40000000   # finite scales ...
    e = rng.integers(100, 150, size=n).astype(np.uint32)      # ... mostly of moderate exponent,
    abits[: n // 2] = (abits[: n // 2] & 0x807fffff) | (e[: n // 2] << 23)
    ties = slice(n // 2, n // 2 + 150)                        # exact ties: low 16 bits 0x8000
    abits[ties] = (abits[ties] & 0xffff0000) | 0x8000
    abits[ties] = (abits[ties] & 0x807fffff) | (e[ties] << 23)
    abits[-9:] = [0x7f7fffff, 0xff7f8000, 0x00018000, 0x80008000, 0x7fc00000, 0x7fffffff, 0x00000000, 0x80000000, 0x0001ffff]
    alpha = abits.view(np.float32)
    f = rng.integers(-1, k, size=n).astype(np.int32)
    f[n // 2: n // 2 + 200] = rng.integers(0, 2, size=200)      # ties and scales through generators 0 and 1
    f[-9:] = 0
    _, xt = orc.decompress(cbits, f, alpha)
    c32 = (cbits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = np.where(f[:, None] >= 0, alpha[:, None] * c32[np.maximum(f, 0)], np.float32(0)).astype(np.float32)
    want = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(prod)
    assert np.array_equal(_is_nan_bf16(xt), nan)
    assert np.array_equal(xt[~nan], want[~nan])
    # the set really contains ties and overflow
    low = prod.view(np.uint32) & 0xffff
    assert np.count_nonzero(low == 0x8000) > 100
    assert np.any(np.isinf(prod))


def test_column_subset_matches_full():
    X = gauss(60, 10, 22)
    dY = gauss(60, 13, 23)
    r = orc.compress(X, np.array([0, 5, 9]), 0.1)
    full = orc.wgrad(r["C"], r["f"], r["alpha"], dY)
    cols = np.array([12, 0, 7])
    assert np.array_equal(orc.wgrad(r["C"], r["f"], r["alpha"], dY, cols=cols), full[:, cols])


def test_row_subset_matches_full():
    X = gauss(60, 10, 24, "bf16")
    g = np.array([2, 30, 44, 59])
    full = orc.compress(X, g, 0.25)
    rows = np.array([59, 3, 30, 17])
    sub = orc.compress(X, g, 0.25, rows=rows)
    for key in ("f", "alpha", "cos", "margin"):
        assert np.array_equal(sub[key], full[key][rows])


# --------------------------------------------------------------------------
# degenerate inputs
# --------------------------------------------------------------------------

def test_duplicate_generators_tie_to_lowest_slot():
    X = gauss(30, 8, 25)
    X[12] = X[4]          # two identical rows, both generators
    X[20] = 2 * X[4]      # collinear with both
    g = np.array([4, 12, 25])
    r = orc.compress(X, g, 0.0)
    assert r["f"][4] == 0 and r["f"][12] == 0 and r["f"][20] == 0
    assert r["alpha"][20] == 2.0


def test_zero_rows_and_zero_generator():
    X = gauss(20, 6, 26)
    X[3] = 0.0  # zero generator
    X[7] = 0.0  # zero row (not a generator)
    g = np.array([3, 10, 15])
    r = orc.compress(X, g, 0.0)
    assert r["f"][7] == 0 and r["alpha"][7] == 0.0 and r["cos"][7] == 0.0
    assert np.all(r["f"][np.setdiff1d(np.arange(20), [3, 7])] != 0)  # zero generator never wins
    r1 = orc.compress(X, g, 0.1)
    assert r1["f"][7] == -1 and r1["f"][3] == -1


def test_nan_row_is_dropped():
    X = gauss(20, 6, 27)
    X[5, 2] = np.nan
    r = orc.compress(X, np.array([0, 9]), 0.0)
    assert r["f"][5] == -1 and r["alpha"][5] == 0.0
    assert np.all(r["f"][np.arange(20) != 5] >= 0)
    # even when a zero generator offers a finite score of 0
    X[11] = 0.0
    r = orc.compress(X, np.array([0, 9, 11]), 0.0)
    assert r["f"][5] == -1 and r["alpha"][5] == 0.0


def test_no_generators_drops_everything():
    X = gauss(10, 4, 28)
    r = orc.compress(X, np.zeros(0, dtype=np.int32), 0.0)
    assert np.all(r["f"] == -1)


def test_clustered_inputs_assign_by_cluster():
    # rows of the synthetic workload fall to a generator of their own cluster
    # 8 clusters and 96 generators: a cluster without a generator has
    # probability 8 * (7/8)^96 < 1e-4
    X = synth.clustered_activations(512, 64, 8, seed=5, dtype="f32")
    g = orc.sample_generators(512, 96, 6)
    r = orc.compress(X, g, 0.5)
    assert (r["f"] >= 0).mean() > 0.9
    assert np.median(r["cos"]) > 0.95


# --------------------------------------------------------------------------
# decisions in fp32 (reading R8), NaN generators (R5), dropped rows in the
# gradient, strided views, the rounding-band margin
# --------------------------------------------------------------------------

def test_argmax_decided_on_fp32_scores():
    # Rows r0 = (1, 2^-12) and r1 = (1, 2^-13) are the generators; row r2 =
    # (1, 0) scores 1/sqrt(1 + 2^-24) against r0 and 1/sqrt(1 + 2^-26)
    # against r1.  The second is larger, but both lie within half an fp32
    # ulp of 1 (1 - 2^-25 + O(2^-48) is just above the midpoint 1 - 2^-25,
    # 1 - 2^-27 well above it), so both round to 1.0f: a tie, which the
    # lowest slot wins.  An fp64 argmax would pick slot 1.
    X = np.array([[1.0, 2.0 ** -12], [1.0, 2.0 ** -13], [1.0, 0.0]], dtype=np.float32)
    r = orc.compress(X, np.array([0, 1]), 0.0)
    assert r["f"][2] == 0
    # alpha = fp32(1 / (1 + 2^-24)) = fp32(1 - 2^-24 + 2^-48) = 1 - 2^-24
    assert r["alpha"][2] == np.float32(1.0 - 2.0 ** -24)
    # the scores themselves still differ in fp64
    s = orc.compress(X, np.array([0, 1]), 0.0, want_scores=True)["scores"][2]
    assert s[1] > s[0] and np.float32(s[0]) == np.float32(s[1]) == np.float32(1.0)


def test_eps_decided_on_fp32_cosine():
    # Row (1, 0) against the single generator (1, 2^-12): cosine
    # 1/sqrt(1 + 2^-24) < 1, which rounds to 1.0f.  With eps = 1 the fp32
    # test keeps the row; an fp64 test would drop it.
    X = np.array([[1.0, 2.0 ** -12], [1.0, 0.0]], dtype=np.float32)
    r = orc.compress(X, np.array([0]), 1.0)
    assert r["cos"][1] < 1.0
    assert r["f"][1] == 0 and r["alpha"][1] == np.float32(1.0 - 2.0 ** -24)
    # just above 1 nothing is kept
    r = orc.compress(X, np.array([0]), float(np.nextafter(np.float32(1.0), np.float32(2.0))))
    assert r["f"][1] == -1


@pytest.mark.parametrize("bad", [np.inf, np.nan])
def test_nonfinite_generator_never_wins(bad):
    # A generator holding +inf scores NaN (inf / inf) against every row, and
    # a NaN score never wins; one holding NaN has no usable norm and must
    # not win either.  Checked with the bad generator in the first slot and
    # in the last; the bad row itself is dropped (its cosine is NaN).
    X = gauss(12, 5, 29)
    X[2, 3] = bad
    for g in (np.array([2, 6]), np.array([1, 2])):
        r = orc.compress(X, g, 0.0)
        bad_slot = int(np.nonzero(g == 2)[0][0])
        other = [i for i in range(12) if i != 2]
        assert np.all(r["f"][other] == 1 - bad_slot)
        assert r["f"][2] == -1


def test_wgrad_ignores_rows_outside_the_generators():
    # f = -1 (dropped) and f >= k contribute nothing, whatever alpha says:
    # dW equals that of the triple with those rows removed.
    n, k, d, dout = 40, 5, 7, 6
    rng = np.random.default_rng(31)
    C = gauss(k, d, 32)
    dY = gauss(n, dout, 33)
    f = rng.integers(0, k, n).astype(np.int32)
    alpha = rng.normal(size=n).astype(np.float32)
    out = rng.random(n) < 0.4
    f[out] = np.where(rng.random(out.sum()) < 0.5, -1, k)
    full = orc.wgrad(C, f, alpha, dY)
    kept = ~out
    sub = orc.wgrad(C, f[kept], alpha[kept], dY[kept])
    assert out.any() and kept.any()
    assert np.array_equal(full, sub)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_views_match_dense_copies(dtype):
    # X and dY as column slices of wider matrices whose extra columns hold
    # NaN: any read past a row's d (or d_out) columns would poison the result.
    n, d, dout, pad = 48, 10, 9, 6
    X = gauss(n, d, 34, dtype)
    dY = gauss(n, dout, 35, dtype)
    nan = synth.f32_to_bf16_bits(np.float32(np.nan)) if dtype == "bf16" else np.float32(np.nan)
    Xw = np.full((n, d + pad), nan, dtype=X.dtype)
    Xw[:, :d] = X
    dYw = np.full((n, dout + pad), nan, dtype=dY.dtype)
    dYw[:, :dout] = dY
    g = orc.sample_generators(n, 6, 36)
    rv, rd = orc.compress(Xw[:, :d], g, 0.2), orc.compress(X, g, 0.2)
    for key in ("C", "f", "alpha", "cos", "margin"):
        assert np.array_equal(rv[key], rd[key]), key
    assert np.array_equal(orc.wgrad(rd["C"], rd["f"], rd["alpha"], dYw[:, :dout]),
                          orc.wgrad(rd["C"], rd["f"], rd["alpha"], dY))


def test_margin_and_scores_closed_form():
    # Generators e1 and e2; the row (3, 4) scores 3 and 4, cosine 4/5, and
    # the gap to the runner-up is (4 - 3)/5.
    X = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, 4.0]], dtype=np.float32)
    r = orc.compress(X, np.array([0, 1]), 0.0)
    assert r["f"][2] == 1 and r["alpha"][2] == 4.0
    assert abs(r["cos"][2] - 0.8) < 1e-15
    assert abs(r["margin"][2] - 0.2) < 1e-15
    # every generator's cosine: 3/5 and 4/5
    sc = orc.compress(X, np.array([0, 1]), 0.0, want_scores=True)["scores"][2]
    assert np.allclose(sc, [0.6, 0.8], rtol=0, atol=1e-15)
    # a single generator has no runner-up
    assert orc.compress(X, np.array([1]), 0.0)["margin"][2] == np.inf
