"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes a property that the pages or the mathematics determine:
brute force on tiny inputs, reductions to textbook routines (alpha = inf,
alpha = 0), the worked channel example, planted outliers, the quantization
error bound and its noise level, round-half-to-even ties and invariants.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth
from brute_force import brute, exact_product

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lists(a):
    return [[float(v) for v in row] for row in np.asarray(a, dtype=np.float64)]


def _check_against_brute(X, W, alpha, bias=None):
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, alpha, bias)
    b = brute(_lists(X), _lists(W), alpha,
              None if bias is None else [float(v) for v in np.asarray(bias, np.float64)])
    assert r.idx.tolist() == b["idx"]
    assert np.array_equal(aw, np.array(b["aw"], dtype=np.float32))
    # the stand-alone column absmax (the expected w_absmax of the GPU path)
    assert np.array_equal(O.weight_absmax(W), np.array(b["aw"], dtype=np.float32))
    assert np.array_equal(Wq, np.array(b["Wq"], dtype=np.int8).reshape(Wq.shape))
    assert np.array_equal(r.x_absmax, np.array(b["ax"], dtype=np.float32))
    assert np.array_equal(r.Xq, np.array(b["Xq"], dtype=np.int8).reshape(r.Xq.shape))
    assert np.array_equal(r.A.astype(np.int64), np.array(b["A"], dtype=np.int64).reshape(r.A.shape))
    M, N = r.Y64.shape
    for i in range(M):
        for j in range(N):
            ex = b["Yexact"][i][j]
            err = abs(Fraction(float(r.Y64[i, j])) - ex)
            assert err <= Fraction(1, 10**12) * (abs(ex) + 1), (i, j)
    # the fp16 output is the exact value rounded once
    ex16 = np.array([[float(v) for v in row] for row in b["Yexact"]]).astype(np.float16) if M and N else r.Y16
    assert np.array_equal(r.Y16.view(np.uint16), ex16.view(np.uint16))
    return r


def test_brute_tiny_workload():
    X, W, dims, _ = synth.make("tiny")
    r = _check_against_brute(X, W, 6.0)
    assert r.idx.tolist() == [17, 200]


@pytest.mark.parametrize("alpha", [0.0, 0.5, 6.0, float("inf")])
@pytest.mark.parametrize("seed,M,K,N,nout", [(1, 3, 8, 5, 1), (2, 7, 32, 9, 3),
                                             (3, 1, 17, 4, 2), (4, 12, 64, 16, 0),
                                             (5, 5, 40, 3, 6)])
def test_brute_random(alpha, seed, M, K, N, nout):
    X, W, _ = synth.random_case(seed, M, K, N, nout)
    _check_against_brute(X, W, alpha)


def test_brute_hypothesis_shapes():
    """Brute force on shapes and values drawn by hypothesis: arbitrary small
    M, K, N (K and N need not be multiples of anything here), fp16 values
    from a wide range with planted large magnitudes, several thresholds."""
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies

    @hyp.settings(max_examples=40, deadline=None, derandomize=True)
    @hyp.given(M=st.integers(1, 6), K=st.integers(1, 24), N=st.integers(1, 6),
               seed=st.integers(0, 2**31 - 1),
               alpha=st.sampled_from([0.0, 1.0, 6.0, 100.0, float("inf")]),
               scale=st.sampled_from([0.01, 1.0, 30.0]))
    def check(M, K, N, seed, alpha, scale):
        rng = np.random.default_rng(seed)
        X = (rng.standard_normal((M, K)) * scale).astype(np.float16)
        big = rng.random((M, K)) < 0.1
        X[big] = (rng.uniform(7, 120, big.sum()) * rng.choice([-1, 1], big.sum())).astype(np.float16)
        W = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
        _check_against_brute(X, W, alpha)

    check()


@pytest.mark.parametrize("alpha", [0.0, 6.0, float("inf")])
def test_brute_with_bias(alpha):
    """The layer bias ([GB "Exemple pratique"]) is added before the single
    rounding: pinned against the exact rational result."""
    X, W, _ = synth.random_case(11, 6, 48, 10, 2)
    bias = (np.arange(10) * 0.37 - 1.5).astype(np.float16)
    r = _check_against_brute(X, W, alpha, bias)
    r0 = O.mixed_matmul(X, *O.quantize_weight(W), W, alpha)
    assert np.array_equal(r.A, r0.A) and np.array_equal(r.idx, r0.idx)


@pytest.mark.parametrize("which", ["all", "some", "none"])
def test_cached_outlier_rows(which):
    """Static outlier-row cache: with every runtime outlier cached the result
    is exactly mixed_matmul's; otherwise the missing rows are the int8 rows
    dequantized to fp16 (brute force with struct-rounded binary32/binary16),
    and they are reported."""
    X, W, _ = synth.random_case(23, 7, 64, 12, 4)
    Wq, aw = O.quantize_weight(W)
    idx = O.detect_outliers(X, 6.0)
    dims = {"all": list(idx) + [3], "some": list(idx[1:3]), "none": []}[which]
    dims = np.array(sorted(set(int(d) for d in dims)), dtype=np.int32)
    r, missed = O.mixed_matmul_cached(X, Wq, aw, dims, W[dims], 6.0)
    assert sorted(missed.tolist()) == sorted(set(idx.tolist()) - set(dims.tolist()))
    if which == "all":
        r0 = O.mixed_matmul(X, Wq, aw, W, 6.0)
        assert np.array_equal(r.Y64, r0.Y64)
    b = brute(_lists(X), _lists(W), 6.0, cache_dims=set(dims.tolist()))
    for i in range(r.Y64.shape[0]):
        for j in range(r.Y64.shape[1]):
            ex = b["Yexact"][i][j]
            assert abs(Fraction(float(r.Y64[i, j])) - ex) <= Fraction(1, 10**12) * (abs(ex) + 1)
    if which == "none":  # the fallback really differs from the fp16 rows
        r0 = O.mixed_matmul(X, Wq, aw, W, 6.0)
        assert not np.array_equal(r.Y64, r0.Y64)


def test_dequantized_rows_match_brute_force():
    W = synth.random_case(5, 2, 32, 24, 0)[1]
    Wq, aw = O.quantize_weight(W)
    rows = O.dequant_weight_rows(Wq, aw, [0, 7, 31])
    from brute_force import f16, f32
    for r, k in enumerate([0, 7, 31]):
        for j in range(24):
            exp = f16(f32(int(Wq[k, j]) * f32(float(aw[j]) / 127.0)))
            assert float(rows[r, j]) == exp


def test_brute_zero_and_degenerate_rows():
    # row 1: only outlier entries are nonzero; row 2: all zero; column 3 of W zero
    X = np.zeros((4, 8), np.float16)
    X[0] = [1, -2, 3, 0.5, 20, 0, 0.25, -4]
    X[1, 4] = -30
    X[3] = [0.5, 1.5, 2.5, -0.5, 9, -1.5, 5, -5]
    W = np.linspace(-0.05, 0.05, 8 * 6).reshape(8, 6).astype(np.float16)
    W[:, 3] = 0
    r = _check_against_brute(X, W, 6.0)
    assert r.idx.tolist() == [4]
    assert r.x_absmax[1] == 0 and not r.Xq[1].any()
    assert r.x_absmax[2] == 0 and not r.Xq[2].any()
    assert np.isfinite(r.Y64).all()


def test_planted_outliers_all_workloads():
    """Normals are clipped at +-5 < 6, and every planted dim has entries far
    above 6, so detection at alpha=6 must return the planted dims exactly."""
    for name, w in synth.WORKLOADS.items():
        X, dims, rows = synth.make_x(w)
        assert O.detect_outliers(X, 6.0).tolist() == sorted(dims.tolist()), name
        assert O.detect_outliers(X, float("inf")).size == 0
        if name == "ffn175b":
            for a in (4.0, 8.0):
                assert O.detect_outliers(X, a).tolist() == sorted(dims.tolist())


def test_threshold_is_strict():
    X = np.zeros((3, 4), np.float16)
    X[0, 1] = 6.0                      # exactly alpha: not an outlier
    X[2, 2] = np.float16(6.00390625)   # next fp16 above 6
    X[1, 3] = -6.0
    X[1, 0] = -6.00390625
    assert O.detect_outliers(X, 6.0).tolist() == [0, 2]


def test_round_half_even_ties():
    """absmax 127 gives s = 127/127 = 1 exactly, so q = round-half-even(x)."""
    x = np.array([[127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -126.5, 125.5]], np.float16)
    q, ax = O.quantize_activations(x, np.zeros(0, np.int32))
    assert ax[0] == 127
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 4, -126, 126]
    # same for a weight column
    wq, aw = O.quantize_weight(x.T)
    assert wq[:, 0].tolist() == [127, 0, 2, 2, 0, -2, -2, 4, -126, 126]


def test_absmax_maps_to_127_and_range():
    X, W, _, _ = synth.make("tiny")
    idx = O.detect_outliers(X, 6.0)
    q, ax = O.quantize_activations(X, idx)
    keep = np.setdiff1d(np.arange(X.shape[1]), idx)
    for i in range(X.shape[0]):
        j = keep[np.argmax(np.abs(X[i, keep].astype(np.float32)))]
        assert abs(int(q[i, j])) == 127
    assert np.abs(q.astype(int)).max() <= 127 and not q[:, idx].any()
    wq, aw = O.quantize_weight(W)
    assert (np.abs(wq.astype(int)).max(axis=0) == 127).all()


def test_power_of_two_row_scaling_and_permutation():
    X, W, dims = synth.random_case(7, 9, 48, 11, 2)
    idx = O.detect_outliers(X, 6.0)
    q, ax = O.quantize_activations(X, idx)
    X2 = X.copy()
    X2[3, np.setdiff1d(np.arange(48), idx)] *= np.float16(0.5)  # stays below alpha
    q2, ax2 = O.quantize_activations(X2, idx)
    assert np.array_equal(q2, q) and ax2[3] == ax[3] / 2
    perm = np.random.default_rng(0).permutation(9)
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, 6.0)
    rp = O.mixed_matmul(X[perm], Wq, aw, W, 6.0)
    assert np.array_equal(rp.Xq, r.Xq[perm]) and np.array_equal(rp.A, r.A[perm])
    assert np.array_equal(rp.x_absmax, r.x_absmax[perm])


def test_alpha_zero_is_fp16_matmul():
    """alpha = 0 routes every nonzero column to the fp16 path: the result is
    the exact product X.W (here numpy's fp64 matmul of the fp16 values)."""
    X, W, _, _ = synth.make("tiny")
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, 0.0)
    assert not r.Xq.any() and not r.A.any()
    nzcols = np.nonzero(np.abs(X.astype(np.float32)).max(axis=0) > 0)[0]
    assert r.idx.tolist() == nzcols.tolist()
    ref = X.astype(np.float64) @ W.astype(np.float64)
    np.testing.assert_allclose(r.Y64, ref, rtol=1e-12, atol=1e-12)
    # exact rationals on a slice
    ex = exact_product(_lists(X[:2]), _lists(W[:, :3]))
    for i in range(2):
        for j in range(3):
            assert abs(Fraction(float(r.Y64[i, j])) - ex[i][j]) <= Fraction(1, 10**12)


def _error_terms(X, W, idx):
    keep = np.setdiff1d(np.arange(X.shape[1]), idx)
    Xk = np.abs(X[:, keep].astype(np.float64))
    Wk = np.abs(W[keep, :].astype(np.float64))
    ax = Xk.max(axis=1)
    aw = np.abs(W.astype(np.float64)).max(axis=0)
    bound = ((ax / 254)[:, None] * Wk.sum(axis=0)[None, :]
             + Xk.sum(axis=1)[:, None] * (aw / 254)[None, :]
             + keep.size * (ax / 254)[:, None] * (aw / 254)[None, :])
    # uniform rounding noise: step^2/12 per term
    var = (((ax / 127) ** 2 / 12)[:, None] * (Wk ** 2).sum(axis=0)[None, :]
           + (Xk ** 2).sum(axis=1)[:, None] * ((aw / 127) ** 2 / 12)[None, :])
    return bound, var


@pytest.mark.parametrize("name,alpha,cols", [("tiny", 6.0, None), ("tiny", float("inf"), None),
                                             ("channel", 6.0, 512), ("ffn13b", 6.0, 256)])
def test_error_bound_and_noise_level(name, alpha, cols):
    """|Y - X.W| is bounded by the half-step rounding of every int8 term, and
    its mean square matches the uniform-rounding-noise prediction."""
    X, dims, _ = synth.make_x(name)
    W = synth.make_w(name)
    if cols is not None:
        W = W[:, :cols]
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, alpha)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    bound, var = _error_terms(X, W, r.idx)
    err = np.abs(r.Y64 - exact)
    assert (err <= bound * (1 + 1e-4) + 1e-9).all()
    ratio = (err ** 2).mean() / var.mean()
    assert 0.8 < ratio < 1.25, ratio


def test_alpha_inf_is_plain_vectorwise():
    """With alpha = inf nothing is routed to fp16: the output is the plain
    vector-wise int8 product, whose rows that hold outliers lose the small
    channels (their step is set by the outlier)."""
    X, dims, rows = synth.make_x("tiny")
    W = synth.make_w("tiny")
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, float("inf"))
    assert r.idx.size == 0 and r.X_out.shape[1] == 0 and r.W_out.shape[0] == 0
    assert np.array_equal(r.x_absmax, np.abs(X.astype(np.float32)).max(axis=1))
    r6 = O.mixed_matmul(X, Wq, aw, W, 6.0)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    e_inf = np.abs(r.Y64 - exact)[rows].mean()
    e_6 = np.abs(r6.Y64 - exact)[rows].mean()
    assert e_inf > 3 * e_6


def test_channel_example_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "channel_example.json")))
    X, dims, rows = synth.make_x("channel")
    assert X.shape[1] == g["n_channels"] and dims.size == g["n_outlier_channels"]
    normal = np.setdiff1d(np.arange(X.shape[1]), dims)
    Xn = np.abs(X[:, normal].astype(np.float64))
    assert abs(Xn.mean() - g["normal_mean_abs"]) < 0.01
    assert Xn.max() <= g["normal_max"]
    Xo = np.abs(X[np.ix_(rows, dims)].astype(np.float64))
    assert abs(Xo.mean() - g["outlier_mean_abs"]) < 1.0 and Xo.max() == g["outlier_max"]

    # tensor-wise: one scale set by 130 -> step 130/127, "about 1.0"
    q, amax, deq = O.tensorwise_quantize(X)
    step = float(amax) / 127
    assert amax == g["outlier_max"] and abs(step - g["tensorwise_step_about"]) < 0.05
    qn = np.abs(q[:, normal].astype(int))
    # closed form for |N(0, s^2)| with E|x| = 0.5: P(q=0) = 0.5859, P(|q|<=1) = 0.9857
    assert abs((qn == 0).mean() - 0.5859) < 0.005
    assert abs((qn <= g["normal_codes_collapse_to_abs_at_most"]).mean() - 0.9857) < 0.005
    xn = X[:, normal].astype(np.float64)
    rel_tw = np.sqrt(((deq[:, normal] - xn) ** 2).mean() / (xn ** 2).mean())

    # decomposition: outlier channels leave, the row step drops to ~ax/127
    idx = O.detect_outliers(X, g["threshold_alpha"])
    assert idx.tolist() == dims.tolist()
    qd, ax = O.quantize_activations(X, idx)
    assert ax.max() <= g["normal_max"]
    deqd = qd[:, normal].astype(np.float64) * (ax.astype(np.float64) / 127)[:, None]
    rel_dec = np.sqrt(((deqd - xn) ** 2).mean() / (xn ** 2).mean())
    assert rel_tw > 0.3 and rel_dec < 0.03
    # closed form step^2/12: tensor-wise ~0.47, decomposed ~0.009
    assert abs(rel_tw - (step / np.sqrt(12)) / np.sqrt((xn ** 2).mean())) < 0.02


def test_int_gemm_exact():
    X, dims, _ = synth.make_x("channel")
    W = synth.make_w("channel")[:, :64]
    idx = O.detect_outliers(X, 6.0)
    Xq, ax = O.quantize_activations(X[:128], idx)
    Wq, aw = O.quantize_weight(W)
    A = O.int_gemm(Xq, Wq)
    ref = Xq.astype(np.int64) @ Wq.astype(np.int64)  # numpy integer matmul
    assert np.array_equal(A.astype(np.int64), ref)
    # largest possible accumulator stays exact
    big = np.full((2, 12288), 127, np.int8)
    big[1] = -127
    A2 = O.int_gemm(big, big.T.copy())
    assert A2[0, 0] == 16129 * 12288 and A2[0, 1] == -16129 * 12288


def test_sampled_equals_full():
    X, W, _, _ = synth.make("tiny")
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, 6.0)
    rows = np.array([0, 5, 15])
    cols = np.array([1, 17, 200, 255])
    s = O.mixed_matmul_sampled(X, W, 6.0, rows, cols)
    assert np.array_equal(s["A"], r.A[np.ix_(rows, cols)])
    assert np.array_equal(s["Y16"].view(np.uint16), r.Y16[np.ix_(rows, cols)].view(np.uint16))
    assert np.array_equal(s["Wq"], Wq[:, cols]) and np.array_equal(s["Xq"], r.Xq[rows])


def test_synth_deterministic():
    a = synth.make("tiny")
    b = synth.make("tiny")
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u), np.asarray(v))
    X4, d4, r4 = synth.make_x("qkv175b_decode")
    assert X4.shape == (32, 12288) and d4.size == 7 and r4.size == 24


def test_weight_absmax_closed_forms():
    """Column absmax of W over all K rows: the planted largest magnitude of
    each column (either sign, any row) is its absmax; an empty column is 0."""
    rng = np.random.default_rng(8)
    K, N = 37, 11
    W = (rng.uniform(-0.5, 0.5, (K, N))).astype(np.float16)
    rows = rng.integers(0, K, N)
    mags = np.linspace(1.0, 3.5, N).astype(np.float16)
    W[rows, np.arange(N)] = np.where(np.arange(N) % 2 == 0, -mags, mags)
    assert np.array_equal(O.weight_absmax(W), mags.astype(np.float32))
    assert np.array_equal(O.weight_absmax(W.T.copy().T), mags.astype(np.float32))
    assert O.weight_absmax(np.zeros((0, 5), np.float16)).tolist() == [0.0] * 5
    assert np.array_equal(O.weight_absmax(W), O.quantize_weight(W)[1])


@pytest.mark.parametrize("block", [1, 64, 100, 4096])
def test_column_blocks_equal_full(block):
    """The column-blocked evaluation is the full one cut into pieces: the
    same outlier list, constants and int32 accumulators bit for bit, and
    the same fp64 output (up to the summation order of the short fp16
    product)."""
    X, W, _ = synth.random_case(606, 37, 192, 272, 5)
    b = synth.random_bias(607, 272)
    Wq, aw = O.quantize_weight(W)
    r = O.mixed_matmul(X, Wq, aw, W, 6.0, bias=b)
    seen = 0
    for c0, c1, blk in O.mixed_matmul_col_blocks(X, W, 6.0, block, bias=b):
        assert c0 == seen and c1 > c0
        seen = c1
        assert np.array_equal(blk["idx"], r.idx)
        assert np.array_equal(blk["x_absmax"], r.x_absmax)
        assert np.array_equal(blk["w_absmax"], aw[c0:c1])
        assert np.array_equal(blk["A"], r.A[:, c0:c1])
        assert np.allclose(blk["Y64"], r.Y64[:, c0:c1], rtol=1e-13, atol=1e-13)
    assert seen == 272

