"""GPU parity of the two stage exports (int8_detect_outliers,
int8_quantize_activations) against the CPU oracle, through the C-ABI.

Every result here is integer or byte work (column absmax, outlier mask and
list, header, row absmax, int8 activations, gathered fp16 outliers), so
every comparison is bit-exact.  The workspace starts filled with a garbage
byte pattern, so a field the stage fails to write shows up.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import int8_mixed_precision_outlier_amd as i8
from packing import unpack

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def garbage_ws(M, K, N, n_cap):
    return torch.full((i8.workspace_size(M, K, N, n_cap),), 0xA5, dtype=torch.uint8,
                      device="cuda")


def mask_words(idx, K):
    m = np.zeros((K + 31) // 32, dtype=np.uint32)
    for k in idx:
        m[k // 32] |= np.uint32(1) << np.uint32(k % 32)
    return m.view(np.int32)


CASES = [  # (M, K, N, n_out, alpha, n_cap)
    (1, 64, 48, 1, 6.0, 64),
    (17, 48, 272, 3, 6.0, 48),
    (33, 4112, 80, 65, 6.0, 100),
    (300, 1040, 784, 63, 6.0, 64),
    (513, 512, 304, 100, 6.0, 512),
    (64, 160, 64, 0, float("inf"), 0),
    (70, 32, 32, 4, 0.0, 32),
    # two-pass column absmax (M > 512, M*K >= 2^25), ragged in both
    (1000, 40000, 64, 5, 6.0, 64),
    # rows of 6145-12288 columns: two quantizer wavefronts per row, the
    # second ragged; then just past that form (one workgroup per row)
    (100, 8208, 48, 7, 6.0, 64),
    (47, 12288, 32, 9, 6.0, 64),
    (40, 12304, 32, 7, 6.0, 32),
]


@pytest.mark.parametrize("M,K,N,nout,alpha,n_cap", CASES)
def test_stages_match_oracle(M, K, N, nout, alpha, n_cap):
    print(f"[stages] M={M} K={K} N={N} nout={nout} alpha={alpha} n_cap={n_cap}", flush=True)
    X, W, _ = synth.random_case(M * 7919 + K * 31 + N, M, K, N, nout)
    Xd, Wd = dev(X), dev(W)
    ws = garbage_ws(M, K, N, n_cap)
    i8.detect_outliers(Xd, ws, alpha=alpha, n_cap=n_cap)
    torch.cuda.synchronize()
    idx = O.detect_outliers(X, alpha)
    g = i8.read_workspace(ws, M, K, N, n_cap)
    assert g["status"] == 0 and g["n"] == idx.size and g["n_found"] == idx.size
    assert np.array_equal(g["idx"].cpu().numpy(), idx)
    assert np.array_equal(g["mask"].cpu().numpy(), mask_words(idx, K))
    colmax = np.abs(X.astype(np.float32)).max(axis=0)
    assert np.array_equal(g["colmax"].cpu().numpy(), colmax)

    i8.quantize_activations(Xd, Wd, ws, n_cap=n_cap)
    torch.cuda.synchronize()
    Xq, ax = O.quantize_activations(X, idx)
    X_out, W_out = O.gather_outliers(X, W, idx)
    g = i8.read_workspace(ws, M, K, N, n_cap)
    assert g["status"] == 0 and np.array_equal(g["idx"].cpu().numpy(), idx)
    assert np.array_equal(unpack(g["X_i8"].cpu().numpy(), M, K)[:M, :K], Xq)
    assert np.array_equal(g["x_absmax"].cpu().numpy(), ax)
    n, npad = idx.size, (idx.size + 15) // 16 * 16
    ob = g["X_out"].shape[1]
    xo = np.ascontiguousarray(unpack(g["X_out"].cpu().numpy(), M, ob)).view(np.uint16)
    wo = np.ascontiguousarray(unpack(g["W_outT"].cpu().numpy(), N, ob)).view(np.uint16)
    assert np.array_equal(xo[:M, :n], X_out.view(np.uint16)) and not xo[:M, n:npad].any()
    assert np.array_equal(wo[:, :n], W_out.T.view(np.uint16)) and not wo[:, n:npad].any()


def test_staged_equals_fused():
    """Stage 1 + stage 2 leave the same intermediates as the fused call, and
    the fused call's Y is unchanged by running on their workspace."""
    M, K, N, n_cap = 130, 2048, 512, 256
    X, W, _ = synth.random_case(4242, M, K, N, 11)
    Xd, Wd = dev(X), dev(W)
    Wi8, wabs = i8.quantize_weight(Wd)
    ws_f, ws_s = garbage_ws(M, K, N, n_cap), garbage_ws(M, K, N, n_cap)
    Y = i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=6.0, n_cap=n_cap, workspace=ws_f)
    i8.detect_outliers(Xd, ws_s, alpha=6.0, n_cap=n_cap)
    i8.quantize_activations(Xd, Wd, ws_s, n_cap=n_cap)
    torch.cuda.synchronize()
    f = i8.read_workspace(ws_f, M, K, N, n_cap)
    s = i8.read_workspace(ws_s, M, K, N, n_cap)
    assert f["n"] == s["n"] == 11 and f["status"] == s["status"] == 0
    npad = (f["n"] + 15) // 16 * 16
    for k in ("colmax", "mask", "idx", "x_absmax", "X_i8"):
        assert torch.equal(f[k], s[k]), k
    ob = f["X_out"].shape[1]
    for k, rows in (("X_out", M), ("W_outT", N)):
        a = np.ascontiguousarray(unpack(f[k].cpu().numpy(), rows, ob)).view(np.uint16)
        b = np.ascontiguousarray(unpack(s[k].cpu().numpy(), rows, ob)).view(np.uint16)
        assert np.array_equal(a[:rows, :npad], b[:rows, :npad]), k


def test_detect_capacity_overflow():
    M, K, N = 48, 128, 64
    X, W, _ = synth.random_case(5, M, K, N, 9)
    ws = garbage_ws(M, K, N, 4)
    i8.detect_outliers(dev(X), ws, alpha=6.0, n_cap=4)
    torch.cuda.synchronize()
    g = i8.read_workspace(ws, M, K, N, 4)
    idx = O.detect_outliers(X, 6.0)
    assert idx.size == 9
    assert g["status"] == 1 and g["n"] == 4 and g["n_found"] == 9
    assert np.array_equal(g["idx"].cpu().numpy(), idx[:4])


@pytest.mark.parametrize("K,N,nout,alpha", [(64, 48, 1, 6.0), (12288, 256, 7, 6.0),
                                            (4112, 80, 30, 6.0), (48, 32, 4, 0.0),
                                            (256, 64, 0, float("inf"))])
def test_one_row_call_fills_detector_fields(K, N, nout, alpha):
    """A one-row call derives the outlier mask inside the quantizer (no
    detection launch); the detector's fields it writes on the way, column
    absmax and mask, match the oracle bit for bit, as do the list and the
    header."""
    M, n_cap = 1, K
    X, W, _ = synth.random_case(K * 13 + nout, M, K, N, nout)
    Xd, Wd = dev(X), dev(W)
    Wi8, wabs = i8.quantize_weight(Wd)
    ws = garbage_ws(M, K, N, n_cap)
    i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=alpha, n_cap=n_cap, workspace=ws)
    torch.cuda.synchronize()
    idx = O.detect_outliers(X, alpha)
    g = i8.read_workspace(ws, M, K, N, n_cap)
    assert g["status"] == 0 and g["n"] == idx.size and g["n_found"] == idx.size
    assert np.array_equal(g["idx"].cpu().numpy(), idx)
    assert np.array_equal(g["mask"].cpu().numpy(), mask_words(idx, K))
    assert np.array_equal(g["colmax"].cpu().numpy(), np.abs(X.astype(np.float32)).max(axis=0))


@pytest.mark.parametrize("M", [1, 40])
def test_quantize_without_weights_when_n_is_zero(M):
    """int8_quantize_activations with N = 0 and no weight matrix (NULL, which
    the validator accepts for an empty W) and outliers present: nothing reads
    weight rows; the activations' results match the oracle bit for bit."""
    K, n_cap = 256, 256
    X, _, _ = synth.random_case(4600 + M, M, K, 16, 5)
    Xd = dev(X)
    W0 = torch.empty((K, 0), dtype=torch.float16, device="cuda")
    ws = garbage_ws(M, K, 0, n_cap)
    i8.detect_outliers(Xd, ws, alpha=6.0, n_cap=n_cap)
    i8.quantize_activations(Xd, W0, ws, n_cap=n_cap)
    torch.cuda.synchronize()
    idx = O.detect_outliers(X, 6.0)
    assert idx.size > 0
    g = i8.read_workspace(ws, M, K, 0, n_cap)
    assert g["status"] == 0 and np.array_equal(g["idx"].cpu().numpy(), idx)
    Xq, ax = O.quantize_activations(X, idx)
    assert np.array_equal(g["x_absmax"].cpu().numpy(), ax)
    assert np.array_equal(unpack(g["X_i8"].cpu().numpy(), M, K)[:M, :K], Xq)
