"""int8_mixed_matmul_noalloc: the matmul whose workspace is the library's
static per-device scratch array, for callers that cannot allocate.  Checked
against int8_mixed_matmul (the same kernels on a caller workspace) bit for
bit and against the oracle within tolerance, on consecutive calls that
share the array, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import synth
import int8_mixed_precision_outlier_amd as i8

TOL = 2e-3
SCRATCH = 64 << 20  # INT8MM_NOALLOC_SCRATCH_BYTES


def y_err(Y16, Y64):
    Y = np.asarray(Y16, dtype=np.float64)
    tau = 1e-2 * np.sqrt(np.mean(Y64 ** 2))
    return float(np.max(np.abs(Y - Y64) / np.maximum(np.abs(Y64), tau)))


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """Checked on the host before any launch: a shape whose workspace exceeds
    the static array is INT8MM_ESCRATCH; bad shapes are rejected as by
    int8_mixed_matmul."""
    lib = i8.load()
    f = ctypes.c_float(6.0)
    assert lib.int8_mixed_matmul_workspace_size(4096, 12288, 49152, 12288, None) > SCRATCH
    assert lib.int8_mixed_matmul_noalloc(None, 4096, 12288, None, None, None, 49152, f, None,
                                         None, 12288, None) == i8.STATUS_ESCRATCH
    assert lib.int8_mixed_matmul_workspace_size(4096, 12288, 49152, 128, None) <= SCRATCH
    assert lib.int8_mixed_matmul_noalloc(None, 16, 24, None, None, None, 32, f, None, None, 0,
                                         None) == i8.STATUS_EINVAL  # K % 16 != 0: no size
    assert lib.int8_mixed_matmul_noalloc(None, 16, 64, None, None, None, 32, f, None, None, 65,
                                         None) == i8.STATUS_EINVAL  # n_cap > K
    assert lib.int8_mixed_matmul_noalloc(None, 0, 64, None, None, None, 32, f, None, None, 64,
                                         None) == i8.STATUS_OK  # M == 0: no-op


CALLS = [  # (M, K, N, planted outliers, alpha, n_cap, bias): each workspace smaller than the last
    (2048, 256, 20480, 7, 6.0, 256, True),   # columns split between two tile sizes
    (300, 2048, 4096, 9, 6.0, 256, True),    # 128x128 tiles
    (64, 5120, 15360, 6, 6.0, 64, True),     # decode, four token blocks per wavefront
    (48, 6400, 12288, 7, 6.0, 64, False),    # decode, three token blocks; two quantizer waves per row
    (24, 1024, 2048, 5, 6.0, 64, False),     # decode, up to 32 tokens
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    """Calls in a row on the shared array, each needing less of it than the
    one before (tiled, column-split and decode paths): each Y is
    bit-identical to int8_mixed_matmul's on a fresh workspace and within
    tolerance of the oracle."""
    assert torch.cuda.is_available()
    for case, (M, K, N, nout, alpha, n_cap, with_bias) in enumerate(CALLS):
        print(f"[noalloc] call {case}: M={M} K={K} N={N} n_cap={n_cap}", flush=True)
        X, W, _ = synth.random_case(4700 + case, M, K, N, nout)
        b = synth.random_bias(4800 + case, N) if with_bias else None
        Xd = torch.from_numpy(X).cuda()
        Wd = torch.from_numpy(W).cuda()
        bd = torch.from_numpy(b).cuda() if b is not None else None
        Wi8, wabs = i8.quantize_weight(Wd)
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        i8.mixed_matmul_noalloc(Xd, Wi8, wabs, Wd, Y, alpha=alpha, bias=bd, n_cap=n_cap)
        ws = torch.full((i8.workspace_size(M, K, N, n_cap),), 0x5A, dtype=torch.uint8,
                        device="cuda")
        ref = i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=alpha, bias=bd, n_cap=n_cap,
                              workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), case
        Wq, aw = O.quantize_weight(W)
        r = O.mixed_matmul(X, Wq, aw, W, alpha, bias=b)
        assert y_err(Y.cpu().numpy(), r.Y64) <= TOL, case
