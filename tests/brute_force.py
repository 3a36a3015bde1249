"""Pure-Python brute force of the decomposed matmul, for tiny inputs only.

A second, independent derivation used to pin the numpy oracle: explicit
loops, Python integers for the int8 product and exact rationals
(fractions.Fraction) for the output, with no numpy arithmetic at all.

fp32 rounding is emulated by computing one operation in Python's binary64
and rounding the result to binary32 with struct: for a single +, -, x or /
of binary32 operands, binary64 has more than 2*24+2 bits, so this double
rounding always equals the correctly rounded binary32 result.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _rne(v: float) -> int:
    # Python's round() on a float rounds half to even.
    return int(round(v))


def f16(x: float) -> float:
    return struct.unpack("<e", struct.pack("<e", x))[0]


def brute(X, W, alpha, bias=None, cache_dims=None):
    """X: list of rows of Python floats (fp16 values), W: K rows of N floats,
    bias: None or N floats added to every output row, cache_dims: None (the
    fp16 rows of every outlier are available) or the dims whose fp16 rows
    are cached; any other outlier uses its int8 row dequantized to fp16.

    Returns a dict with idx, Xq, ax, Wq, aw, A, Yexact (Fractions).
    """
    M = len(X)
    K = len(W)
    N = len(W[0]) if K else 0
    a = f32(alpha)
    # outlier columns: any |x| > alpha, compared in binary32
    idx = [j for j in range(K) if any(abs(X[i][j]) > a for i in range(M))]
    out = set(idx)
    # weights: column absmax over all K rows
    aw = []
    Wq = [[0] * N for _ in range(K)]
    for j in range(N):
        m = 0.0
        for k in range(K):
            m = max(m, abs(W[k][j]))
        aw.append(m)
        s = f32(127.0 / m) if m > 0 else 0.0
        for k in range(K):
            Wq[k][j] = max(-127, min(127, _rne(f32(W[k][j] * s))))
    # activations: row absmax over non-outlier columns
    ax = []
    Xq = [[0] * K for _ in range(M)]
    for i in range(M):
        m = 0.0
        for k in range(K):
            if k not in out:
                m = max(m, abs(X[i][k]))
        ax.append(m)
        s = f32(127.0 / m) if m > 0 else 0.0
        for k in range(K):
            if k not in out:
                Xq[i][k] = max(-127, min(127, _rne(f32(X[i][k] * s))))
    # int8 x int8 -> exact integer accumulator
    A = [[sum(Xq[i][k] * Wq[k][j] for k in range(K)) for j in range(N)]
         for i in range(M)]
    # exact decomposition: A/(c_x c_w) + X_out W_out
    Y = []
    for i in range(M):
        row = []
        for j in range(N):
            v = Fraction(A[i][j]) * Fraction(ax[i]) * Fraction(aw[j]) / (127 * 127)
            for t in idx:
                if cache_dims is None or t in cache_dims:
                    w = W[t][j]
                else:  # int8 row dequantized: q * (aw/127) in binary32, then binary16
                    w = f16(f32(Wq[t][j] * f32(aw[j] / 127.0)))
                v += Fraction(X[i][t]) * Fraction(w)
            if bias is not None:
                v += Fraction(bias[j])
            row.append(v)
        Y.append(row)
    return dict(idx=idx, Xq=Xq, ax=ax, Wq=Wq, aw=aw, A=A, Yexact=Y)


def exact_product(X, W):
    """Exact X.W as Fractions (the un-quantized reference)."""
    M, K = len(X), len(W)
    N = len(W[0]) if K else 0
    return [[sum((Fraction(X[i][k]) * Fraction(W[k][j]) for k in range(K)), Fraction(0))
             for j in range(N)] for i in range(M)]


def is_finite(v) -> bool:
    return not (math.isinf(v) or math.isnan(v))
