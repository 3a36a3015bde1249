"""CPU oracle for the LLM.int8() mixed-precision decomposed matmul.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP kernels.

Pages cited (by title and section):
  [JS]  "LLM.int8() — 大模型激活值里藏着几个超大异常通道", Jason's Study
        (estelledc.github.io/study/papers/llm-int8-2022/).
  [ALI] "AI 十大核心论文解读系列 — LLM.int8()", developer.aliyun.com
        article 1691675.
  [KD]  "論文閱讀 : LLM.int8(): 8-bit Matrix Multiplication for Transformers
        at Scale", hackmd.io/@KuoDong.
  [GB]  "LLM.int8()", brain.gartu.xyz (IA / LLM / quantification).
  [MD]  "LLM.int8() — 스케일 트랜스포머의 8-bit 행렬곱", moduai.site.

What the method computes (Y = X.W, X fp16 [M,K] activations, W fp16 [K,N]):
  1. Outlier columns: column j of X is an outlier feature iff some
     |X[i,j]| > alpha (alpha = 6.0 by default) -- [JS 方法 2],
     [GB "Seuil de détection α"].
  2. Decomposition: the outlier columns of X and the matching rows of W go
     through an fp16 matmul; everything else is quantized to int8 --
     [ALI §2.2 and 图2], [GB "La solution : Décomposition Mixed-Precision"].
  3. Vector-wise quantization: one constant per row of X, c_x[i], and one per
     column of W, c_w[j], each 127 / absmax of that vector -- [JS 方法 1],
     [KD 向量級量化], [GB "Vector-wise INT8 Quantization"].
  4. int8 x int8 matmul with int32 accumulation, dequantized by the outer
     product of the constants: Out_i32[i,j] / (c_x[i] c_w[j]) -- [ALI 图2],
     [JS 方法 1].
  5. Y = dequantized int8 result + X_out . W_out, output in fp16 --
     [JS 方法 2], [ALI 图2].

Readings taken where the pages are silent, garbled or disagree:
  R1  Strict ">" against alpha (the runtime rule of [JS 方法 2] and
      [GB "Seuil de détection α"]); [KD]'s ">= 6" is its analysis
      definition.  The comparison is made in fp32 with alpha rounded to fp32.
  R2  Detection runs over all M rows of the call, on every call.
  R3  A row's absmax c_x is taken over its non-outlier columns only (the
      pages decompose first, then quantize what is left).
  R4  A column's absmax c_w is taken over all K rows of W (weights are
      quantized once, before any activation is seen); rows of outlier dims
      meet zeros in the int8 activations and add nothing.
  R5  Scale = 127/absmax, symmetric range [-127, 127] ([GB]'s formulas drop
      the 127 factor and [JS 案例 1] writes the range as -128..127; -128 is
      never produced).
  R6  Rounding: s = RN32(127/absmax), q = RNE(RN32(x*s)), i.e. fp32 ops with
      round-to-nearest-even and a round-half-to-even integer rounding.
  R7  An all-zero vector (absmax 0) gets s = 0 and q = 0.
  R8  Dequantization uses the exact constants (absmax/127, not 1/s).  The
      fp16 path multiplies fp16 values exactly and accumulates in fp64; the
      sum of the two paths is rounded once to fp16.
  R9  Non-finite inputs are outside the method's domain.
  R11 Memory-lean weights: only the fp16 rows of a static set of outlier
      dims are kept ([JS 观察 2]; [ALI §2.2]).  A runtime outlier outside
      that set takes its int8 row dequantized to fp16, RN16(RN32(q *
      RN32(aw/127))), in the fp16 path; the pages define no such case, so
      the call reports it.
  R10 The optional layer bias ([GB "Exemple pratique"]: the int8 layer is a
      drop-in for a linear layer with bias) is fp16 [N], added to every
      output row in full precision before the single rounding to fp16.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "weight_absmax", "quantize_weight", "detect_outliers", "row_absmax",
    "quantize_activations", "gather_outliers", "int_gemm", "dequant_sum",
    "mixed_matmul", "mixed_matmul_sampled", "mixed_matmul_col_blocks", "tensorwise_quantize",
    "dequant_weight_rows", "gather_outliers_cached", "mixed_matmul_cached",
    "MixedResult",
]

_127 = np.float32(127.0)


def _abs32(a) -> np.ndarray:
    """|a| as float32; fp16 -> fp32 and abs are both exact."""
    return np.abs(np.asarray(a, dtype=np.float16).astype(np.float32))


def _scale(absmax: np.ndarray) -> np.ndarray:
    """s = RN32(127 / absmax), 0 where absmax == 0 (readings R5-R7)."""
    absmax = np.asarray(absmax, dtype=np.float32)
    s = np.zeros_like(absmax)
    nz = absmax > 0
    s[nz] = _127 / absmax[nz]  # IEEE float32 division: correctly rounded
    return s


def _round_q(x32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """q = clamp(RNE(RN32(x*s)), -127, 127) as int8 (reading R6)."""
    prod = np.multiply(x32, s32, dtype=np.float32)
    q = np.rint(prod)  # round half to even
    return np.clip(q, -127, 127).astype(np.int8)


# ---------------------------------------------------------------- weights

def weight_absmax(W16) -> np.ndarray:
    """absmax of every column of W over all K rows -> float32 [N] (R4); an
    empty column (K = 0) has absmax 0 (R7)."""
    W32 = _abs32(W16)
    if W32.shape[0] == 0:
        return np.zeros(W32.shape[1], np.float32)
    return W32.max(axis=0)


def quantize_weight(W16):
    """Vector-wise int8 weights [JS 方法 1: one constant per column of B].

    Returns (Wq int8 [K,N], w_absmax float32 [N]).  c_w[j] = 127/w_absmax[j].
    """
    W32 = np.asarray(W16, dtype=np.float16).astype(np.float32)
    aw = np.abs(W32).max(axis=0) if W32.shape[0] else np.zeros(W32.shape[1], np.float32)
    s = _scale(aw)
    return _round_q(W32, s[None, :]), aw.astype(np.float32)


# ------------------------------------------------------------ activations

def detect_outliers(X16, alpha) -> np.ndarray:
    """Ascending int32 indices j with max_i |X[i,j]| > alpha (R1, R2).

    [JS 方法 2]: a column with any element of magnitude above the threshold
    goes to the fp16 path; [GB "Seuil de détection α"]: max(|X[:,j]|) > α.
    """
    X32 = _abs32(X16)
    a32 = np.float32(alpha)
    if X32.shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    colmax = X32.max(axis=0)
    return np.nonzero(colmax > a32)[0].astype(np.int32)


def row_absmax(X16, idx) -> np.ndarray:
    """absmax of each row of X over its non-outlier columns (R3) -> f32 [M]."""
    X32 = _abs32(X16)
    keep = np.ones(X32.shape[1], dtype=bool)
    keep[np.asarray(idx, dtype=np.int64)] = False
    if X32.shape[0] == 0:
        return np.zeros(0, np.float32)
    sub = X32[:, keep]
    if sub.shape[1] == 0:
        return np.zeros(X32.shape[0], np.float32)
    return sub.max(axis=1)


def quantize_activations(X16, idx):
    """Vector-wise int8 activations with the outlier columns removed.

    [JS 方法 1]: one constant c_x[i] per row of the input; [ALI 图2]: the
    large-magnitude columns are split off before the 8-bit path.  Outlier
    columns of the returned int8 matrix are 0.
    Returns (Xq int8 [M,K], x_absmax float32 [M]).
    """
    X32 = np.asarray(X16, dtype=np.float16).astype(np.float32)
    ax = row_absmax(X16, idx)
    s = _scale(ax)
    q = _round_q(X32, s[:, None])
    q[:, np.asarray(idx, dtype=np.int64)] = 0
    return q, ax


def gather_outliers(X16, W16, idx):
    """Dense fp16 outlier sub-matrices [ALI 图2]: X_out = X[:, idx] [M,n],
    W_out = W[idx, :] [n,N]."""
    idx = np.asarray(idx, dtype=np.int64)
    X16 = np.asarray(X16, dtype=np.float16)
    W16 = np.asarray(W16, dtype=np.float16)
    return X16[:, idx].copy(), W16[idx, :].copy()


# ------------------------------------------------------------------ GEMMs

def int_gemm(Xq, Wq) -> np.ndarray:
    """Out_i32 = Xq . Wq, exact [ALI 图2: the 8-bit matmul output Out_i32].

    Evaluated as an fp64 BLAS product of the int8 values: every partial sum
    is an integer of magnitude <= 127*127*K < 2^53, so no rounding occurs in
    any summation order.  Result is int32 (|A| <= 16129*K < 2^31 needs
    K <= 133144).
    """
    Xq = np.asarray(Xq, dtype=np.int8)
    Wq = np.asarray(Wq, dtype=np.int8)
    K = Xq.shape[1]
    if K > 133144:
        raise ValueError("K too large for an exact int32 accumulator")
    acc = Xq.astype(np.float64) @ Wq.astype(np.float64)
    return acc.astype(np.int64).astype(np.int32)


def dequant_sum(A, x_absmax, w_absmax, X_out, W_out, bias=None) -> np.ndarray:
    """Y64 = A / (c_x (x) c_w) + X_out . W_out (+ bias) in fp64 (R8, R10).

    [JS 方法 1]: Out[i,j] = (A_int8 . B_int8)[i,j] / (c_x[i] c_w[j]);
    [JS 方法 2]: Y = that + X_fp16 . W_fp16.  With c = 127/absmax the
    division is A * (absmax_x/127) * (absmax_w/127).  The layer of [GB
    "Exemple pratique"] carries an optional fp16 bias [N], added to every
    output row before the single rounding to fp16 (R10).
    """
    rx = np.asarray(x_absmax, dtype=np.float64) / 127.0
    rw = np.asarray(w_absmax, dtype=np.float64) / 127.0
    y = np.asarray(A, dtype=np.float64) * rx[:, None] * rw[None, :]
    Xo = np.asarray(X_out, dtype=np.float16).astype(np.float64)
    Wo = np.asarray(W_out, dtype=np.float16).astype(np.float64)
    if Xo.shape[1]:
        y = y + Xo @ Wo
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    return y


@dataclass
class MixedResult:
    idx: np.ndarray        # int32 [n]   ascending outlier columns
    Xq: np.ndarray         # int8  [M,K] (zeros at outlier columns)
    x_absmax: np.ndarray   # f32   [M]
    X_out: np.ndarray      # f16   [M,n]
    W_out: np.ndarray      # f16   [n,N]
    A: np.ndarray          # int32 [M,N] Out_i32
    Y64: np.ndarray        # f64   [M,N] the decomposition, unrounded
    Y16: np.ndarray        # f16   [M,N] RNE(Y64)


def mixed_matmul(X16, Wq, w_absmax, W16, alpha=6.0, bias=None) -> MixedResult:
    """The whole decomposed matmul, step by step ([ALI 图2] order).

    Wq/w_absmax come from quantize_weight (done once, offline); W16 is the
    fp16 weight the outlier rows are read from; bias is an optional fp16 [N].
    """
    idx = detect_outliers(X16, alpha)
    Xq, ax = quantize_activations(X16, idx)
    X_out, W_out = gather_outliers(X16, W16, idx)
    A = int_gemm(Xq, Wq)
    Y64 = dequant_sum(A, ax, w_absmax, X_out, W_out, bias)
    return MixedResult(idx, Xq, ax, X_out, W_out, A, Y64, Y64.astype(np.float16))


def mixed_matmul_sampled(X16, W16, alpha, rows, cols, bias=None):
    """The same computation restricted to output rows x cols.

    Every quantity is computed exactly as in mixed_matmul: detection over all
    of X, row constants over the full rows, column constants over the full
    columns of W; only the outputs outside rows x cols are skipped.
    Returns a dict with idx, Xq/x_absmax (sampled rows), Wq/w_absmax
    (sampled cols), A, Y64, Y16 [len(rows), len(cols)].
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    X16 = np.asarray(X16, dtype=np.float16)
    idx = detect_outliers(X16, alpha)
    Xs = X16[rows]
    Xq, ax = quantize_activations(Xs, idx)
    Wc = np.asarray(W16, dtype=np.float16)[:, cols]
    Wq, aw = quantize_weight(Wc)
    X_out, W_out = gather_outliers(Xs, Wc, idx)
    A = int_gemm(Xq, Wq)
    Y64 = dequant_sum(A, ax, aw, X_out, W_out,
                      None if bias is None else np.asarray(bias, dtype=np.float16)[cols])
    return dict(idx=idx, Xq=Xq, x_absmax=ax, Wq=Wq, w_absmax=aw, A=A,
                X_out=X_out, W_out=W_out, Y64=Y64, Y16=Y64.astype(np.float16))


def mixed_matmul_col_blocks(X16, W16, alpha, block=4096, bias=None):
    """The whole decomposed matmul with its output produced one block of
    output columns at a time, for shapes whose full fp64 product does not
    fit comfortably in memory.  Detection, the row constants and the int8
    activations are computed once over all of X, exactly as in
    mixed_matmul; a column's weight constant depends on that column alone,
    so quantizing W one column block at a time gives the same Wq and
    w_absmax.  Yields (c0, c1, dict(idx, x_absmax, w_absmax, A, Y64)) for
    columns c0..c1-1."""
    X16 = np.asarray(X16, dtype=np.float16)
    W16 = np.asarray(W16, dtype=np.float16)
    idx = detect_outliers(X16, alpha)
    Xq, ax = quantize_activations(X16, idx)
    X_out = X16[:, np.asarray(idx, dtype=np.int64)].copy()
    N = W16.shape[1]
    for c0 in range(0, N, block):
        c1 = min(N, c0 + block)
        Wc = W16[:, c0:c1]
        Wq, aw = quantize_weight(Wc)
        W_out = Wc[np.asarray(idx, dtype=np.int64), :]
        A = int_gemm(Xq, Wq)
        b = None if bias is None else np.asarray(bias, dtype=np.float16)[c0:c1]
        yield c0, c1, dict(idx=idx, x_absmax=ax, w_absmax=aw, A=A,
                           Y64=dequant_sum(A, ax, aw, X_out, W_out, b))


# ------------------------------------------- static outlier-row cache

def dequant_weight_rows(Wq, w_absmax, dims) -> np.ndarray:
    """fp16 rows rebuilt from the int8 weights: RN16(RN32(Wq[k,j] *
    RN32(aw[j]/127))) for each k in dims (reading R11: the stand-in for an
    outlier row that is not in the fp16 cache)."""
    dims = np.asarray(dims, dtype=np.int64)
    r = np.asarray(w_absmax, dtype=np.float32) / np.float32(127.0)
    rows = np.asarray(Wq, dtype=np.int8)[dims].astype(np.float32) * r[None, :]
    return rows.astype(np.float16)


def gather_outliers_cached(X16, Wq, w_absmax, cache_dims, W_cache, idx):
    """X_out = X[:, idx]; W_out row t = the cached fp16 row of dim idx[t]
    when idx[t] is one of cache_dims, else the dequantized int8 row (R11).

    [JS 观察 2]: the outlier dims are few and fixed across tokens and
    batches, so their fp16 weight rows can be kept once (W_cache =
    W[cache_dims, :]) instead of the whole fp16 W; [ALI §2.2] puts the
    extra memory at about 0.1 %.  Returns (X_out, W_out, missed) where
    missed lists the outlier dims absent from the cache.
    """
    idx = np.asarray(idx, dtype=np.int64)
    cache_dims = np.asarray(cache_dims, dtype=np.int64)
    pos = {int(k): s for s, k in enumerate(cache_dims)}
    W_cache = np.asarray(W_cache, dtype=np.float16)
    N = np.asarray(Wq).shape[1]
    W_out = np.zeros((idx.size, N), dtype=np.float16)
    missed = [int(k) for k in idx if int(k) not in pos]
    for t, k in enumerate(idx):
        if int(k) in pos:
            W_out[t] = W_cache[pos[int(k)]]
    if missed:
        rows = dequant_weight_rows(Wq, w_absmax, missed)
        for r, k in zip(rows, missed):
            W_out[int(np.searchsorted(idx, k))] = r
    X16 = np.asarray(X16, dtype=np.float16)
    return X16[:, idx].copy(), W_out, np.asarray(missed, dtype=np.int32)


def mixed_matmul_cached(X16, Wq, w_absmax, cache_dims, W_cache, alpha=6.0, bias=None):
    """The decomposed matmul with the fp16 weights held only as a cache of
    outlier rows (gather_outliers_cached).  Detection is unchanged (R2);
    with every detected outlier in the cache the result is exactly that of
    mixed_matmul.  Returns (MixedResult, missed)."""
    idx = detect_outliers(X16, alpha)
    Xq, ax = quantize_activations(X16, idx)
    X_out, W_out, missed = gather_outliers_cached(X16, Wq, w_absmax, cache_dims, W_cache, idx)
    A = int_gemm(Xq, Wq)
    Y64 = dequant_sum(A, ax, w_absmax, X_out, W_out, bias)
    return MixedResult(idx, Xq, ax, X_out, W_out, A, Y64, Y64.astype(np.float16)), missed


# --------------------------------------------------- tensor-wise baseline

def tensorwise_quantize(X16):
    """Tensor-wise absmax int8 (one constant for the whole tensor).

    This is the failure mode of [JS 案例 1]: the single largest magnitude
    sets the step for every channel.  Not part of the decomposed path; kept
    here only to reproduce that worked example.
    Returns (q int8, absmax float32, dequantized float64).
    """
    X32 = np.asarray(X16, dtype=np.float16).astype(np.float32)
    amax = np.float32(np.abs(X32).max()) if X32.size else np.float32(0)
    s = _scale(np.array([amax], dtype=np.float32))[0]
    q = _round_q(X32, s)
    deq = q.astype(np.float64) * (float(amax) / 127.0)
    return q, amax, deq
