"""Seeded synthetic workloads for the int8 mixed-precision outlier matmul.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no thresholds, no scales, no rounding to int8).
Both the CPU oracle's tests and the GPU path's tests/bench take their inputs
from here, so the two sides see identical bytes.

The activation statistics follow what the pages report about emergent
outlier features:
  * "LLM.int8() — 大模型激活值里藏着几个超大异常通道" (estelledc.github.io,
    案例 1): in one OPT-13B FFN input, 4095 ordinary channels have mean
    magnitude 0.5 and maximum 5, while 7 outlier channels have mean 65 and
    maximum 130.
  * developer.aliyun.com article 1691675 (§2.1): at most 7 outlier feature
    dimensions, covering 75 % of the sequence dimension, about 20x the
    ordinary magnitude.
  * hackmd.io/@KuoDong "論文閱讀 : LLM.int8()" (混合精度處理): the outliers
    sit in as few as 6 dimensions and cover about 75 % of positions.
The pages' own measurements use trained OPT/BLOOM models and text corpora;
those are replaced here by draws with the same shape, magnitude and
sparsity structure.

Recipe (all draws from one numpy PCG64 generator, seed = 1000 + config
number, in this order): outlier dims, outlier rows, X normals, outlier
magnitudes, outlier signs, W.  X normals are drawn in float64, clipped and
cast to fp16 (round-to-nearest-even).  W ~ N(0, 0.02^2) is drawn in float32
row blocks and cast to fp16.  "In 75 % of rows" is one shared random subset
of round(0.75*M) rows for all outlier dims.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_x", "make_w", "make", "sha256", "device_normal",
           "device_case_x"]

W_STD = 0.02
_W_ROW_BLOCK = 512


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic call Y[M,N] = X[M,K] . W[K,N]."""

    number: int            # 1..5; the generator seed is 1000 + number
    name: str
    M: int
    K: int
    N: int
    normal_std: float      # std of the ordinary activations before clipping
    clip: float            # ordinary activations are clipped to +-clip
    n_outlier_dims: int
    outlier_lo: float      # outlier magnitudes ~ U(outlier_lo, outlier_hi)
    outlier_hi: float
    outlier_row_frac: float = 0.75
    fixed_dims: tuple = ()  # if set, these are the outlier dims (no draw)
    force_max: float | None = None  # one outlier entry set to exactly this
    alphas: tuple = (6.0,)
    description: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def n_outlier_rows(self) -> int:
        return int(round(self.outlier_row_frac * self.M))


WORKLOADS = {
    w.name: w
    for w in [
        Workload(1, "tiny", 16, 256, 256, 1.0, 5.0, 2, 20.0, 60.0,
                 fixed_dims=(17, 200),
                 description="X[16x256] N(0,1) clipped +-5; cols 17, 200 outliers "
                             "|x|~U(20,60) in 12 of 16 rows; W[256x256]"),
        Workload(2, "channel", 2048, 4096, 4096, 0.6267, 5.0, 7, 0.0, 130.0,
                 force_max=130.0,
                 description="channel example: 4089 normal channels E|x|=0.5 clipped "
                             "at 5; 7 outlier channels |x|~U(0,130) (mean 65, one "
                             "entry exactly 130) in 75% of rows; W[4096x4096]"),
        Workload(3, "ffn13b", 2048, 5120, 20480, 0.6, 5.0, 6, 8.0, 60.0,
                 description="13B-scale FFN expansion prefill; 6 outlier dims "
                             "|x|~U(8,60) in 75% of rows"),
        Workload(4, "qkv175b_decode", 32, 12288, 36864, 0.5, 5.0, 7, 20.0, 130.0,
                 description="175B-scale fused QKV projection decode, M=32; 7 "
                             "outlier dims |x|~U(20,130) in 24 of 32 rows"),
        Workload(5, "ffn175b", 4096, 12288, 49152, 0.5, 5.0, 7, 20.0, 130.0,
                 alphas=(4.0, 6.0, 8.0, float("inf")),
                 description="175B-scale FFN expansion prefill; 7 outlier dims "
                             "|x|~U(20,130) in 75% of rows"),
    ]
}


def _draw_x(w: Workload, rng: np.random.Generator):
    if w.fixed_dims:
        dims = np.array(sorted(w.fixed_dims), dtype=np.int64)
    else:
        dims = np.sort(rng.choice(w.K, size=w.n_outlier_dims, replace=False))
    rows = np.sort(rng.choice(w.M, size=w.n_outlier_rows, replace=False))
    x = rng.normal(0.0, w.normal_std, size=(w.M, w.K))
    np.clip(x, -w.clip, w.clip, out=x)
    mag = rng.uniform(w.outlier_lo, w.outlier_hi, size=(rows.size, dims.size))
    sign = np.where(rng.random(size=(rows.size, dims.size)) < 0.5, -1.0, 1.0)
    if w.force_max is not None:
        mag[0, 0] = w.force_max
    x[np.ix_(rows, dims)] = mag * sign
    return x.astype(np.float16), dims, rows


def make_x(w: Workload | str):
    """Return (X fp16 [M,K], planted outlier dims, planted outlier rows)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    return _draw_x(w, rng)


def make_w(w: Workload | str) -> np.ndarray:
    """Return W fp16 [K,N] ~ N(0, 0.02^2), drawn after X from the same stream."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    _draw_x(w, rng)  # advance the stream exactly as make_x does
    out = np.empty((w.K, w.N), dtype=np.float16)
    for r0 in range(0, w.K, _W_ROW_BLOCK):
        r1 = min(w.K, r0 + _W_ROW_BLOCK)
        blk = rng.standard_normal(size=(r1 - r0, w.N), dtype=np.float32)
        blk *= np.float32(W_STD)
        out[r0:r1] = blk.astype(np.float16)
    return out


def make(w: Workload | str):
    """Return (X, W, planted dims, planted rows) for a workload."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    x, dims, rows = make_x(w)
    return x, make_w(w), dims, rows


def random_case(seed: int, M: int, K: int, N: int, n_out: int = 0,
                out_lo: float = 8.0, out_hi: float = 40.0, std: float = 1.0,
                clip: float = 5.0):
    """Small seeded case for edge-shape tests: returns (X fp16, W fp16, dims)."""
    rng = np.random.default_rng(seed)
    n_out = min(n_out, K)
    dims = np.sort(rng.choice(K, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    x = np.clip(rng.normal(0.0, std, size=(M, K)), -clip, clip)
    if n_out and M:
        rows = rng.random(M) < 0.75
        rows[rng.integers(0, M)] = True
        mag = rng.uniform(out_lo, out_hi, size=(M, n_out))
        sign = np.where(rng.random(size=(M, n_out)) < 0.5, -1.0, 1.0)
        sub = x[:, dims]
        sub[rows] = (mag * sign)[rows]
        x[:, dims] = sub
    wmat = (rng.standard_normal(size=(K, N), dtype=np.float32) * np.float32(W_STD))
    return x.astype(np.float16), wmat.astype(np.float16), dims


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def random_int8(seed: int, shape, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Seeded uniform int8 values in [lo, hi] (inputs of the integer GEMM)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.int8)


def random_bias(seed: int, N: int, scale: float = 0.5) -> np.ndarray:
    """Seeded layer bias, fp16 [N] ~ N(0, scale^2)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, scale, size=N).astype(np.float16)


def device_normal(seed: int, shape, scale: float, chunk_rows: int = 4096):
    """Seeded fp16 matrix ~ N(0, scale^2) generated on the GPU in row chunks,
    for sizes whose host generation would take minutes (the size-limit
    tests).  The same seed gives the same values."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    rows, cols = shape
    out = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = (torch.randn((r1 - r0, cols), generator=g, device="cuda") * scale).half()
    return out


def device_case_x(seed: int, M: int, K: int, n_out: int, out_lo: float = 8.0,
                  out_hi: float = 40.0, clip: float = 5.0, chunk_rows: int = 2048):
    """Seeded X [M, K] fp16 on the GPU with random_case's recipe: N(0, 1)
    clipped at +-clip, n_out planted dims whose entries in ~75 % of the rows
    (one row always) have magnitudes uniform in [out_lo, out_hi] and random
    sign.  Returns (X on the GPU, planted dims as a sorted numpy array)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((M, K), dtype=torch.float16, device="cuda")
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        x[r0:r1] = torch.randn((r1 - r0, K), generator=g, device="cuda").clamp_(-clip, clip).half()
    dims = torch.sort(torch.randperm(K, generator=g, device="cuda")[:n_out]).values
    if n_out and M:
        rows = torch.rand(M, generator=g, device="cuda") < 0.75
        rows[int(torch.randint(0, M, (1,), generator=g, device="cuda"))] = True
        mag = torch.rand((M, n_out), generator=g, device="cuda") * (out_hi - out_lo) + out_lo
        sign = torch.where(torch.rand((M, n_out), generator=g, device="cuda") < 0.5, -1.0, 1.0)
        sub = x[:, dims]
        sub[rows] = (mag * sign)[rows].half()
        x[:, dims] = sub
    return x, dims.cpu().numpy()
