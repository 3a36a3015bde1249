"""Python binding of libint8mm.so, the gfx950 LLM.int8() decomposed matmul.

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback -- if the library is not built, importing works but
every call raises.

    W_i8, w_absmax = quantize_weight(W)            # once, offline
    Y = mixed_matmul(X, W_i8, w_absmax, W, alpha=6.0)

Method: "LLM.int8() — 大模型激活值里藏着几个超大异常通道" (方法 1, 方法 2);
developer.aliyun.com "LLM.int8()" §2.2 图2.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "LIB_PATH", "Int8mmError", "load", "quantize_weight", "workspace_size",
    "workspace_layout", "mixed_matmul", "mixed_matmul_noalloc", "detect_outliers", "quantize_activations", "gemm_i32", "read_workspace", "DECODE_MAX_M",
    "timing_enable", "timing_read", "default_n_cap", "kpad", "rpad", "packed_size", "pack_rows",
    "kernel_config", "outlier_cache_size", "build_outlier_cache", "mixed_matmul_cached",
    "STATUS_OK", "STATUS_EINVAL", "STATUS_EALIGN", "STATUS_EWORKSPACE", "STATUS_EHIP",
    "STATUS_ESCRATCH", "FLAG_OVERFLOW", "FLAG_CACHE_MISS", "FLAG_CACHE_MISMATCH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint8mm.so")
DECODE_MAX_M = 32
STATUS_OK, STATUS_EINVAL, STATUS_EALIGN, STATUS_EWORKSPACE, STATUS_EHIP, STATUS_ESCRATCH = range(6)
# bits of the workspace status word (read_workspace(...)["status"])
FLAG_OVERFLOW, FLAG_CACHE_MISS, FLAG_CACHE_MISMATCH = 1, 2, 4
WS_FIELDS = ["header", "colmax", "mask", "idx", "x_absmax", "X_i8", "X_out", "W_outT",
             "rowmax"]

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class Int8mmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"int8mm status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libint8mm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m int8_mixed_precision_outlier_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.int8mm_status_string.restype = ctypes.c_char_p
    lib.int8mm_status_string.argtypes = [ctypes.c_int]
    lib.int8mm_last_hip_error.restype = ctypes.c_int
    lib.int8mm_last_hip_error.argtypes = []
    lib.int8_packed_size.restype = ctypes.c_int64
    lib.int8_packed_size.argtypes = [_i64, _i64]
    lib.int8_pack_rows.restype = ctypes.c_int
    lib.int8_pack_rows.argtypes = [_vp, _i64, _i64, _vp, _vp]
    lib.int8_quantize_weight.restype = ctypes.c_int
    lib.int8_quantize_weight.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    lib.int8_mixed_matmul_workspace_size.restype = ctypes.c_size_t
    lib.int8_mixed_matmul_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _vp]
    lib.int8_mixed_matmul.restype = ctypes.c_int
    lib.int8_mixed_matmul.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _i64, ctypes.c_float,
                                      _vp, _vp, _vp, ctypes.c_size_t, _i64, _vp]
    lib.int8_detect_outliers.restype = ctypes.c_int
    lib.int8_detect_outliers.argtypes = [_vp, _i64, _i64, ctypes.c_float, _i64, _vp,
                                         ctypes.c_size_t, _vp]
    lib.int8_quantize_activations.restype = ctypes.c_int
    lib.int8_quantize_activations.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                              ctypes.c_size_t, _vp]
    lib.int8_outlier_cache_size.restype = ctypes.c_int64
    lib.int8_outlier_cache_size.argtypes = [_i64, _i64, _i64]
    lib.int8_build_outlier_cache.restype = ctypes.c_int
    lib.int8_build_outlier_cache.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, ctypes.c_size_t, _vp]
    lib.int8_mixed_matmul_cached.restype = ctypes.c_int
    lib.int8_mixed_matmul_cached.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _i64, ctypes.c_float,
                                             _vp, _vp, _vp, ctypes.c_size_t, _i64, _vp]
    lib.int8mm_timing_enable.restype = ctypes.c_int
    lib.int8mm_timing_enable.argtypes = [ctypes.c_int]
    lib.int8mm_timing_read.restype = ctypes.c_int
    lib.int8mm_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.int8_gemm_i32.restype = ctypes.c_int
    lib.int8_gemm_i32.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, _vp]
    lib.int8_mixed_matmul_noalloc.restype = ctypes.c_int
    lib.int8_mixed_matmul_noalloc.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _i64,
                                              ctypes.c_float, _vp, _vp, _i64, _vp]
    lib.int8mm_kernel_config.restype = ctypes.c_int
    lib.int8mm_kernel_config.argtypes = [_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int32)]
    _lib = lib
    return lib


def _check(status: int):
    if status != STATUS_OK:
        lib = load()
        msg = lib.int8mm_status_string(status).decode()
        if status == STATUS_EHIP:
            msg += f" (hipError {lib.int8mm_last_hip_error()})"
        raise Int8mmError(status, msg)


def _ptr(t: torch.Tensor | None):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for the temporary allocations of a call launched on `stream`:
    torch's caching allocator ties a block to the stream current at
    allocation, so buffers the call's kernels use are allocated there."""
    import contextlib
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _raise_on_overflow(workspace: torch.Tensor, n_cap: int):
    """check=True: wait for the call and raise if it found more outlier
    columns than n_cap (status bit 0; Y is then all NaN)."""
    hdr = workspace[:16].view(torch.int32).cpu()
    if int(hdr[0]) & FLAG_OVERFLOW:
        raise Int8mmError(STATUS_EINVAL, f"{int(hdr[2])} outlier columns found, more than "
                                         f"n_cap={n_cap}: pass a larger n_cap (n_cap=K always fits)")


def _dev(t: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def kpad(K: int) -> int:
    """K rounded up to the 64-byte blocks of the packed int8 layout."""
    return (K + 63) // 64 * 64


def rpad(R: int) -> int:
    """Rows rounded up to the 16-row blocks of the packed int8 layout."""
    return (R + 15) // 16 * 16


def packed_size(R: int, K: int) -> int:
    return int(load().int8_packed_size(R, K))


def pack_rows(A: torch.Tensor, stream=None) -> torch.Tensor:
    """Row-major int8 [R,K] -> packed layout, as an int8 tensor [rpad(R), kpad(K)]
    (an opaque byte buffer; see include/int8mm.h)."""
    lib = load()
    _dev(A, torch.int8, "A", 2)
    R, K = A.shape
    with _on(stream):
        out = torch.empty((rpad(R), kpad(K)), dtype=torch.int8, device=A.device)
    _check(lib.int8_pack_rows(_ptr(A), R, K, _ptr(out), _stream(stream)))
    return out


def quantize_weight(W: torch.Tensor, stream=None):
    """W fp16 [K,N] -> (W_i8 packed int8 [N, kpad(K)], w_absmax fp32 [N])."""
    lib = load()
    _dev(W, torch.float16, "W", 2)
    K, N = W.shape
    with _on(stream):
        W_i8 = torch.empty((N, kpad(K)), dtype=torch.int8, device=W.device)
        w_absmax = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(lib.int8_quantize_weight(_ptr(W), K, N, _ptr(W_i8), _ptr(w_absmax), _stream(stream)))
    return W_i8, w_absmax


def workspace_layout(M: int, K: int, N: int, n_cap: int):
    """(total bytes, {field: byte offset}) of the mixed-matmul workspace."""
    lib = load()
    offs = (ctypes.c_int64 * len(WS_FIELDS))()
    total = lib.int8_mixed_matmul_workspace_size(M, K, N, n_cap, offs)
    if total == 0:
        raise Int8mmError(STATUS_EINVAL, f"invalid shape M={M} K={K} N={N} n_cap={n_cap}")
    return int(total), dict(zip(WS_FIELDS, [int(o) for o in offs]))


def workspace_size(M: int, K: int, N: int, n_cap: int) -> int:
    return workspace_layout(M, K, N, n_cap)[0]


def default_n_cap(K: int) -> int:
    """Outlier capacity used when the caller gives none: all of K for small K,
    else 1024 columns (the pages report fewer than ten outlier dims).  A call
    that finds more sets status bit 0 and returns an all-NaN Y; check=True
    raises instead."""
    return K if K <= 8192 else 1024


def kernel_config(M: int, N: int, K: int):
    """The kernel configuration a call of this shape launches on the current
    device: ("decode", row blocks per workgroup, K-splitting wavefronts,
    token blocks), ("tiled", BM, BN, wavefronts), or ("split", n1, BN,
    wavefronts): columns below n1 in 256x256 tiles, the rest in a second
    launch of BN-column tiles."""
    cfg = (ctypes.c_int32 * 4)()
    _check(load().int8mm_kernel_config(M, N, K, cfg))
    kind = ("decode", "tiled", "split")[cfg[0]]
    return (kind, int(cfg[1]), int(cfg[2]), int(cfg[3]))


def mixed_matmul(X: torch.Tensor, W_i8: torch.Tensor, w_absmax: torch.Tensor,
                 W: torch.Tensor, alpha: float = 6.0, bias: torch.Tensor | None = None,
                 n_cap: int | None = None, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, stream=None,
                 check: bool = False) -> torch.Tensor:
    """Y fp16 [M,N] = LLM.int8() decomposition of X fp16 [M,K] . W fp16 [K,N]
    (+ bias fp16 [N]).

    W_i8/w_absmax come from quantize_weight(W).  `workspace` (uint8, device)
    may be passed to reuse memory and to inspect the intermediates with
    read_workspace(); its size is workspace_size(M, K, N, n_cap).  With more
    than n_cap outlier columns the call sets status bit 0 in the workspace
    and every element of Y is NaN; n_cap = K is always enough.  check=True
    waits for the call and raises Int8mmError in that case (a host sync;
    not for graph capture).  Buffers the call allocates (out, workspace) are
    allocated on `stream` when one is given.
    """
    lib = load()
    _dev(X, torch.float16, "X", 2)
    _dev(W_i8, torch.int8, "W_i8", 2)
    _dev(w_absmax, torch.float32, "w_absmax", 1)
    _dev(W, torch.float16, "W", 2)
    M, K = X.shape
    N = W_i8.shape[0]
    if W_i8.shape != (N, kpad(K)) or W.shape != (K, N) or w_absmax.shape != (N,):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W_i8 {tuple(W_i8.shape)}, "
                         f"W {tuple(W.shape)}, w_absmax {tuple(w_absmax.shape)}")
    if bias is not None:
        _dev(bias, torch.float16, "bias", 1)
        if bias.shape != (N,):
            raise ValueError(f"bias must have shape ({N},)")
    if n_cap is None:
        n_cap = default_n_cap(K)
    with _on(stream):
        if out is None:
            out = torch.empty((M, N), dtype=torch.float16, device=X.device)
        else:
            _dev(out, torch.float16, "out", 2)
            if out.shape != (M, N):
                raise ValueError("out has the wrong shape")
        need = lib.int8_mixed_matmul_workspace_size(M, K, N, n_cap, None)
        if workspace is None:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=X.device)
        else:
            _dev(workspace, torch.uint8, "workspace", 1)
    a = float(alpha)
    st = lib.int8_mixed_matmul(_ptr(X), M, K, _ptr(W_i8), _ptr(w_absmax), _ptr(W), N,
                               ctypes.c_float(a), _ptr(bias) if bias is not None else None,
                               _ptr(out), _ptr(workspace), workspace.numel(), n_cap,
                               _stream(stream))
    _check(st)
    if check and M and N:
        _raise_on_overflow(workspace, n_cap)
    return out


def mixed_matmul_noalloc(X: torch.Tensor, W_i8: torch.Tensor, w_absmax: torch.Tensor,
                         W: torch.Tensor, out: torch.Tensor, alpha: float = 6.0,
                         bias: torch.Tensor | None = None, n_cap: int | None = None,
                         stream=None) -> torch.Tensor:
    """mixed_matmul for callers that cannot allocate: the library's static
    per-device scratch array is the workspace (int8_mixed_matmul_noalloc),
    and `out` must be given.  Calls that overlap on one GPU share that array
    and race.  Shapes needing more than the array holds raise
    Int8mmError(STATUS_ESCRATCH)."""
    lib = load()
    _dev(X, torch.float16, "X", 2)
    _dev(W_i8, torch.int8, "W_i8", 2)
    _dev(w_absmax, torch.float32, "w_absmax", 1)
    _dev(W, torch.float16, "W", 2)
    _dev(out, torch.float16, "out", 2)
    M, K = X.shape
    N = W_i8.shape[0]
    if (W_i8.shape != (N, kpad(K)) or W.shape != (K, N) or w_absmax.shape != (N,)
            or out.shape != (M, N)):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W_i8 {tuple(W_i8.shape)}, "
                         f"W {tuple(W.shape)}, w_absmax {tuple(w_absmax.shape)}, "
                         f"out {tuple(out.shape)}")
    if bias is not None:
        _dev(bias, torch.float16, "bias", 1)
        if bias.shape != (N,):
            raise ValueError(f"bias must have shape ({N},)")
    if n_cap is None:
        n_cap = default_n_cap(K)
    _check(lib.int8_mixed_matmul_noalloc(_ptr(X), M, K, _ptr(W_i8), _ptr(w_absmax), _ptr(W), N,
                                         ctypes.c_float(float(alpha)),
                                         _ptr(bias) if bias is not None else None, _ptr(out),
                                         n_cap, _stream(stream)))
    return out


def detect_outliers(X: torch.Tensor, workspace: torch.Tensor, alpha: float = 6.0,
                    n_cap: int | None = None, stream=None) -> torch.Tensor:
    """Stage 1 alone: fills the colmax, mask, idx and header fields of
    `workspace` (a mixed_matmul workspace for this M, K, n_cap and any N)
    for X fp16 [M,K].  Returns `workspace`; read_workspace() reads it."""
    lib = load()
    _dev(X, torch.float16, "X", 2)
    _dev(workspace, torch.uint8, "workspace", 1)
    M, K = X.shape
    if n_cap is None:
        n_cap = default_n_cap(K)
    _check(lib.int8_detect_outliers(_ptr(X), M, K, ctypes.c_float(float(alpha)), n_cap,
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def quantize_activations(X: torch.Tensor, W: torch.Tensor, workspace: torch.Tensor,
                         n_cap: int | None = None, stream=None) -> torch.Tensor:
    """Stage 2 alone, after detect_outliers on the same workspace: fills
    x_absmax, X_i8, X_out, W_outT (and idx, header) for X fp16 [M,K] and the
    outlier rows of W fp16 [K,N].  Returns `workspace`."""
    lib = load()
    _dev(X, torch.float16, "X", 2)
    _dev(W, torch.float16, "W", 2)
    _dev(workspace, torch.uint8, "workspace", 1)
    M, K = X.shape
    if W.shape[0] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}")
    N = W.shape[1]
    if n_cap is None:
        n_cap = default_n_cap(K)
    _check(lib.int8_quantize_activations(_ptr(X), M, K, _ptr(W), N, n_cap, _ptr(workspace),
                                         workspace.numel(), _stream(stream)))
    return workspace


def gemm_i32(X_p: torch.Tensor, W_p: torch.Tensor, M: int, N: int, K: int,
             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Out_i32 [M,N] = X . W^T from packed int8 operands (pack_rows of X [M,K]
    and W [N,K]); exact int32."""
    lib = load()
    _dev(X_p, torch.int8, "X_p", 2)
    _dev(W_p, torch.int8, "W_p", 2)
    if X_p.numel() != packed_size(M, K) or W_p.numel() != packed_size(N, K):
        raise ValueError("packed operand sizes do not match M, N, K")
    if out is None:
        with _on(stream):
            out = torch.empty((M, N), dtype=torch.int32, device=X_p.device)
    _check(lib.int8_gemm_i32(_ptr(X_p), M, K, _ptr(W_p), N, _ptr(out), _stream(stream)))
    return out


def outlier_cache_size(K: int, N: int, n_dims: int) -> int:
    n = int(load().int8_outlier_cache_size(K, N, n_dims))
    if n < 0:
        raise Int8mmError(STATUS_EINVAL, f"invalid cache shape K={K} N={N} n_dims={n_dims}")
    return n


def build_outlier_cache(W: torch.Tensor, dims, stream=None) -> torch.Tensor:
    """The fp16 rows W[dims, :] of a static set of outlier dims (strictly
    ascending), as the opaque cache buffer (uint8, device) that
    mixed_matmul_cached takes instead of the whole fp16 W.  Load-time call:
    it synchronizes the stream."""
    import numpy as _np
    lib = load()
    _dev(W, torch.float16, "W", 2)
    K, N = W.shape
    d = _np.ascontiguousarray(_np.asarray(dims, dtype=_np.int32).reshape(-1))
    with _on(stream):
        cache = torch.empty((outlier_cache_size(K, N, d.size),), dtype=torch.uint8,
                            device=W.device)
    _check(lib.int8_build_outlier_cache(_ptr(W), K, N, d.ctypes.data_as(ctypes.c_void_p) if d.size
                                        else None, d.size, _ptr(cache), cache.numel(),
                                        _stream(stream)))
    return cache


def mixed_matmul_cached(X: torch.Tensor, W_i8: torch.Tensor, w_absmax: torch.Tensor,
                        cache: torch.Tensor, alpha: float = 6.0,
                        bias: torch.Tensor | None = None, n_cap: int | None = None,
                        workspace: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, stream=None,
                        check: bool = False) -> torch.Tensor:
    """mixed_matmul with the outlier rows from build_outlier_cache instead of
    the whole fp16 W.  Outlier dims outside the cache use their dequantized
    int8 rows and set bit 1 of read_workspace(...)["status"]; a cache built
    for another K or N is not used at all (bit 2)."""
    lib = load()
    _dev(X, torch.float16, "X", 2)
    _dev(W_i8, torch.int8, "W_i8", 2)
    _dev(w_absmax, torch.float32, "w_absmax", 1)
    _dev(cache, torch.uint8, "cache", 1)
    M, K = X.shape
    N = W_i8.shape[0]
    if W_i8.shape != (N, kpad(K)) or w_absmax.shape != (N,):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W_i8 {tuple(W_i8.shape)}, "
                         f"w_absmax {tuple(w_absmax.shape)}")
    if bias is not None:
        _dev(bias, torch.float16, "bias", 1)
        if bias.shape != (N,):
            raise ValueError(f"bias must have shape ({N},)")
    if cache.numel() < outlier_cache_size(K, N, 0):
        raise ValueError(f"cache of {cache.numel()} bytes is too small for K={K}, N={N}: "
                         "build it with build_outlier_cache(W) for this weight")
    if n_cap is None:
        n_cap = default_n_cap(K)
    with _on(stream):
        if out is None:
            out = torch.empty((M, N), dtype=torch.float16, device=X.device)
        else:
            _dev(out, torch.float16, "out", 2)
            if out.shape != (M, N):
                raise ValueError("out has the wrong shape")
        need = lib.int8_mixed_matmul_workspace_size(M, K, N, n_cap, None)
        if workspace is None:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=X.device)
        else:
            _dev(workspace, torch.uint8, "workspace", 1)
    _check(lib.int8_mixed_matmul_cached(_ptr(X), M, K, _ptr(W_i8), _ptr(w_absmax), _ptr(cache),
                                        N, ctypes.c_float(float(alpha)),
                                        _ptr(bias) if bias is not None else None, _ptr(out),
                                        _ptr(workspace), workspace.numel(), n_cap,
                                        _stream(stream)))
    if check and M and N:
        _raise_on_overflow(workspace, n_cap)
    return out


def read_workspace(workspace: torch.Tensor, M: int, K: int, N: int, n_cap: int):
    """Views of the intermediates a mixed_matmul call left in `workspace`
    (synchronizes the current stream to read the outlier count).  X_i8 is
    the raw packed layout [rpad(M), kpad(K)]; X_out and W_outT are the raw
    packed bytes of fp16 matrices, [rpad(M), kpad(2*n_cap)] and
    [N, kpad(2*n_cap)] (outlier t of a row is bytes 2t, 2t+1 of its packed
    row)."""
    _, off = workspace_layout(M, K, N, n_cap)
    ws = workspace

    def view(field, dtype, count):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off[field]:off[field] + nbytes].view(dtype)

    hdr = view("header", torch.int32, 4).cpu()
    n = int(hdr[1])
    ob = kpad(2 * n_cap)
    return dict(
        status=int(hdr[0]), n=n, n_found=int(hdr[2]),
        colmax=view("colmax", torch.float32, K),
        mask=view("mask", torch.int32, (K + 31) // 32),
        idx=view("idx", torch.int32, n),
        x_absmax=view("x_absmax", torch.float32, M),
        X_i8=view("X_i8", torch.int8, packed_size(M, K)).view(rpad(M), kpad(K)),
        X_out=view("X_out", torch.int8, rpad(M) * ob).view(rpad(M), ob),
        W_outT=view("W_outT", torch.int8, N * ob).view(N, ob),
    )


def timing_enable(on: bool = True) -> None:
    """Have the main kernel of every mixed_matmul call record HIP events at its
    start and end (recorded by the kernel dispatch itself)."""
    _check(load().int8mm_timing_enable(1 if on else 0))


def timing_read():
    """(summed main-kernel milliseconds, launches) since timing_enable; clears."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(load().int8mm_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
