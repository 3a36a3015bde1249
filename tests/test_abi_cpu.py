"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/int8mm.h, and rejects bad arguments before any launch."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import int8_mixed_precision_outlier_amd as i8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8mm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(i8.LIB_PATH),
                                reason="libint8mm.so not built (run __graft_entry__.build())")


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", src)) - {"if", "sizeof"})


def test_probe_library_exports_every_declared_symbol():
    """include/int8mm_probes.h (the peak probes) against libint8mm_probes.so."""
    from int8_mixed_precision_outlier_amd import probes
    if not os.path.exists(probes.LIB_PATH):
        pytest.skip("libint8mm_probes.so not built")
    lib = probes.load()
    names = declared_functions(os.path.join(ROOT, "include", "int8mm_probes.h"))
    assert set(names) == {"int8mm_probe_mfma_i8", "int8mm_probe_mfma_f16", "int8mm_probe_read"}
    for n in names:
        assert hasattr(lib, n), n


def test_exports_every_declared_symbol():
    lib = i8.load()
    names = declared_functions()
    assert {"int8_quantize_weight", "int8_mixed_matmul", "int8_gemm_i32",
            "int8_mixed_matmul_workspace_size", "int8mm_status_string",
            "int8mm_last_hip_error", "int8_pack_rows", "int8_packed_size",
            "int8mm_timing_enable", "int8mm_timing_read", "int8_detect_outliers",
            "int8_quantize_activations"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


C_CONSUMER = r"""
#include <stdio.h>
#include "int8mm.h"
int main(void) {
  int64_t off[INT8MM_WS_NFIELDS];
  size_t total = int8_mixed_matmul_workspace_size(4096, 12288, 49152, 1024, off);
  printf("%s %zu %lld %d\n", int8mm_status_string(INT8MM_OK), total,
         (long long)off[INT8MM_WS_WOUT], int8_pack_rows(NULL, 8, 24, NULL, NULL));
  return total == 0;
}
"""


def test_header_is_a_c_abi(tmp_path):
    """The header compiles as C99 and a C program links against the library
    and calls it (host-only entry points; no GPU work)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(i8.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-L", libdir, "-lint8mm",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    total, off = i8.workspace_layout(4096, 12288, 49152, 1024)
    assert out == ["ok", str(total), str(off["W_outT"]), str(i8.STATUS_EALIGN)]


def test_status_strings():
    lib = i8.load()
    for s in range(6):
        assert lib.int8mm_status_string(s)
    assert lib.int8mm_last_hip_error() == 0


def test_workspace_layout_arithmetic():
    total, off = i8.workspace_layout(4096, 12288, 49152, 1024)
    assert all(o % 256 == 0 for o in off.values())
    order = list(off.values())
    assert order == sorted(order)
    assert off["X_i8"] >= off["x_absmax"] + 4 * 4096
    assert off["X_out"] >= off["X_i8"] + 4096 * 12288
    assert off["W_outT"] >= off["X_out"] + 2 * 4096 * 1024
    assert total >= off["W_outT"] + 2 * 49152 * 1024
    lib = i8.load()
    assert lib.int8_mixed_matmul_workspace_size(16, 256, 256, 257, None) == 0  # n_cap > K
    assert lib.int8_mixed_matmul_workspace_size(16, 250, 256, 0, None) == 0    # K % 16
    assert lib.int8_mixed_matmul_workspace_size(16, 65536 + 16, 256, 0, None) == 0
    assert lib.int8_mixed_matmul_workspace_size(0, 256, 256, 0, None) > 0


FAKE = ctypes.c_void_p(1 << 20)  # aligned non-null; never dereferenced (checks fail first)


def mm(lib, M=64, K=256, N=256, alpha=6.0, ws_bytes=1 << 30, n_cap=16, X=FAKE, Wi8=FAKE,
       wabs=FAKE, W=FAKE, Y=FAKE, ws=FAKE, bias=None):
    return lib.int8_mixed_matmul(X, M, K, Wi8, wabs, W, N, ctypes.c_float(alpha), bias, Y, ws,
                                 ws_bytes, n_cap, None)


def test_mixed_matmul_rejects_bad_arguments():
    lib = i8.load()
    assert mm(lib, alpha=float("nan")) == i8.STATUS_EINVAL
    assert mm(lib, alpha=-1.0) == i8.STATUS_EINVAL
    assert mm(lib, M=-1) == i8.STATUS_EINVAL
    assert mm(lib, K=-16) == i8.STATUS_EINVAL
    assert mm(lib, K=65536 + 16) == i8.STATUS_EINVAL
    assert mm(lib, K=250) == i8.STATUS_EALIGN
    assert mm(lib, N=250) == i8.STATUS_EALIGN
    assert mm(lib, n_cap=257) == i8.STATUS_EINVAL
    assert mm(lib, n_cap=-1) == i8.STATUS_EINVAL
    assert mm(lib, X=None) == i8.STATUS_EINVAL
    assert mm(lib, W=None) == i8.STATUS_EINVAL
    assert mm(lib, Y=None) == i8.STATUS_EINVAL
    assert mm(lib, ws=None) == i8.STATUS_EINVAL
    assert mm(lib, X=ctypes.c_void_p((1 << 20) + 8)) == i8.STATUS_EALIGN
    assert mm(lib, ws=ctypes.c_void_p((1 << 20) + 16)) == i8.STATUS_EALIGN
    assert mm(lib, bias=ctypes.c_void_p((1 << 20) + 2)) == i8.STATUS_EALIGN
    assert mm(lib, n_cap=1 << 15, M=1 << 16, K=1 << 15, N=16) == i8.STATUS_EINVAL  # X_out > 2^31 B
    assert mm(lib, ws_bytes=1024) == i8.STATUS_EWORKSPACE
    assert mm(lib, M=1 << 20, K=65536) == i8.STATUS_EINVAL  # M*K over 2^31
    # empty problems are accepted without touching the GPU
    assert mm(lib, M=0) == i8.STATUS_OK
    assert mm(lib, N=0) == i8.STATUS_OK
    assert mm(lib, alpha=float("inf"), M=0) == i8.STATUS_OK


def test_quantize_weight_and_gemm_reject_bad_arguments():
    lib = i8.load()
    q = lib.int8_quantize_weight
    assert q(FAKE, 250, 256, FAKE, FAKE, None) == i8.STATUS_EALIGN
    assert q(FAKE, 256, 250, FAKE, FAKE, None) == i8.STATUS_EALIGN
    assert q(FAKE, -16, 256, FAKE, FAKE, None) == i8.STATUS_EINVAL
    assert q(None, 256, 256, FAKE, FAKE, None) == i8.STATUS_EINVAL
    assert q(FAKE, 256, 256, FAKE, None, None) == i8.STATUS_EINVAL
    assert q(FAKE, 256, 256, ctypes.c_void_p((1 << 20) + 4), FAKE, None) == i8.STATUS_EALIGN
    assert q(FAKE, 256, 0, FAKE, FAKE, None) == i8.STATUS_OK
    g = lib.int8_gemm_i32
    assert g(FAKE, 64, 250, FAKE, 256, FAKE, None) == i8.STATUS_EALIGN
    assert g(FAKE, 64, 256, FAKE, 256, None, None) == i8.STATUS_EINVAL
    assert g(FAKE, -1, 256, FAKE, 256, FAKE, None) == i8.STATUS_EINVAL
    assert g(FAKE, 0, 256, FAKE, 256, FAKE, None) == i8.STATUS_OK


def test_stage_exports_reject_bad_arguments():
    lib = i8.load()

    def det(M=64, K=256, alpha=6.0, n_cap=16, X=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.int8_detect_outliers(X, M, K, ctypes.c_float(alpha), n_cap, ws, ws_bytes, None)

    def qa(M=64, K=256, N=256, n_cap=16, X=FAKE, W=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.int8_quantize_activations(X, M, K, W, N, n_cap, ws, ws_bytes, None)

    assert det(alpha=float("nan")) == i8.STATUS_EINVAL
    assert det(alpha=-0.5) == i8.STATUS_EINVAL
    assert det(K=250) == i8.STATUS_EALIGN
    assert det(n_cap=257) == i8.STATUS_EINVAL
    assert det(X=None) == i8.STATUS_EINVAL
    assert det(ws=None) == i8.STATUS_EINVAL
    assert det(ws=ctypes.c_void_p((1 << 20) + 64)) == i8.STATUS_EALIGN
    # the detector needs the fields up to X_out only, for any N
    _, off = i8.workspace_layout(64, 256, 4096, 16)
    assert det(ws_bytes=off["X_out"] - 1) == i8.STATUS_EWORKSPACE
    assert det(M=0) == i8.STATUS_OK
    assert qa(N=250) == i8.STATUS_EALIGN
    assert qa(n_cap=-1) == i8.STATUS_EINVAL
    assert qa(W=None) == i8.STATUS_EINVAL
    assert qa(X=ctypes.c_void_p((1 << 20) + 8)) == i8.STATUS_EALIGN
    total, _ = i8.workspace_layout(64, 256, 256, 16)
    assert qa(ws_bytes=total - 1) == i8.STATUS_EWORKSPACE
    assert qa(M=0) == i8.STATUS_OK


def test_packed_size_and_pack_validation():
    lib = i8.load()
    assert lib.int8_packed_size(37, 80) == 48 * 128
    assert lib.int8_packed_size(4096, 12288) == 4096 * 12288
    assert lib.int8_packed_size(1, 16) == 16 * 64
    assert lib.int8_packed_size(-1, 16) == -1
    assert lib.int8_pack_rows(FAKE, 8, 24, FAKE, None) == i8.STATUS_EALIGN
    assert lib.int8_pack_rows(None, 8, 32, FAKE, None) == i8.STATUS_EINVAL
    assert lib.int8_pack_rows(FAKE, 0, 32, FAKE, None) == i8.STATUS_OK


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    with pytest.raises(TypeError):
        i8.quantize_weight(torch.zeros((16, 16), dtype=torch.float16))


def test_module_requires_gpu_weights():
    import torch
    from int8_mixed_precision_outlier_amd.linear import Int8MixedLinear
    with pytest.raises(TypeError):
        Int8MixedLinear(torch.zeros((16, 16), dtype=torch.float16))


def test_outlier_cache_size_and_validation():
    lib = i8.load()
    assert lib.int8_outlier_cache_size(4096, 4096, 7) >= 256 + 4 * 4096 + 2 * 7 * 4096 + 4 * 7
    assert lib.int8_outlier_cache_size(4096, 4096, 0) > 0
    assert lib.int8_outlier_cache_size(16, 16, 17) == -1
    assert lib.int8_outlier_cache_size(-1, 16, 0) == -1
    need = lib.int8_outlier_cache_size(256, 64, 3)

    def build(dims, K=256, N=64, cache=FAKE, nbytes=need, W=FAKE):
        arr = (ctypes.c_int32 * max(len(dims), 1))(*dims)
        return lib.int8_build_outlier_cache(W, K, N, arr, len(dims), cache, nbytes, None)
    assert build([5, 3, 9]) == i8.STATUS_EINVAL          # not ascending
    assert build([3, 3, 9]) == i8.STATUS_EINVAL          # repeated
    assert build([3, 9, 256]) == i8.STATUS_EINVAL        # out of range
    assert build([-1, 3, 9]) == i8.STATUS_EINVAL
    assert build([3, 9, 17], cache=ctypes.c_void_p((1 << 20) + 16)) == i8.STATUS_EALIGN
    assert build([3, 9, 17], nbytes=need - 1) == i8.STATUS_EWORKSPACE
    assert build([3, 9, 17], K=250) == i8.STATUS_EALIGN
    assert build([3, 9, 17], cache=None) == i8.STATUS_EINVAL
    mc = lib.int8_mixed_matmul_cached
    assert mc(FAKE, 64, 256, FAKE, FAKE, None, 256, ctypes.c_float(6.0), None, FAKE, FAKE,
              1 << 30, 16, None) == i8.STATUS_EINVAL
    assert mc(FAKE, 64, 256, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 16), 256,
              ctypes.c_float(6.0), None, FAKE, FAKE, 1 << 30, 16, None) == i8.STATUS_EALIGN
    # the plain entry point requires the fp16 weights
    assert lib.int8_mixed_matmul(FAKE, 64, 256, FAKE, FAKE, None, 256, ctypes.c_float(6.0), None,
                                 FAKE, FAKE, 1 << 30, 16, None) == i8.STATUS_EINVAL


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "single-GPU" in r.stderr


def test_quantize_stage_accepts_null_weights_when_n_is_zero():
    """The validator lets int8_quantize_activations run with N = 0 and a NULL
    weight pointer (an empty matrix); only the launch (no GPU here) may
    fail, never the argument checks."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers; the GPU test runs the real call")
    lib = i8.load()
    M, K, n_cap = 4, 64, 64
    size = lib.int8_mixed_matmul_workspace_size(M, K, 0, n_cap, None)
    assert size > 0
    fake = ctypes.c_void_p(1 << 20)  # 256-byte aligned, never dereferenced on the host
    st = lib.int8_quantize_activations(fake, M, K, None, 0, n_cap, fake, size, None)
    assert st in (i8.STATUS_OK, i8.STATUS_EHIP)


def test_kernel_config_reaches_every_decode_instantiation():
    """Host rule of the decode launcher on a 256-CU device: the N values the
    GPU parity tests use reach all twelve (row blocks, wavefronts)
    instantiations; 33-64 tokens take it with 3 or 4 token blocks where it
    streams the weights faster than the tiled kernel, larger M the tiled one."""
    expect = {272: (1, 8), 4112: (1, 2), 8224: (1, 2), 5120: (2, 8), 12320: (2, 2),
              16448: (2, 2), 12288: (3, 2), 16416: (3, 2), 24624: (3, 2), 15360: (4, 2),
              8320: (4, 8), 24640: (4, 2), 41024: (4, 2), 20480: (5, 2), 24576: (6, 2),
              32768: (8, 2), 36864: (9, 2), 49152: (12, 2)}
    got = {N: i8.kernel_config(32, N, 1040)[1:3] for N in expect}
    assert got == expect and len(set(got.values())) == 12
    assert i8.kernel_config(16, 4096, 64) == ("decode", 1, 2, 1)
    assert i8.kernel_config(4096, 49152, 12288) == ("tiled", 256, 256, 8)
    assert i8.kernel_config(96, 49152, 12288) == ("tiled", 128, 128, 4)
    # 33-64 tokens: the decode kernel with 3 or 4 token blocks (4 only for
    # N <= 16384), two wavefronts
    assert i8.kernel_config(48, 49152, 12288) == ("decode", 12, 2, 3)
    assert i8.kernel_config(64, 15360, 5120) == ("decode", 4, 2, 4)
    assert i8.kernel_config(64, 49152, 12288) == ("tiled", 128, 128, 4)
    assert i8.kernel_config(2048, 5120, 5120) == ("tiled", 256, 160, 8)
    assert i8.kernel_config(2048, 20480, 5120) == ("split", 16384, 128, 8)
    assert i8.kernel_config(2048, 4096, 4096) == ("tiled", 256, 128, 8)
    assert i8.kernel_config(1100, 20000, 208) == ("split", 13056, 128, 4)
    assert i8.kernel_config(2048, 20992, 128) == ("split", 16384, 160, 8)
    with pytest.raises(i8.Int8mmError):
        i8.kernel_config(32, 24, 64)  # N % 16 != 0



def test_newer_path_sweep_reaches_every_new_launch_path():
    """The seeded sweep over the newer launch paths (a GPU test) takes each of
    them at least once: 33-64-token decode with three and with four token
    blocks, 256x160 and 256x128 tiles, the column split, and rows of more
    than 6144 columns on the prefill and the decode side."""
    from test_gpu_parity import newpath_case
    seen = set()
    for case in range(18):
        M, K, N, _, _ = newpath_case(case)
        c = i8.kernel_config(M, N, K)
        if c[0] == "decode" and M > 32:
            seen.add(("decode", c[3]))
        elif c[0] == "tiled" and c[1] == 256 and c[2] in (160, 128):
            seen.add(("tiled", c[2]))
        elif c[0] == "split":
            seen.add("split")
        if K > 6144 and M > 32:
            seen.add(("long rows", c[0]))
    assert {("decode", 3), ("decode", 4), ("tiled", 160), ("tiled", 128), "split",
            ("long rows", "decode"), ("long rows", "tiled")} <= seen, seen


def test_launch_plan_invariants_over_seeded_shapes():
    """The launch planner's choice, over 3000 seeded shapes (256 CUs, the
    count assumed without a device): decode only up to 64 tokens and always
    up to 32; tiles only of the shapes the library builds; a column split
    only at a multiple of 256 strictly inside N, its first launch as many
    columns of 256x256 tiles as its rounds hold and its second a smaller
    tile."""
    rng = np.random.default_rng(515)
    tiles = {(256, 256, 8), (128, 128, 4), (256, 160, 8), (256, 128, 8)}
    for _ in range(3000):
        M = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 9000))]))
        N = int(rng.integers(1, 4000)) * 16
        K = int(rng.integers(1, 1025)) * 16  # N * K stays below the packed-size limit
        kind, a, b, c = i8.kernel_config(M, N, K)
        shape = (M, N, K)
        if M <= 32:
            assert kind == "decode", shape
        if kind == "decode":
            assert M <= 64 and c == (M + 15) // 16 and b in (2, 4, 8), (shape, a, b, c)
            assert a in (1, 2, 3, 4, 5, 6, 8, 9, 12), (shape, a)
        elif kind == "tiled":
            assert (a, b, c) in tiles, (shape, a, b, c)
        else:
            # the second launch: 128x128 tiles (4 wavefronts) or 256xBN (8)
            assert kind == "split" and (128 if c == 4 else 256, b, c) in tiles and b < 256, \
                (shape, a, b, c)
            assert a % 256 == 0 and 0 < a < N, (shape, a)
            # the first launch's R rounds hold as many whole tile columns as fit
            tm = (M + 255) // 256
            t1 = tm * (a // 256)
            rounds = -(-t1 // 256)
            assert t1 + tm > rounds * 256, (shape, a)
