"""Binding of libint8mm_probes.so: the chip's measured ceilings.

measure_peaks() times an MFMA-only int8 loop (random and fixed operands) and
a streaming read of a buffer far larger than the 256 MB last-level cache
(plain and nontemporal loads) on the current device.  The roofline
fractions of the matmul kernels are reported against these as well as
against the published peaks (5.0 POP/s int8 MFMA, 8 TB/s HBM3E).
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint8mm_probes.so")
_lib = None
_vp, _i64 = ctypes.c_void_p, ctypes.c_int64


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m int8_mixed_precision_outlier_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.int8mm_probe_mfma_i8.restype = ctypes.c_int
        lib.int8mm_probe_mfma_i8.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp]
        lib.int8mm_probe_mfma_f16.restype = ctypes.c_int
        lib.int8mm_probe_mfma_f16.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp]
        lib.int8mm_probe_read.restype = ctypes.c_int
        lib.int8mm_probe_read.argtypes = [_vp, ctypes.c_size_t, ctypes.c_int, _i64, _vp, _vp]
        _lib = lib
    return _lib


def _time(fn, reps: int) -> float:
    """Median milliseconds of `reps` launches (after one untimed launch)."""
    fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2]


def mfma_i8_tops(random: bool = True, iters: int = 20000, reps: int = 5) -> float:
    """TOP/s of the MFMA-only loop over every compute unit (2 workgroups of
    4 wavefronts per CU)."""
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    ops_buf = torch.randint(-127, 128, (8 * 1024,), dtype=torch.int8, device="cuda", generator=g)
    sink = torch.empty((blocks * 256,), dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        rc = lib.int8mm_probe_mfma_i8(ctypes.c_void_p(ops_buf.data_ptr()), int(random), blocks,
                                      iters, ctypes.c_void_p(sink.data_ptr()), st)
        if rc != 0:
            raise RuntimeError(f"MFMA probe launch failed: hipError {rc}")
    ms = _time(run, reps)
    ops = blocks * 4 * iters * 8 * 32768
    return ops / (ms * 1e-3) / 1e12


def mfma_f16_tflops(random: bool = True, iters: int = 20000, reps: int = 5) -> float:
    """TFLOP/s of the fp16 MFMA-only loop (v_mfma_f32_16x16x32_f16), same
    occupancy as mfma_i8_tops, on random halves in [-2, 2)."""
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    ops_buf = (torch.rand((4 * 1024,), device="cuda", generator=g) * 4.0 - 2.0).half()
    sink = torch.empty((blocks * 256,), dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        rc = lib.int8mm_probe_mfma_f16(ctypes.c_void_p(ops_buf.data_ptr()), int(random), blocks,
                                       iters, ctypes.c_void_p(sink.data_ptr()), st)
        if rc != 0:
            raise RuntimeError(f"fp16 MFMA probe launch failed: hipError {rc}")
    ms = _time(run, reps)
    flops = blocks * 4 * iters * 8 * 16384
    return flops / (ms * 1e-3) / 1e12


def read_gbs(nbytes: int = 4 << 30, nontemporal: bool = False, reps: int = 5) -> float:
    """GB/s of a streaming read of `nbytes` (default 4 GiB: 16x the
    last-level cache, so it comes from HBM)."""
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus
    buf = torch.empty((nbytes,), dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.empty((blocks,), dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        rc = lib.int8mm_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, int(nontemporal),
                                   blocks, ctypes.c_void_p(sink.data_ptr()), st)
        if rc != 0:
            raise RuntimeError(f"read probe launch failed: hipError {rc}")
    ms = _time(run, reps)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def measure_peaks() -> dict:
    """The measured ceilings, one dict (TOP/s and GB/s)."""
    return {
        "mfma_i8_random_operands_TOP/s": round(mfma_i8_tops(True), 1),
        "mfma_i8_fixed_operands_TOP/s": round(mfma_i8_tops(False), 1),
        "mfma_f16_random_operands_TFLOP/s": round(mfma_f16_tflops(True), 1),
        "hbm_read_GB/s": round(read_gbs(nontemporal=False), 1),
        "hbm_read_nontemporal_GB/s": round(read_gbs(nontemporal=True), 1),
        "probe": "MFMA: 2 workgroups x 4 wavefronts per CU, 8 v_mfma_i32_16x16x64_i8 (or "
                 "v_mfma_f32_16x16x32_f16) per iteration on 4 accumulators, no memory "
                 "traffic; read: 4 GiB with 16-byte loads, 4 in flight per thread, 8 "
                 "workgroups of 256 threads per CU",
    }
