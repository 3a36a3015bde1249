#!/usr/bin/env python3
"""Throughput of the LLM.int8() decomposed matmul on one MI355X.

A step is one full int8_mixed_matmul call -- outlier detection, row
quantization with the outlier gather, and the int8 MFMA GEMM with the fused
dequantize + fp16 outlier epilogue -- on synthetic inputs already resident
in HBM.  The weight quantization is offline and not timed.

Headline: the 175B-scale FFN expansion prefill X[4096x12288] . W[12288x49152]
(alpha = 6, 7 outlier dims) in effective TOP/s = 2MNK / step time.  The
175B-scale QKV decode X[32x12288] . W[12288x36864] is measured in the same
run and reported in GB/s of compulsory bytes.  The CPU oracle is timed on a
bounded sample of the prefill workload as a reported baseline.

Prints one JSON line.  Only one GPU is used; --gpus N > 1 exits.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TOPS (2MNK/s) and % int8-MFMA peak; decode GB/s, % HBM peak"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s
# untimed load before the secondary lines (per-config, alpha = 0 ratio, layer
# shapes): the clock ramps up over tens of milliseconds after the GPU idled
WARM_MS = 100.0
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s (the alpha -> 0 path)
PREFILL = "ffn175b"
DECODE = "qkv175b_decode"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_only(text: str) -> str:
    """C/C++ source without comments and blank space: what the counters of a
    kernel depend on."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources (comments and layout ignored); the HBM
    counters committed under profiles/ carry the hash they were taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "int8_mixed_precision_outlier_amd", "csrc", "*"))):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str, launches_bytes_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def time_calls(fn, steps, warmup, both=False, warm_ms=0.0):
    """Step time from events around `steps` plain calls; then the main
    kernel's own average duration from the library's per-launch HIP events,
    which the kernel's dispatch records at its start and end on the stream
    it runs on (in a second pass, so the step timing has no timed launches).
    both=True also returns the second pass's own step time, so that the
    step minus the kernel comes from one pass (the chip's clock still moves
    over the first tens of calls); that pass includes the per-launch event
    recording, a few microseconds per call.  warm_ms > 0: after the
    `warmup` calls, keep calling until that much time has passed (the clock
    ramps up over tens of milliseconds of load, not a number of calls)."""
    import torch
    import int8_mixed_precision_outlier_amd as i8
    for s in range(warmup):
        fn(s)
    torch.cuda.synchronize()
    if warm_ms > 0:
        t_w = time.perf_counter()
        while (time.perf_counter() - t_w) * 1e3 < warm_ms:
            for s in range(8):
                fn(s)
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for s in range(steps):
        fn(s)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    i8.timing_enable(True)
    start.record()
    for s in range(steps):
        fn(s)
    stop.record()
    torch.cuda.synchronize()
    ms2 = start.elapsed_time(stop) / steps
    kern_ms, launches = i8.timing_read()
    i8.timing_enable(False)
    if both:
        return ms, kern_ms / max(launches, 1), wall, ms2
    return ms, kern_ms / max(launches, 1), wall


def stage_times(Xd, Wd, ws, alpha, n_cap, n, steps, warmup):
    """The separately callable stage exports timed alone, each on the same
    workspace: outlier detection (reads X; its export also builds the
    outlier list) and quantize + gather (reads X, writes X_i8 and the fp16
    outliers, gathers n rows of W).  Each figure includes its launch gaps.
    The whole call fuses these steps differently (for 2 <= M <= 32 it runs
    a detector and a strip quantizer that the exports do not use), so its
    own prologue is the step time minus the main kernel's.  Rates are in
    algorithmic bytes: X and the outlier rows once, the outputs once."""
    import int8_mixed_precision_outlier_amd as i8
    M, K = Xd.shape
    N = Wd.shape[1]
    ms_d, _, _ = time_calls(lambda _: i8.detect_outliers(Xd, ws, alpha=alpha, n_cap=n_cap),
                            steps, warmup)
    ms_q, _, _ = time_calls(lambda _: i8.quantize_activations(Xd, Wd, ws, n_cap=n_cap),
                            steps, warmup)
    b_d = 2 * M * K
    b_q = 2 * M * K + M * K + 4 * M + 2 * M * n + 4 * n * N
    return {"detect": {"us": round(ms_d * 1e3, 2), "bytes": b_d,
                       "GB/s": round(b_d / (ms_d * 1e-3) / 1e9, 1)},
            "quantize_gather": {"us": round(ms_q * 1e3, 2), "bytes": b_q,
                                "GB/s": round(b_q / (ms_q * 1e-3) / 1e9, 1)}}


def bench_prefill(steps, warmup, alpha, extras=True):
    import numpy as np
    import torch
    import int8_mixed_precision_outlier_amd as i8
    import synth

    w = synth.WORKLOADS[PREFILL]
    log(f"[prefill] generating {PREFILL} {w.M}x{w.K}x{w.N}")
    X, W, dims, _ = synth.make(w)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    Wi8, wabs = i8.quantize_weight(Wd)
    n_cap = i8.default_n_cap(w.K)
    ws = torch.empty(i8.workspace_size(w.M, w.K, w.N, n_cap), dtype=torch.uint8, device="cuda")
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()

    def step(_):
        i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=alpha, n_cap=n_cap, workspace=ws, out=Y)

    ms, kern_ms, wall, ms2 = time_calls(step, steps, warmup, both=True)
    n = i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["n"]
    ops = 2.0 * w.M * w.N * w.K
    log(f"[prefill] {ms:.3f} ms/step, gemm kernel {kern_ms:.3f} ms, n={n}")
    res = dict(M=w.M, K=w.K, N=w.N, n=n, ms=ms, kern_ms=kern_ms, ops=ops, wall=wall, ms2=ms2,
               sha256={"X": synth.sha256(X), "W": synth.sha256(W)})

    if not extras:
        return res, X, W
    res["stages"] = stage_times(Xd, Wd, ws, alpha, n_cap, n, steps, 2)
    log(f"[prefill] stages {res['stages']}")
    # the workload's threshold sweep: three rounds over all thresholds, a
    # few steps each, so that no threshold is always the one timed right
    # after a change of load (the chip's clock follows its power over tens
    # of calls); each threshold's best round is reported, with all rounds
    sweep = {str(a): {"rounds_ms": []} for a in w.alphas}
    for rnd in range(3):
        for a in w.alphas:
            def step_a(_, a=a):
                i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=a, n_cap=n_cap, workspace=ws, out=Y)
            ms_a, _, _ = time_calls(step_a, max(3, steps // 4), 2)
            sweep[str(a)]["rounds_ms"].append(round(ms_a, 4))
            sweep[str(a)]["n_outliers"] = i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["n"]
    for a in w.alphas:
        e = sweep[str(a)]
        e["ms_per_step"] = min(e["rounds_ms"])
        e["TOP/s"] = round(ops / (e["ms_per_step"] * 1e-3) / 1e12, 2)
        log(f"[prefill] alpha={a}: {e['ms_per_step']:.3f} ms/step (rounds {e['rounds_ms']}), "
            f"n={e['n_outliers']}")
    res["alpha_sweep"] = sweep

    # alpha = 0: every column takes the fp16 path (n = K), so the same call
    # becomes an fp16 product through this library's own kernels
    ws0 = torch.empty(i8.workspace_size(w.M, w.K, w.N, w.K), dtype=torch.uint8, device="cuda")

    def step0(_):
        i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=0.0, n_cap=w.K, workspace=ws0, out=Y)
    ms0, kern0, _ = time_calls(step0, max(3, steps // 4), 1)
    n0 = i8.read_workspace(ws0, w.M, w.K, w.N, w.K)["n"]
    res["alpha0"] = dict(ms=ms0, kern_ms=kern0, n=n0)
    log(f"[prefill] alpha=0: {ms0:.3f} ms/step (gemm kernel {kern0:.3f} ms), n={n0}")
    del ws0

    # memory-lean weights: the fp16 rows of the outlier dims only
    cache = i8.build_outlier_cache(Wd, np.asarray(sorted(dims), dtype=np.int32))

    def step_lean(_):
        i8.mixed_matmul_cached(Xd, Wi8, wabs, cache, alpha=alpha, n_cap=n_cap, workspace=ws, out=Y)
    ms_l, _, _ = time_calls(step_lean, max(3, steps // 2), 2)
    status = i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["status"]
    res["lean"] = dict(ms=ms_l, status=status, cache_bytes=cache.numel(),
                       w_i8_bytes=Wi8.numel() + 4 * w.N, w_f16_bytes=2 * w.K * w.N)
    log(f"[prefill] cached outlier rows: {ms_l:.3f} ms/step, status={status}")
    del cache

    # context: the plain fp16 product of the same shape through torch (vendor GEMM)
    def fp16(_):
        torch.matmul(Xd, Wd, out=Y)
    ms16, _, _ = time_calls(fp16, max(3, steps // 2), 2)
    res["fp16_ms"] = ms16
    log(f"[prefill] torch fp16 matmul {ms16:.3f} ms")
    return res, X, W


def alpha0_ratio(name, steps, alpha):
    """t(alpha = 0) / t(alpha) on one workload, both through this library:
    at alpha = 0 every column takes the fp16 path (n = K), so the same call
    is an fp16 product on the library's own kernels."""
    import torch
    import int8_mixed_precision_outlier_amd as i8
    import synth
    w = synth.WORKLOADS[name]
    log(f"[alpha0] generating {name} {w.M}x{w.K}x{w.N}")
    X, W, _, _ = synth.make(w)
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    Wi8, wabs = i8.quantize_weight(Wd)
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    out = {}
    for a, n_cap in ((alpha, i8.default_n_cap(w.K)), (0.0, w.K)):
        ws = torch.empty(i8.workspace_size(w.M, w.K, w.N, n_cap), dtype=torch.uint8, device="cuda")
        ms, kms, _ = time_calls(lambda _: i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=a, n_cap=n_cap,
                                                          workspace=ws, out=Y), steps, 2,
                                warm_ms=WARM_MS)
        out[str(a)] = {"ms_per_step": round(ms, 4), "gemm_kernel_ms": round(kms, 4),
                       "n_outliers": i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["n"]}
        del ws
    out["t_alpha0_over_t_alpha"] = round(out["0.0"]["ms_per_step"] / out[str(alpha)]["ms_per_step"], 3)
    log(f"[alpha0] {name}: {out}")
    return {"workload": f"{name} {w.M}x{w.K}x{w.N}", **out}


def bench_decode(steps, warmup, alpha, extras=True):
    import torch
    import int8_mixed_precision_outlier_amd as i8
    import synth

    w = synth.WORKLOADS[DECODE]
    log(f"[decode] generating {DECODE} {w.M}x{w.K}x{w.N}")
    X, W, dims, _ = synth.make(w)
    sha = {"X": synth.sha256(X), "W": synth.sha256(W)}
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    del W
    Wi8, wabs = i8.quantize_weight(Wd)
    # a second copy of the int8 weights: alternating between the two keeps
    # the 906 MB working set far above the 256 MB last-level cache, so every
    # step streams its weights from HBM
    Wi8b = Wi8.clone()
    n_cap = i8.default_n_cap(w.K)
    ws = torch.empty(i8.workspace_size(w.M, w.K, w.N, n_cap), dtype=torch.uint8, device="cuda")
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    wts = (Wi8, Wi8b)

    def step(s):
        i8.mixed_matmul(Xd, wts[s & 1], wabs, Wd, alpha=alpha, n_cap=n_cap, workspace=ws, out=Y)

    ms, kern_ms, wall, ms2 = time_calls(step, steps, warmup, both=True)
    n = i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["n"]
    nbytes = w.K * w.N + 2 * w.M * w.K + 2 * w.M * w.N + 4 * w.N + 2 * n * w.N
    log(f"[decode] {ms * 1e3:.1f} us/step, kernel {kern_ms * 1e3:.1f} us, n={n}")
    stages = graph_ms = None
    if extras:
        stages = stage_times(Xd, Wd, ws, alpha, n_cap, n, 50, 5)
        log(f"[decode] stages {stages}")
        # the same calls replayed from HIP graphs (one per weight copy): the
        # call only enqueues kernels, so it captures as is
        graphs = []
        for c in wts:
            i8.mixed_matmul(Xd, c, wabs, Wd, alpha=alpha, n_cap=n_cap, workspace=ws, out=Y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                i8.mixed_matmul(Xd, c, wabs, Wd, alpha=alpha, n_cap=n_cap, workspace=ws, out=Y)
            graphs.append(g)
        graph_ms, _, _ = time_calls(lambda s: graphs[s & 1].replay(), steps, warmup)
        log(f"[decode] graph replay {graph_ms * 1e3:.1f} us/step")
        del graphs
    return dict(M=w.M, K=w.K, N=w.N, n=n, ms=ms, kern_ms=kern_ms, bytes=nbytes, wall=wall, ms2=ms2,
                stages=stages, graph_ms=graph_ms, sha256=sha)


def bench_config(name, steps, warmup, alpha):
    """One whole call of a workload other than the headline ones (the tiny
    case, the pages' channel example, the 13B-scale FFN prefill): time per
    call, effective TOP/s (2MNK / t) and, for decode shapes, GB/s of
    compulsory bytes.  The untimed calls run for at least WARM_MS first:
    these lines follow the host-only oracle timing, after which the GPU's
    clock ramps up over tens of milliseconds of load.  Returns (record, X, W)
    so the oracle can be timed on the same inputs."""
    import torch
    import int8_mixed_precision_outlier_amd as i8
    import synth
    w = synth.WORKLOADS[name]
    log(f"[config] generating {name} {w.M}x{w.K}x{w.N}")
    X, W, _, _ = synth.make(w)
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    Wi8, wabs = i8.quantize_weight(Wd)
    n_cap = i8.default_n_cap(w.K)
    ws = torch.empty(i8.workspace_size(w.M, w.K, w.N, n_cap), dtype=torch.uint8, device="cuda")
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    ms, kms, _ = time_calls(lambda _: i8.mixed_matmul(Xd, Wi8, wabs, Wd, alpha=alpha,
                                                      n_cap=n_cap, workspace=ws, out=Y),
                            steps, warmup, warm_ms=WARM_MS)
    n = i8.read_workspace(ws, w.M, w.K, w.N, n_cap)["n"]
    ops = 2.0 * w.M * w.N * w.K
    nbytes = w.K * w.N + 2 * w.M * w.K + 2 * w.M * w.N + 4 * w.N + 2 * n * w.N
    rec = {"shape": f"{w.M}x{w.K}x{w.N}", "alpha": alpha, "n_outliers": n,
           "us_per_call": round(ms * 1e3, 2), "main_kernel_us": round(kms * 1e3, 2),
           "warmup_calls": warmup, "warmup_ms_at_least": WARM_MS,
           "TOP/s": round(ops / (ms * 1e-3) / 1e12, 2),
           "pct_int8_peak": round(100 * ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
           "GB/s_compulsory": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "kernel_config": list(i8.kernel_config(w.M, w.N, w.K))}
    log(f"[config] {name}: {rec}")
    del Xd, Wd, Wi8, wabs, ws, Y
    torch.cuda.empty_cache()
    return rec, X, W


def oracle_time(X, W, alpha, runs=3):
    """The oracle's whole call (detection, quantization, exact integer GEMM,
    dequantize + outlier sum, fp16 cast) on host arrays: median seconds of
    `runs` runs.  The offline weight quantization is not timed."""
    import numpy as np
    import oracle as O
    Wq, aw = O.quantize_weight(W)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        O.mixed_matmul(X, Wq, aw, W, alpha).Y16
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    M, K = X.shape
    N = W.shape[1]
    return {"seconds_median": round(t, 4), "runs": runs,
            "TOP/s": round(2.0 * M * N * K / t / 1e12, 4)}


def cpu_baseline(X, W, alpha, target_s):
    """The oracle as it stands, on a bounded sample of the prefill workload:
    outlier detection over the full X, then quantization, exact integer GEMM
    and dequantize + outlier sum for the first `rows` rows and `cols` output
    columns.  The sample grows until one run lasts about `target_s` seconds
    or covers the whole workload, which is then repeated up to `target_s`.
    Work is scaled to effective TOP/s like the GPU figure."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    M, K = X.shape
    N = W.shape[1]

    def run(rows, cols):
        Wc = np.ascontiguousarray(W[:, :cols])
        Wq, aw = O.quantize_weight(Wc)  # offline step, not timed
        t0 = time.perf_counter()
        idx = O.detect_outliers(X, alpha)
        Xq, ax = O.quantize_activations(X[:rows], idx)
        Xo, Wo = O.gather_outliers(X[:rows], Wc, idx)
        A = O.int_gemm(Xq, Wq)
        O.dequant_sum(A, ax, aw, Xo, Wo).astype(np.float16)
        t = time.perf_counter() - t0
        log(f"[cpu] rows={rows} cols={cols}: {t:.2f} s")
        return t

    # grow the sample (rows, then columns) until one run lasts target_s or
    # covers the whole workload; at full size repeat runs up to target_s
    rows, cols = min(M, 512), min(N, 4096)
    while True:
        t = run(rows, cols)
        if t >= target_s or (rows, cols) == (M, N):
            break
        grow = max(2.0, min(8.0, 0.8 * target_s / max(t, 1e-3)))
        if rows < M:
            rows = min(M, int(rows * grow))
        else:
            cols = min(N, int(cols * grow) // 1024 * 1024 or N)
    runs, total = 1, t
    while total < target_s and (rows, cols) == (M, N):
        total += run(rows, cols)
        runs += 1
    t = total / runs
    ops = 2.0 * rows * cols * K
    return {"value": round(ops / t / 1e12, 4), "unit": "TOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{PREFILL}: outlier detection over all {M} rows, then rows 0..{rows - 1} x "
                      f"output cols 0..{cols - 1} (K={K}); numpy fp64 BLAS; mean of {runs} "
                      f"run(s), {t:.2f} s each",
            "seconds": round(t, 3), "host_cpus": len(os.sched_getaffinity(0))}


def operand_sweep():
    """The same int8 GEMM (int32 output, prefill shape) on operands of
    different value statistics: the chip's clock under this kernel depends
    on how many operand bits toggle, so the time does too."""
    import torch
    import int8_mixed_precision_outlier_amd as i8
    w = synth_workload(PREFILL)
    M, K, N = w.M, w.K, w.N
    g = torch.Generator(device="cuda")
    g.manual_seed(1)

    def make(kind, rows):
        if kind == "uniform":
            return torch.randint(-127, 128, (rows, K), dtype=torch.int8, device="cuda", generator=g)
        if kind == "normal25":
            return (torch.randn((rows, K), device="cuda", generator=g) * 25).round().clamp(
                -127, 127).to(torch.int8)
        if kind == "ternary":
            return torch.randint(-1, 2, (rows, K), dtype=torch.int8, device="cuda", generator=g)
        return torch.zeros((rows, K), dtype=torch.int8, device="cuda")

    Wp = i8.pack_rows(make("uniform", N))
    out = torch.empty((M, N), dtype=torch.int32, device="cuda")
    res = {}
    for kind in ("uniform", "normal25", "ternary", "zeros"):
        Xp = i8.pack_rows(make(kind, M))
        ms, _, _ = time_calls(lambda _: i8.gemm_i32(Xp, Wp, M, N, K, out=out), 10, 3)
        res[kind] = {"ms": round(ms, 4), "TOP/s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        log(f"[operands] X {kind}: {ms:.3f} ms")
    return {"workload": f"{PREFILL} int8 K-loop, W uniform in [-127,127]", "X": res}


def layer_shapes():
    """The layers the pages analyse for outliers ("論文閱讀 : LLM.int8(): 8-bit
    Matrix Multiplication for Transformers at Scale", hackmd.io/@KuoDong,
    section 隨模型規模擴大而出現的「極端特徵值」, Outlier 定義: attention
    Q/K/V/output projections and the FFN expansion) at 13B (hidden 5120) and
    175B (hidden 12288) scale, prefill
    (M = 2048 / 4096 tokens) and decode (M = 32).  Synthetic activations with
    7 outlier dims of magnitude 20..60 in 75 % of the rows, weights
    N(0, 0.02^2).  Reports the call's time, effective TOP/s, the weight
    streaming rate and the torch fp16 product of the same shape.  At M = 32
    both sides rotate through enough weight copies (>= 768 MB) that every
    call streams its weights from HBM, as a model's successive layers do."""
    import torch
    import int8_mixed_precision_outlier_amd as i8
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    out = []
    for model, hid, m_pre in (("13B", 5120, 2048), ("175B", 12288, 4096)):
        for layer, K, N in (("qkv", hid, 3 * hid), ("out_proj", hid, hid),
                            ("ffn_expansion", hid, 4 * hid)):
            W = (torch.randn((K, N), device="cuda", generator=g) * 0.02).half()
            Wi8, wabs = i8.quantize_weight(W)
            # rotate enough copies (>= 768 MB) that decode streams its
            # weights from HBM, not from the 256 MB last-level cache
            ncopy = max(2, -(-(768 << 20) // Wi8.numel()))
            wts = [Wi8] + [Wi8.clone() for _ in range(ncopy - 1)]
            dims = torch.randperm(K, device="cuda", generator=g)[:7]
            for M in (m_pre, 32):
                X = torch.randn((M, K), device="cuda", generator=g).clamp_(-5, 5)
                rows = torch.rand(M, device="cuda", generator=g) < 0.75
                mag = torch.rand((M, 7), device="cuda", generator=g) * 40 + 20
                sub = X[:, dims]
                sub[rows] = (mag * torch.sign(torch.randn((M, 7), device="cuda", generator=g)))[rows]
                X[:, dims] = sub
                X = X.half()
                n_cap = i8.default_n_cap(K)
                ws = torch.empty(i8.workspace_size(M, K, N, n_cap), dtype=torch.uint8, device="cuda")
                Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                steps = 50 if M == 32 else 10
                ms, kms, _ = time_calls(lambda s: i8.mixed_matmul(
                    X, wts[s % len(wts)], wabs, W, alpha=6.0, n_cap=n_cap, workspace=ws, out=Y),
                    steps, 3, warm_ms=WARM_MS)
                w16 = [W] + ([W.clone() for _ in range(max(1, -(-(768 << 20) // (2 * W.numel()))))]
                             if M == 32 else [])
                ms16, _, _ = time_calls(lambda s: torch.matmul(X, w16[s % len(w16)], out=Y), steps, 3,
                                        warm_ms=WARM_MS)
                del w16
                ops = 2.0 * M * N * K
                rec = {"model": model, "layer": layer, "M": M, "K": K, "N": N,
                       "ms": round(ms, 4), "kernel_ms": round(kms, 4),
                       "TOP/s": round(ops / (ms * 1e-3) / 1e12, 1),
                       "weight_GB/s": round(K * N / (ms * 1e-3) / 1e9, 0),
                       "torch_fp16_ms": round(ms16, 4), "speedup_vs_fp16": round(ms16 / ms, 3)}
                log(f"[layers] {rec}")
                out.append(rec)
                del X, ws, Y
            del W, Wi8, wts
            torch.cuda.empty_cache()
    return {"layer_shapes": out}


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, pattern):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    return hits[0] if hits else None


def _per_dispatch(d, counter, name_has):
    """Mean of `counter` per dispatch of the kernels whose name contains
    name_has, from a rocprofv3 --pmc counter_collection CSV under d."""
    path = _find(d, "*counter_collection.csv")
    if path is None:
        return None, 0
    per = {}
    for r in _read_csv(path):
        if r.get("Counter_Name") != counter or name_has not in r.get("Kernel_Name", ""):
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)


def _trace_table(d, title, command, note, last_n=20):
    """Markdown summary of a rocprofv3 --kernel-trace run under d: per
    kernel, calls, mean / min / max / median duration, the mean of the last
    last_n calls and the share of the total."""
    path = _find(d, "*kernel_trace.csv")
    rows = _read_csv(path)
    by = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), dur))
    total = sum(dd for v in by.values() for _, dd in v)
    out = [f"# {title}", "", "Command (from the repository root on the MI355X host):", "", "```",
           command, "```", "", note, "",
           "| kernel | calls | avg us | min us | max us | median us | avg of the last %d calls us | total %% |" % last_n,
           "|---|---|---|---|---|---|---|---|"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(dd for _, dd in kv[1])):
        v.sort()
        ds = [dd for _, dd in v]
        srt = sorted(ds)
        med = srt[len(srt) // 2]
        last = ("%.2f" % (sum(ds[-last_n:]) / len(ds[-last_n:]))) if len(ds) >= last_n else "-"
        short = name.split("(")[0].replace("void ", "")
        out.append(f"| `{short}` | {len(ds)} | {sum(ds) / len(ds):.2f} | {srt[0]:.2f} | {srt[-1]:.2f} "
                   f"| {med:.2f} | {last} | {100 * sum(ds) / total:.2f} |")
    return "\n".join(out) + "\n"


def _bench_line(log):
    """The JSON line bench.py printed in a profiled run (None if absent)."""
    if not os.path.exists(log):
        return None
    for line in reversed(open(log, errors="replace").read().splitlines()):
        if line.startswith("{"):
            try:
                return json.loads(line)
            except ValueError:
                return None
    return None


MFMA_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA")


def _mfma_clock_table(d, h):
    """profiles/ table of the prefill GEMM's shader clock and MFMA
    utilisation per dispatch, from one rocprofv3 --pmc run of MFMA_COUNTERS
    under d.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, so cycles per XCD
    = GRBM / 8; clock = those cycles / the dispatch's duration; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD x 1024 SIMDs)."""
    path = _find(d, "*counter_collection.csv")
    if path is None:
        return None
    per = {}
    for r in _read_csv(path):
        if "k_gemm<" not in r.get("Kernel_Name", ""):
            continue
        e = per.setdefault(int(r["Dispatch_Id"]), {"dur": (int(r["End_Timestamp"]) -
                                                           int(r["Start_Timestamp"])) / 1e3})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    cmd = ("rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + " --kernel-trace --output-format csv "
           "-d <out>/prefill_mfma -o run -- python3 bench.py --only prefill --steps 3 --warmup 1")
    out = [f"# k_gemm on {PREFILL}: shader clock and MFMA utilisation (rocprofv3 PMC)", "",
           "Command (from the repository root, TMPDIR=/tmp):", "", "```", cmd, "```", "",
           "Summarized by `python3 bench.py --summarize-profiles <out>`. GRBM_GUI_ACTIVE is summed "
           "over the 8 XCDs (an MFMA-only probe at a known 2.24 GHz reads 8x its cycle count), so "
           "cycles per XCD = GRBM/8 and clock = cycles / kernel duration. MFMA utilisation = "
           "SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD x 1024 SIMDs). Kernel sources hash "
           f"`{h}`.", "",
           "| dispatch | duration us | GRBM/8 cycles | clock GHz | MFMA instructions | MFMA busy % |",
           "|---|---|---|---|---|---|"]
    for k in sorted(per):
        e = per[k]
        if not all(c in e for c in MFMA_COUNTERS):
            continue
        cyc = e["GRBM_GUI_ACTIVE"] / 8
        out.append(f"| {k} | {e['dur']:.1f} | {cyc:.4g} | {cyc / (e['dur'] * 1e3):.2f} | "
                   f"{e['SQ_INSTS_MFMA']:.4g} | {100 * e['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1f} |")
    return "\n".join(out) + "\n"


def summarize_profiles(d):
    """Write the profiles/ summaries from the raw rocprofv3 output of the
    commands they name (run from the repository root into directory d):
    <d>/prefill_trace and <d>/decode_trace (--kernel-trace),
    <d>/{copy,prefill,decode}_{FETCH_SIZE,WRITE_SIZE} (--pmc, one counter
    per run), <d>/prefill_mfma (--pmc MFMA_COUNTERS), <d>/layers.json
    (bench.py --layer-shapes) and <d>/operands.json (bench.py
    --operand-sweep)."""
    prof = os.path.join(ROOT, "profiles")
    h = kernel_source_hash()
    pre, dec = synth_workload(PREFILL), synth_workload(DECODE)
    if os.path.isdir(os.path.join(d, "prefill_mfma")):
        t = _mfma_clock_table(os.path.join(d, "prefill_mfma"), h)
        if t:
            with open(os.path.join(prof, f"k_gemm_{PREFILL}_mfma_clock.md"), "w") as f:
                f.write(t)
    ops = _bench_line(os.path.join(d, "operands.json"))
    if ops and ops.get("X"):
        out = [f"# k_gemm K-loop on the {PREFILL} shape: time against operand statistics", "",
               "Command (from the repository root):", "", "```",
               "python3 bench.py --operand-sweep > <out>/operands.json", "```", "",
               f"Summarized by `python3 bench.py --summarize-profiles <out>`. The same int8 GEMM "
               f"(int32 output, {pre.M}x{pre.K}x{pre.N}, W uniform in [-127, 127]) with four kinds "
               "of activations. Only the operand values change; the instruction stream is "
               "identical. The spread is the chip's clock under this kernel following the MFMA "
               f"switching power: the kernel is power-bound. Kernel sources hash `{h}`.", "",
               "| X values | ms | TOP/s |", "|---|---|---|"]
        for k, v in ops["X"].items():
            out.append(f"| {k} | {v['ms']} | {v['TOP/s']} |")
        with open(os.path.join(prof, f"k_gemm_{PREFILL}_operand_statistics.md"), "w") as f:
            f.write("\n".join(out) + "\n")
    tcmd = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <out>/{w}_trace -o run "
            "--output-format csv -- python3 /root/repo/bench.py --only {w}{extra}")
    if os.path.isdir(os.path.join(d, "prefill_trace")):
        note = (f"One step = k_colmax_part + k_detect (two-pass column absmax) + k_quant_act + k_gemm "
                f"on {PREFILL} ({pre.M}x{pre.K}x{pre.N}, alpha 6). The run also holds the one-time "
                "weight quantization and the calls bench.py makes: warm-up, timed, and timed again with "
                "per-launch events; the last calls are those whose events give `roofline.achieved`. "
                f"Kernel sources hash `{h}`.")
        b = _bench_line(os.path.join(d, "prefill_trace.log"))
        tail = ""
        if b and b.get("kernel_ms"):
            tail = (f"\nbench.py's own per-launch events for the main kernel in this traced run: "
                    f"{1e3 * b['kernel_ms']:.2f} us (whole step "
                    f"{1e3 * b['ms_per_step']:.2f} us; the profiler's per-dispatch tracing adds to "
                    "the step).\n")
        with open(os.path.join(prof, f"k_gemm_{PREFILL}_kernel_trace.md"), "w") as f:
            f.write(_trace_table(os.path.join(d, "prefill_trace"),
                                 f"Kernel trace, {PREFILL} prefill",
                                 tcmd.format(w="prefill", extra=""), note) + tail)
    if os.path.isdir(os.path.join(d, "decode_trace")):
        note = (f"One step = k_detect_small + k_quant_strips + k_decode_mm on {DECODE} "
                f"({dec.M}x{dec.K}x{dec.N}, alpha 6; two weight copies alternate so the weights "
                f"stream from HBM). Kernel sources hash `{h}`.")
        b = _bench_line(os.path.join(d, "decode_trace.log"))
        tail = ""
        if b and b.get("kernel_ms"):
            tail = (f"\nbench.py's own per-launch events for the decode kernel in this traced run: "
                    f"{1e3 * b['kernel_ms']:.2f} us (whole step {1e3 * b['ms_per_step']:.2f} us; "
                    "under the profiler the event-recording dispatches run longer than the traced "
                    "kernel itself, which the untraced bench run does not show).\n")
        with open(os.path.join(prof, f"k_decode_{DECODE}_kernel_trace.md"), "w") as f:
            f.write(_trace_table(os.path.join(d, "decode_trace"),
                                 f"Kernel trace, {DECODE} decode",
                                 tcmd.format(w="decode", extra=" --decode-steps 50"), note, 50)
                    + tail)
    lay = _bench_line(os.path.join(d, "layers.json"))
    if lay and lay.get("layer_shapes"):
        out = ["# Layer coverage: attention projections and FFN expansion, 13B and 175B scale", "",
               "Command (from the repository root):", "", "```",
               "python3 bench.py --layer-shapes > <out>/layers.json", "```", "",
               "Synthetic activations (7 outlier dims, |x| in 20..60 in 75 % of rows, normals clipped "
               "at 5), weights N(0, 0.02^2); alpha = 6; decode (M = 32) rotates enough weight copies "
               "(>= 768 MB, for the int8 call and for torch) that the weights stream from HBM rather "
               "than the 256 MB last-level cache. `call ms` is the whole call (detection, "
               "quantization, GEMM); `kernel ms` the GEMM or decode kernel alone, from the events "
               "its dispatch records (a separate pass); torch fp16 is `torch.matmul` on the same "
               f"fp16 operands. Kernel sources hash `{h}`.", "",
               "| model | layer | M | K | N | call ms | kernel ms | TOP/s | weight GB/s | torch fp16 ms "
               "| int8 call vs fp16 |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in lay["layer_shapes"]:
            out.append(f"| {r['model']} | {r['layer']} | {r['M']} | {r['K']} | {r['N']} | {r['ms']} | "
                       f"{r['kernel_ms']} | {r['TOP/s']} | {r['weight_GB/s']} | {r['torch_fp16_ms']} | "
                       f"{r['speedup_vs_fp16']}x |")
        with open(os.path.join(prof, "layer_shapes_13b_175b.md"), "w") as f:
            f.write("\n".join(out) + "\n")
    cf, _ = _per_dispatch(os.path.join(d, "copy_FETCH_SIZE"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _per_dispatch(os.path.join(d, "copy_WRITE_SIZE"), "WRITE_SIZE", "copyBuffer")
    if cf is None or cw is None:
        return
    fs, ws = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
    lines = []
    for tag, name_has, wl, alg in (
            ("gemm", "k_gemm<", PREFILL, "6.54e8 compulsory operands (X_i8 + W_i8 + epilogue "
                                          "operands) and 4.03e8 of Y; operand panels re-read per tile"),
            ("decode", "k_decode_mm<", DECODE, "4.568e8 (compulsory bytes of the whole step)")):
        kind = "prefill" if tag == "gemm" else "decode"
        f_kib, n1 = _per_dispatch(os.path.join(d, f"{kind}_FETCH_SIZE"), "FETCH_SIZE", name_has)
        w_kib, n2 = _per_dispatch(os.path.join(d, f"{kind}_WRITE_SIZE"), "WRITE_SIZE", name_has)
        if f_kib is None or w_kib is None:
            continue
        total = int(f_kib * 1024 * fs + w_kib * 1024 * ws)
        rec = {"source_hash": h, "kernel": name_has, "workload": wl, "launches": min(n1, n2),
               "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": fs, "write_scale": ws,
               "hbm_bytes_per_launch": total}
        with open(os.path.join(prof, f"{tag}_{wl}_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        w_ = synth_workload(wl)
        lines.append(f"| `{name_has}` | {wl} {w_.M}x{w_.K}x{w_.N} | {min(n1, n2)} | {f_kib:.1f} | "
                     f"{w_kib:.1f} | {total:.4g} | {alg} |")
    pcmd = ("rocprofv3 --pmc {c} --kernel-trace --output-format csv -d <out>/{k}_{c} -o run -- "
            "python3 bench.py {a}")
    args = {"copy": "--copy-calibration", "prefill": "--only prefill --steps 3 --warmup 1 --no-peaks",
            "decode": "--only decode --decode-steps 10 --warmup 2 --no-peaks"}
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Each counter in a run of its own, from the repository root (TMPDIR=/tmp):", "", "```"]
    for k in ("copy", "prefill", "decode"):
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            md.append(pcmd.format(c=c, k=k, a=args[k]))
    md += ["```", "", "Summarized by `python3 bench.py --summarize-profiles <out>`.", "",
           f"Calibration: a plain 1 GiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = "
           f"{cf:.1f} KiB and WRITE_SIZE = {cw:.1f} KiB per launch, so bytes = KiB x 1024 x {fs:.4f} "
           f"(fetch) and x {ws:.4f} (write).", "",
           f"Kernel sources hash (code without comments or layout): `{h}`", "",
           "| kernel | workload | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch (scaled) "
           "| algorithmic bytes / launch |", "|---|---|---|---|---|---|---|"] + lines
    with open(os.path.join(prof, f"hbm_traffic_{PREFILL}_{DECODE}.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def synth_workload(name):
    import synth
    return synth.WORKLOADS[name]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed calls first (the clock settles over the first ~20 prefill calls)")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--alpha", type=float, default=6.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target duration of the CPU-oracle baseline sample (0: skip)")
    ap.add_argument("--only", choices=("all", "prefill", "decode"), default="all",
                    help="profiling runs: time one workload only, no sweep or context")
    ap.add_argument("--layer-shapes", action="store_true",
                    help="time the call on the attention projection and FFN expansion shapes "
                         "of 13B- and 175B-scale layers, prefill and decode, and exit")
    ap.add_argument("--operand-sweep", action="store_true",
                    help="time the int8 K-loop (int32 output) on the prefill shape with "
                         "operands of different value statistics and exit")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the MFMA-only and streaming-read peak probes")
    ap.add_argument("--peaks", action="store_true",
                    help="run only the peak probes (measured ceilings) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy a few times and exit (the "
                         "reference kernel that scales the HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the raw rocprofv3 output under DIR "
                         "(no GPU needed) and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only: the library computes one GPU's "
              "share of a layer and has no multi-GPU mode (a tensor-parallel layer would give "
              "each GPU a slice of W's columns and run this same call on it).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_mixed_precision_outlier_amd as i8
    i8.load()  # fails loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.layer_shapes:
        print(json.dumps(layer_shapes()), flush=True)
        return
    if args.peaks:
        from int8_mixed_precision_outlier_amd import probes
        print(json.dumps(probes.measure_peaks()), flush=True)
        return
    if args.operand_sweep:
        print(json.dumps(operand_sweep()), flush=True)
        return
    if args.copy_calibration:
        nbytes = 1 << 30
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                          "launches": 4}), flush=True)
        return
    if args.only == "prefill":
        pre, _, _ = bench_prefill(args.steps, args.warmup, args.alpha, extras=False)
        print(json.dumps({"workload": PREFILL, "ms_per_step": pre["ms"],
                          "kernel_ms": pre["kern_ms"]}), flush=True)
        return
    if args.only == "decode":
        dec = bench_decode(args.decode_steps, args.warmup, args.alpha, extras=False)
        print(json.dumps({"workload": DECODE, "ms_per_step": dec["ms"],
                          "kernel_ms": dec["kern_ms"]}), flush=True)
        return

    pre, X, W = bench_prefill(args.steps, args.warmup, args.alpha)
    dec = bench_decode(args.decode_steps, args.warmup, args.alpha)
    a0_13b = alpha0_ratio("ffn13b", max(5, args.steps // 2), args.alpha)
    cpu = cpu_baseline(X, W, args.alpha, args.cpu_seconds) if args.cpu_seconds > 0 else None
    del X, W
    # the other configurations: whole-call lines, and the oracle on each
    per_config = {}
    for name in ("tiny", "channel", "ffn13b"):
        rec, Xc, Wc = bench_config(name, max(args.steps, 50 if name == "tiny" else 20),
                                   args.warmup, args.alpha)
        if args.cpu_seconds > 0:
            rec["oracle"] = oracle_time(Xc, Wc, args.alpha)
            log(f"[cpu] {name}: {rec['oracle']}")
        per_config[name] = rec
        del Xc, Wc
    if args.cpu_seconds > 0:
        import synth
        Xc, Wc, _, _ = synth.make(DECODE)
        dec["oracle"] = oracle_time(Xc, Wc, args.alpha)
        log(f"[cpu] {DECODE}: {dec['oracle']}")
        del Xc, Wc
    peaks = None
    if not args.no_peaks:
        from int8_mixed_precision_outlier_amd import probes
        peaks = probes.measure_peaks()
        log(f"[peaks] {peaks}")

    tops = pre["ops"] / (pre["ms"] * 1e-3) / 1e12
    k_tops = pre["ops"] / (pre["kern_ms"] * 1e-3) / 1e12
    gbs = dec["bytes"] / (dec["ms"] * 1e-3) / 1e9
    k_gbs = dec["bytes"] / (dec["kern_ms"] * 1e-3) / 1e9
    traffic = traffic_from_profile(f"gemm_{PREFILL}", pre["ops"])
    dtraffic = traffic_from_profile(f"decode_{DECODE}", dec["bytes"])
    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{PREFILL}: 175B-scale FFN expansion prefill, X[{pre['M']}x{pre['K']}] fp16 "
                        f". W[{pre['K']}x{pre['N']}] fp16 (int8 pre-quantized), alpha={args.alpha}, "
                        f"{pre['n']} outlier dims",
            "M": pre["M"], "K": pre["K"], "N": pre["N"], "alpha": args.alpha,
            "n_outliers": pre["n"], "parallelism": "single GPU",
            "inputs_sha256": pre["sha256"],
        },
        "pct_int8_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
        "roofline": {
            "kernel": "k_gemm (int8 MFMA + fused dequant/outlier epilogue)",
            "bound": "mfma", "achieved": round(k_tops, 2), "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s", "frac": round(k_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "algorithmic_per_launch": pre["ops"], "kernel_ms": round(pre["kern_ms"], 4),
            "measured_peak": None if peaks is None else peaks["mfma_i8_random_operands_TOP/s"],
            "frac_of_measured_peak": None if peaks is None else round(
                k_tops / peaks["mfma_i8_random_operands_TOP/s"], 4),
        },
        "measured_peaks": peaks,
        "per_config": per_config,
        # the second (kernel-timed) pass's step minus its kernel (the headline
        # pass runs earlier, while the clock still rises; the second pass
        # also holds the per-launch event recording, a few us per call)
        "prologue_ms_per_step": round(pre["ms2"] - pre["kern_ms"], 4),
        "second_pass_ms_per_step": round(pre["ms2"], 4),
        # the same call at steady state: its best round in the threshold sweep
        "steady_state_ms_per_step": pre["alpha_sweep"].get(str(args.alpha), {}).get("ms_per_step"),
        "stage_exports_alone": pre["stages"],
        "alpha_sweep": pre["alpha_sweep"],
        "fp16_context": {"torch_fp16_matmul_ms": round(pre["fp16_ms"], 4),
                         "speedup_vs_fp16": round(pre["fp16_ms"] / pre["ms"], 3)},
        "lean_weights": {
            "ms_per_step": round(pre["lean"]["ms"], 4), "status": pre["lean"]["status"],
            "resident_bytes_vs_fp16": round(
                (pre["lean"]["w_i8_bytes"] + pre["lean"]["cache_bytes"]) / pre["lean"]["w_f16_bytes"], 5),
            "with_full_fp16_w_vs_fp16": round(
                (pre["lean"]["w_i8_bytes"] + pre["lean"]["w_f16_bytes"]) / pre["lean"]["w_f16_bytes"], 5),
            "cache_bytes": pre["lean"]["cache_bytes"]},
        "fp16_path_alpha0": {
            "ms_per_step": round(pre["alpha0"]["ms"], 4), "n_outliers": pre["alpha0"]["n"],
            "gemm_kernel_ms": round(pre["alpha0"]["kern_ms"], 4),
            "fp16_TFLOP/s": round(pre["ops"] / (pre["alpha0"]["kern_ms"] * 1e-3) / 1e12, 1),
            "frac_of_fp16_peak": round(pre["ops"] / (pre["alpha0"]["kern_ms"] * 1e-3) / 1e12
                                       / PEAK_FP16_TFLOPS, 4),
            "frac_of_measured_fp16_peak": None if peaks is None else round(
                pre["ops"] / (pre["alpha0"]["kern_ms"] * 1e-3) / 1e12
                / peaks["mfma_f16_random_operands_TFLOP/s"], 4),
            "t_alpha0_over_t_alpha": round(pre["alpha0"]["ms"] / pre["ms"], 3),
            "ffn13b": a0_13b},
        "cpu_baseline": cpu,
        "decode": {
            "workload": f"{DECODE}: 175B-scale QKV decode, X[{dec['M']}x{dec['K']}] . "
                        f"W[{dec['K']}x{dec['N']}], {dec['n']} outlier dims",
            "value": round(gbs, 1), "unit": "GB/s", "steps": args.decode_steps,
            "us_per_step": round(dec["ms"] * 1e3, 2),
            "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "compulsory_bytes": dec["bytes"],
            "inputs_sha256": dec["sha256"],
            "roofline": {
                "kernel": "k_decode (int8 weight streaming)", "bound": "hbm",
                "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(k_gbs / PEAK_HBM_GBS, 4), "traffic": dtraffic,
                "kernel_us": round(dec["kern_ms"] * 1e3, 2),
                "measured_peak": None if peaks is None else peaks["hbm_read_nontemporal_GB/s"],
                "frac_of_measured_peak": None if peaks is None else round(
                    k_gbs / peaks["hbm_read_nontemporal_GB/s"], 4),
            },
            "oracle": dec.get("oracle"),
            "prologue_us_per_step": round((dec["ms"] - dec["kern_ms"]) * 1e3, 2),
            "stage_exports_alone": dec["stages"],
            "graph_replay": None if dec["graph_ms"] is None else {
                "us_per_step": round(dec["graph_ms"] * 1e3, 2),
                "GB/s": round(dec["bytes"] / (dec["graph_ms"] * 1e-3) / 1e9, 1)},
        },
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
