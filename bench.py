#!/usr/bin/env python3
"""Benchmark of the gfx950 NVFP4 weight quantizer on one MI355X.

Workload: 4096 x 4096 bf16 attention-projection-shaped weights (Student-t, nu = 4, std 0.02, plus
outlier columns scaled by 20). Twelve distinct matrices (384 MiB, more than the 256 MB Infinity Cache)
stay resident in HBM and are visited in turn, so each step starts from HBM rather than from cache.

One step = one matrix quantised in each of the four modes, back to back on one stream:
MAX, FourOverSix, CJSO (8 rounds), SOAR (CJSO(8) + the decoupled search). Consecutive steps (different
matrices, separate outputs and workspaces) rotate over three HIP streams, the way a model's
independent weight matrices are quantised (three streams and torch's default stream use the four
hardware queues a process gets; two streams give about 10 % less, four share a queue and lose);
`single_stream_ms_per_step` gives the same steps on one stream. `value` is the weight bytes quantised per second (4 x 32 MiB per step). Per mode the JSON line
also gives its own GB/s and its share of the HBM peak.

The dominant kernel is the CJSO round (k_cjso_iter): sixteen launches per step, fourteen of them rounds
other than the last (the roofline kernel). It is timed live: the
library records HIP events around each of its kernels on the stream it launches them on (the
`stage_events` hook of the C ABI). Its achieved rate is algorithmic bytes / duration against the 8 TB/s
HBM peak; a round that is not the last reads the block (2 B per element) and its scale byte and writes
the new scale byte: 2.125 B per element. The search is reported the same way (2.75 B per element:
read the block, its scale and its two-byte scale bracket; write codes and scale), and once more with
NVFP4_FLAG_FULL_SEARCH (all 202 candidates) against the FP32 vector peak: per block 101 quantise
scales x 16 elements x 9 FLOPs.

w4a16: the W4A16 product the format is for, Y = X @ What.T with the quantised 4096 x 4096 weights, at
M = 1, 16 and 64 (GB/s against HBM peak), 256, 1024 and 4096 (TFLOP/s against the 2.5 PFLOP/s bf16 MFMA
peak), each beside torch's dense bf16 product.

c5_whole_model: the 224 matrices of a 7B-shaped model (32 layers; 12.95 GB bf16) quantised one after
another in each mode, total time and aggregate GB/s, and the same for its 128 square 4096 x 4096
matrices alone (skipped with --no-c5).

cold_warm: one call per mode timed alone, "cold" after a 1 GiB fill has evicted the Infinity Cache,
and "warm" repeated at once.

fp32_input: the first matrix widened to fp32, one warm call per mode (the binary32 input path).

quality: the reconstruction MSE of each mode and search variant on the first matrix (GPU error statistics),
its ratio to the max rule's, and the time of one call with those settings.

c3_mlp: the MLP-shaped matrices (14336 x 4096 and 4096 x 14336 bf16) in FourOverSix and CJSO(8): time,
GB/s, the M=4 share and the MSE per matrix.

step_roofline: the algorithmic bytes of every kernel of a step (25 passes over W and the outputs)
over the timed step time, against the HBM peak and the measured copy rate.

roofline.anatomy: the CJSO round timed the same way at 4096 and 16384 rows; the difference gives the
round's marginal streaming rate and, extrapolated to zero rows, the fixed cost every launch pays.

hbm_attainable: a plain 1 GiB device copy timed on the box (read + write bytes / time): the streaming
rate a kernel can reach here, beside the 8 TB/s figure the roofline uses.

cpu_baseline: the oracle (plain C) on the host, one thread per core (at most 16), each on its own 256 rows
of the first matrix in all four modes; the one-thread rate beside it. speedup_vs_cpu is
value / cpu_baseline.value.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--streams S] [--no-c5]
                       [--only-4096] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of weights quantized (and % HBM / % VALU peak) per mode, 4096×4096 bf16"
PEAK_HBM = 8.0e12  # B/s, MI355X HBM3E
PEAK_FP32 = 157.3e12  # FLOP/s, MI355X FP32 vector (packed FMA = 4 FLOP per lane-cycle)
ROWS = COLS = 4096
N_MATS = 12
ITERS = 8
MODES = (("max", 0), ("4o6", 0), ("cjso", ITERS), ("soar", ITERS))
SEARCH_FLOPS_PER_BLOCK = 101 * 16 * 9
ROUND_BYTES_PER_ELEM = 2 + 1 / 16 + 1 / 16  # CJSO round (not the last): read W and scale, write scale
SEARCH_BYTES_PER_ELEM = 2 + 1 / 16 + 2 / 16 + 1 / 2 + 1 / 16  # read W, scale, bracket; write codes, scale
# algorithmic bytes per element of every kernel of a step (each reads the bf16 block once; outputs as
# written): codes 1/2, scale and M=4 map 1/16 each, the SOAR bracket 2/16
STEP_KERNEL_BYTES_PER_ELEM = {
    "max": [2, 2 + 1 / 2 + 1 / 16],  # k_amax; k_quant: codes and scale
    "4o6": [2, 2 + 1 / 2 + 1 / 16 + 1 / 16],  # k_amax; k_quant: codes, scale and the M=4 map
    # k_amax; k_cjso_init: new scale; ITERS-1 rounds; the last round: read scale, write scale and codes
    "cjso": [2, 2 + 1 / 16] + [ROUND_BYTES_PER_ELEM] * (ITERS - 1) + [2 + 1 / 16 + 1 / 16 + 1 / 2],
    # as CJSO, but the last round writes the bracket instead of the codes (the search writes them); then the
    # search
    "soar": [2, 2 + 1 / 16] + [ROUND_BYTES_PER_ELEM] * (ITERS - 1) + [2 + 1 / 16 + 1 / 16 + 2 / 16,
                                                                      SEARCH_BYTES_PER_ELEM],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_cjso_iter_4096x4096.txt")
COPY_BYTES = 256 << 20
KERNEL_NAMES = {
    "max": ["k_amax", "k_quant"],
    "4o6": ["k_amax", "k_quant"],
    "cjso": ["k_amax", "k_cjso_init"] + ["k_cjso_iter"] * ITERS,
    "soar": ["k_amax", "k_cjso_init"] + ["k_cjso_iter"] * ITERS + ["k_soar"],
}
assert {m: len(v) for m, v in STEP_KERNEL_BYTES_PER_ELEM.items()} == {m: len(v) for m, v in KERNEL_NAMES.items()}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# the sources the CJSO round kernel (and so its counter figures) is built from
ROUND_SOURCES = ("quant_kernels.hip", "block.hpp", "codec.hpp", "launch.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_block_scaled_elem_amd", "csrc")
    for name in ROUND_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(W0: np.ndarray) -> dict:
    """The oracle as it stands, on the host: first one thread on rows 0..255 of the first matrix in all
    four modes, then one thread per available core (at most 16), each on its own 256 rows of the same
    matrix, all four modes (the oracle's C calls release the GIL, so the threads run in parallel; each
    call is independent and the oracle has no mutable global state). `value` is the all-core rate."""
    import concurrent.futures

    import oracle

    oracle.lib()  # load once before any thread calls it
    sample = np.ascontiguousarray(W0[:256])
    t0 = time.perf_counter()
    for mode, iters in MODES:
        oracle.quantize(sample, mode, iters)
    dt1 = time.perf_counter() - t0
    one = len(MODES) * sample.nbytes / dt1

    threads = max(1, min(16, len(os.sched_getaffinity(0)), W0.shape[0] // 256))
    samples = [np.ascontiguousarray(W0[256 * i:256 * (i + 1)]) for i in range(threads)]

    def work(x):
        for mode, iters in MODES:
            oracle.quantize(x, mode, iters)

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(work, samples))
    dtn = time.perf_counter() - t0
    alln = len(MODES) * sum(x.nbytes for x in samples) / dtn
    gptq_leg = gptq_cpu_sample(W0)
    per_config = oracle_per_config(W0)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(alln / 1e9, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{threads} threads, each on its own 256 rows of the first 4096x4096 matrix "
                      f"({256 * 4096} elements), all four modes, {dtn:.1f} s",
            "single_thread": {"value": round(one / 1e9, 6), "unit": "GB/s",
                              "sample": f"rows 0-255, all four modes, {dt1:.1f} s"},
            "gptq": gptq_leg,
            "per_config": per_config,
            "host": {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}}


def oracle_per_config(W0: np.ndarray) -> dict:
    """The oracle, one thread, on a bounded row sample of every workload, extrapolated to the whole
    workload by its element count (labelled so): C1 in full (MAX and FourOverSix); C2 (the 4096 x 4096
    matrix; MAX and FourOverSix) from 64 rows; C3 (14336 x 4096 and 4096 x 14336; FourOverSix and CJSO(8))
    from 32 rows of each; C4 (the C2 matrix; SOAR(8)) from 32 rows; C5 (one 7B-shaped layer of 7
    matrices; FourOverSix and SOAR(8)) from 16 rows of each, times 32 layers."""
    import oracle
    import synth

    def timed(W, runs):
        t0 = time.perf_counter()
        for mode, iters in runs:
            oracle.quantize(np.ascontiguousarray(W), mode, iters)
        return time.perf_counter() - t0

    out = {}
    W1 = synth.c1(0)
    out["C1"] = {"seconds": round(timed(W1, [("max", 0), ("4o6", 0)]), 3), "sample": "whole matrix",
                 "modes": "max, 4o6"}
    dt = timed(W0[:64], [("max", 0), ("4o6", 0)])
    out["C2"] = {"seconds_extrapolated": round(dt * 4096 / 64, 2), "sample": "rows 0-63", "modes": "max, 4o6"}
    tot = 0.0
    for which in (0, 1):
        W = synth.c3(which, 0, rows=32)  # the first 32 rows of the matrix
        dt = timed(W, [("4o6", 0), ("cjso", ITERS)])
        tot += dt * (14336, 4096)[which] / 32
    out["C3"] = {"seconds_extrapolated": round(tot, 2), "sample": "rows 0-31 of each matrix",
                 "modes": f"4o6, cjso({ITERS})"}
    dt = timed(W0[:32], [("soar", ITERS)])
    out["C4"] = {"seconds_extrapolated": round(dt * 4096 / 32, 2), "sample": "rows 0-31", "modes": f"soar({ITERS})"}
    tot = 0.0
    for name in synth.C5_ORDER:
        W = synth.c5(0, name, rows=16)  # the first 16 rows of the matrix
        dt = timed(W, [("4o6", 0), ("soar", ITERS)])
        tot += dt * synth.C5_SHAPES[name][0] / 16
    out["C5"] = {"seconds_extrapolated": round(tot * 32, 1), "layer0_seconds_extrapolated": round(tot, 2),
                 "sample": "rows 0-15 of each matrix of layer 0, times 32 layers", "modes": f"4o6, soar({ITERS})"}
    out["threads"] = 1
    return out


def gptq_cpu_sample(W0: np.ndarray, rows: int = 32) -> dict:
    """The GPTQ oracle (binary64 numpy) on the same 4096 x 4096 problem, its column sweep limited to
    `rows` rows (the frame and H^-1 are computed in full); the whole matrix is extrapolated from the
    sweep's share per row, and labelled so."""
    import synth
    from oracle import gptq as og

    H = synth.hessian(W0.shape[1], 0, n=GPTQ_INPUTS)
    t0 = time.perf_counter()
    og.gptq(W0, H, 0.01, rows=np.arange(1))
    fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    og.gptq(W0, H, 0.01, rows=np.arange(rows))
    dt = time.perf_counter() - t0
    per_row = max(dt - fixed, 0.0) / (rows - 1)
    whole = fixed + per_row * W0.shape[0]
    return {"sample": f"oracle column sweep on rows 0-{rows - 1} (frame and H^-1 in full), {dt:.1f} s",
            "extrapolated_whole_matrix_s": round(whole, 2),
            "TFLOPs_extrapolated": round(gptq_flops(*W0.shape) / whole / 1e12, 5)}


PEAK_BF16_MFMA = 2.5e15  # FLOP/s, MI355X dense bf16 matrix peak
PEAK_FP64 = 78.6e12  # FLOP/s, MI355X FP64 vector (and FP64 matrix) peak
GPTQ_INPUTS = 8192  # synthetic calibration input vectors behind the second moment H


def gptq_flops(rows: int, cols: int) -> float:
    """Algorithmic FLOPs of one GPTQ call: the Cholesky factorisation (cols^3 / 3 multiply-adds) and the
    column sweep (each row's column j takes j multiply-adds for the errors before it: rows * cols^2 / 2)."""
    return 2.0 * (cols ** 3 / 3.0 + rows * cols ** 2 / 2.0)


def gptq_pass(torch, nv, dev, W):
    """GPTQ inside the FourOverSix frame (nvfp4_gptq) on the 4096 x 4096 weights, with the binary64
    second moment of GPTQ_INPUTS synthetic inputs; workspace preallocated; HIP-event average of
    repeated calls on the current stream."""
    import synth

    rows, cols = W.shape
    H = torch.from_numpy(synth.hessian(cols, 0, n=GPTQ_INPUTS)).to(dev)
    ws = torch.empty(nv.gptq_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    for _ in range(2):
        nv.gptq(W, H, 0.01, workspace=ws)
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        nv.gptq(W, H, 0.01, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = gptq_flops(rows, cols)
    log(f"gptq {rows}x{cols}: {ms:.2f} ms")
    return {"workload": f"{rows}x{cols} bf16 weights, H = second moment of {GPTQ_INPUTS} synthetic inputs "
                        f"(binary64), percdamp 0.01", "ms": round(ms, 4),
            "algorithmic_flops": flops, "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 3),
            "frac_fp64_peak": round(flops / (ms * 1e-3) / PEAK_FP64, 4),
            "workspace_bytes": int(ws.numel())}


def w4a16_pass(torch, nv, dev, W):
    """The consumer of the format: Y = X @ What.T with the 4096 x 4096 weights quantised (FourOverSix)
    and bf16 activations, one case per kernel shape: M = 1 (one token, the GEMV: bound by reading 0.5625 B
    per weight), M = 16 and 64 (the skinny MFMA kernel), M = 256 (128 x 64 MFMA tiles with K split),
    M = 1024 (128 x 128 tiles) and M = 4096 (256 x 128 tiles, bf16 MFMA-bound). Times are HIP-event
    averages on the current stream: over a graph of repeated calls for M <= 64 (calls of a few microseconds,
    where host enqueue would dominate), over repeated eager calls for the tiled kernels (tens of
    microseconds and more per call, so the device stays busy), with the K-split scratch preallocated."""
    codes, scales, alpha = nv.quantize(W, "4o6")
    n, k = W.shape
    # context: torch's dense bf16 product (hipBLASLt) on the dequantised weights, same shapes and timing
    WT = nv.dequantize(codes, scales, alpha, torch.bfloat16).t().contiguous()  # [k, n]
    out = {"weights": f"{n}x{k} NVFP4 (FourOverSix)", "cases": {},
           "dense_ref": "torch.matmul bf16 (hipBLASLt) with the dequantised weights, timed the same way"}

    def graph_ms(call, Y, reps):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        eager = Y.clone()
        g = torch.cuda.CUDAGraph()  # the calls back to back on the device, without host overhead between them
        with torch.cuda.graph(g):
            for _ in range(reps):
                call()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        # a replay must reproduce the eager result (library calls inside a graph are checked, not trusted)
        return e0.elapsed_time(e1) / reps if torch.equal(Y, eager) else None
    kernels = {1: "k_w4a16_gemv", 16: "k_w4a16_skinny", 64: "k_w4a16_skinny (4 tiles of X)",
               256: "k_w4a16_gemm 128x64 tiles + k_w4a16_reduce (K split)", 1024: "k_w4a16_gemm 128x128 tiles",
               4096: "k_w4a16_gemm 256x128 tiles"}
    def eager_ms(call, reps):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for m in (1, 16, 64, 256, 1024, 4096):
        X = (torch.randn((m, k), device=dev) * 0.5).to(torch.bfloat16)
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        need = nv.matmul_workspace_bytes(m, k, n)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        reps = 200 if m <= 64 else 20
        timer = graph_ms if m <= 64 else (lambda call, Y, reps: eager_ms(call, reps))
        ms = timer(lambda: nv.matmul(X, codes, scales, alpha, out=Y, workspace=ws), Y, reps)
        if ms is None:
            raise RuntimeError(f"W4A16 product, M={m}: a graph replay differs from the eager call")
        Yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        dense_ms = timer(lambda: torch.matmul(X, WT, out=Yd), Yd, reps)
        wbytes = n * k // 2 + n * k // 16
        moved = wbytes + m * k * 2 + m * n * 2
        flops = 2.0 * m * n * k
        out["cases"][f"M={m}"] = {
            "kernel": kernels[m], "ms": round(ms, 5), "GBps": round(moved / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(moved / (ms * 1e-3) / PEAK_HBM, 4),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(flops / (ms * 1e-3) / PEAK_BF16_MFMA, 4),
            "dense_ref_ms": None if dense_ms is None else round(dense_ms, 5),
            "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms, 2)}
        log(f"w4a16 M={m}: {ms * 1e3:.1f} us (dense bf16 {dense_ms if dense_ms is None else round(dense_ms * 1e3, 1)} us)")
    return out


C5_SHAPES = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
             "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
C5_LAYERS = 32


def c5_pass(torch, nv, dev, streams):
    """Whole-model workload: 32 layers x {q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008}
    bf16 (224 matrices, 12.95 GB), resident in HBM, quantised matrix by matrix in each mode (consecutive
    matrices alternate over the streams). Returns total time and aggregate GB/s per mode. The weights
    follow the same recipe as the parity inputs (Student-t, nu = 5, std 0.02) but are drawn on the GPU
    with torch's generator, so that the pass takes seconds."""
    log("c5: generating 224 matrices on the GPU")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    mats = []
    for layer in range(C5_LAYERS):
        for name, (r, c) in C5_SHAPES.items():
            z = torch.randn((r, c), generator=g, device=dev)
            chi = torch.zeros((r, c), device=dev)
            for _ in range(5):
                chi += torch.randn((r, c), generator=g, device=dev).square()
            t = z / torch.sqrt(chi / 5.0) * (0.02 / (5.0 / 3.0) ** 0.5)
            mats.append(t.to(torch.bfloat16))
            del z, chi, t
    torch.cuda.synchronize()
    total_bytes = sum(m.numel() * 2 for m in mats)
    n_streams = len(streams)
    bufs = []
    for k in range(n_streams):
        b = {}
        for mode, _ in MODES:
            b[mode] = dict(workspace=torch.empty(nv.workspace_bytes(11008, 4096, mode), dtype=torch.uint8, device=dev))
        b["codes"] = {shape: torch.empty((shape[0], shape[1] // 2), dtype=torch.uint8, device=dev)
                      for shape in set(C5_SHAPES.values())}
        b["scales"] = {shape: torch.empty((shape[0], shape[1] // 16), dtype=torch.uint8, device=dev)
                       for shape in set(C5_SHAPES.values())}
        b["alpha"] = torch.empty(1, dtype=torch.float32, device=dev)
        bufs.append(b)

    def run(mode, iters, which=None):
        for i, W in enumerate(mats):
            if which is not None and not which(W):
                continue
            k = i % n_streams
            b = bufs[k]
            shape = tuple(W.shape)
            with torch.cuda.stream(streams[k]):
                nv.quantize(W, mode, iters, codes=b["codes"][shape], scales=b["scales"][shape], alpha=b["alpha"],
                            workspace=b[mode]["workspace"])

    square = lambda W: tuple(W.shape) == (4096, 4096)  # noqa: E731
    sq_bytes = sum(m.numel() * 2 for m in mats if square(m))
    out = {"matrices": len(mats), "bytes": total_bytes, "streams": n_streams, "modes": {},
           "square_4096": {"matrices": sum(1 for m in mats if square(m)), "bytes": sq_bytes, "modes": {}}}
    for mode, iters in MODES:
        run(mode, iters)  # warm-up pass
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(mode, iters)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        out["modes"][mode] = {"total_ms": round(dt * 1e3, 3), "GBps": round(total_bytes / dt / 1e9, 2),
                              "frac_hbm_peak": round(total_bytes / dt / PEAK_HBM, 4)}
        t0 = time.perf_counter()
        run(mode, iters, square)
        torch.cuda.synchronize()
        dq = time.perf_counter() - t0
        out["square_4096"]["modes"][mode] = {"total_ms": round(dq * 1e3, 3), "GBps": round(sq_bytes / dq / 1e9, 2),
                                             "frac_hbm_peak": round(sq_bytes / dq / PEAK_HBM, 4)}
        log(f"c5 {mode}: {dt * 1e3:.1f} ms; square matrices {dq * 1e3:.1f} ms")
    del mats
    torch.cuda.empty_cache()
    return out


def quality_pass(torch, nv, W) -> dict:
    """Reconstruction error of each mode (and of the search variants) on one matrix, from the GPU error
    statistics: MSE = SSE / n, and its ratio to the max rule's."""
    n = W.numel()
    runs = [("max", {}), ("4o6", {}), ("cjso", {"iters": ITERS}), ("cjso", {"iters": ITERS, "init": "4o6"}),
            ("soar", {"iters": ITERS}), ("soar", {"iters": ITERS, "init": "4o6"}),
            ("soar", {"iters": ITERS, "grid": (100, 200, 201)}), ("soar", {"iters": ITERS, "dd_rule": "quant"}),
            ("soar", {"iters": ITERS, "dd_rule": "lsq"})]
    out = {}
    for mode, kw in runs:
        kw = dict(kw)
        iters = kw.pop("iters", 0)
        codes, scales, alpha = nv.quantize(W, mode, iters, **kw)
        sse, _ = nv.error_stats(W, codes, scales, alpha)
        name = mode + "".join(f" {k}={v}" for k, v in kw.items())
        # one more call of the same settings, timed alone (the variants scan the whole grid)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nv.quantize(W, mode, iters, codes=codes, scales=scales, alpha=alpha, **kw)
        e1.record()
        torch.cuda.synchronize()
        out[name] = {"mse": float(sse.item()) / n, "call_ms": round(e0.elapsed_time(e1), 4)}
    base = out["max"]["mse"]
    for v in out.values():
        v["vs_max"] = round(v["mse"] / base, 5)
    return out


def c3_pass(torch, nv, dev) -> dict:
    """The MLP-shaped matrices (14336 x 4096 up, 4096 x 14336 down; N(0, 0.015^2) with per-row std
    log-uniform in [0.5, 2]x, the parity inputs' host generator): FourOverSix then CJSO(8), per matrix
    the call time (HIP events, mean of 5 calls after a warm-up), GB/s, the M=4 share and the MSE."""
    import synth

    out = {}
    for which, name in ((0, "up_14336x4096"), (1, "down_4096x14336")):
        W0 = synth.c3(which, 0)
        W = torch.from_numpy(W0.view(np.int16)).view(torch.bfloat16).to(dev)
        rows, cols = W.shape
        res = {}
        for mode, iters in (("4o6", 0), ("cjso", ITERS)):
            mch = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev) if mode == "4o6" else None
            codes, scales, alpha = nv.quantize(W, mode, iters, mchoice=mch)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                nv.quantize(W, mode, iters, codes=codes, scales=scales, alpha=alpha, mchoice=mch)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            sse, _ = nv.error_stats(W, codes, scales, alpha)
            r = {"ms": round(ms, 4), "GBps": round(W.numel() * 2 / (ms * 1e-3) / 1e9, 1),
                 "mse": float(sse.item()) / W.numel()}
            if mch is not None:
                r["m4_fraction"] = round(float(mch.float().mean().item()), 4)
            res[mode] = r
        out[name] = res
        del W
    torch.cuda.empty_cache()
    return out


def round_anatomy(torch, nv, dev, nk_cjso) -> dict:
    """The CJSO round at two heights (4096 and 16384 rows, 4096 columns; six resident matrices each, drawn
    on the GPU with the whole-model recipe). Round time = span of rounds 1..ITERS-1 over their number
    (HIP events, median of 18 calls). The difference of the two gives the marginal streaming rate of the
    round (algorithmic bytes per extra row over time per extra row) and, extrapolated to zero rows, the
    fixed cost of one launch: the split between what the matrix size pays and what every launch pays."""
    log("round anatomy: 4096 and 16384 rows")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    t = {}
    for rows in (4096, 16384):
        mats = []
        for _ in range(6):
            z = torch.randn((rows, COLS), generator=g, device=dev)
            chi = torch.zeros((rows, COLS), device=dev)
            for _ in range(5):
                chi += torch.randn((rows, COLS), generator=g, device=dev).square()
            mats.append((z / torch.sqrt(chi / 5.0) * (0.02 / (5.0 / 3.0) ** 0.5)).to(torch.bfloat16))
            del z, chi
        o = dict(codes=torch.empty((rows, COLS // 2), dtype=torch.uint8, device=dev),
                 scales=torch.empty((rows, COLS // 16), dtype=torch.uint8, device=dev),
                 alpha=torch.empty(1, dtype=torch.float32, device=dev),
                 workspace=torch.empty(nv.workspace_bytes(rows, COLS, "cjso"), dtype=torch.uint8, device=dev))
        for i in range(6):
            nv.quantize(mats[i], "cjso", ITERS, **o)
        spans = []
        for s in range(18):
            ev = [None] * (nk_cjso + 1)
            ev[2] = torch.cuda.Event(enable_timing=True)
            ev[2 + ITERS - 1] = torch.cuda.Event(enable_timing=True)
            nv.quantize(mats[s % 6], "cjso", ITERS, stage_events=ev, **o)
            spans.append((ev[2], ev[2 + ITERS - 1]))
        torch.cuda.synchronize()
        t[rows] = float(np.median([a.elapsed_time(b) for a, b in spans])) / (ITERS - 1) * 1e-3
        del mats, o
        torch.cuda.empty_cache()
    extra_bytes = (16384 - 4096) * COLS * ROUND_BYTES_PER_ELEM
    marginal = extra_bytes / (t[16384] - t[4096])
    fixed = t[4096] - 4096 * COLS * ROUND_BYTES_PER_ELEM / marginal
    return {"round_ms_4096_rows": round(t[4096] * 1e3, 5), "round_ms_16384_rows": round(t[16384] * 1e3, 5),
            "marginal_GBps": round(marginal / 1e9, 1), "fixed_us_per_launch": round(fixed * 1e6, 2),
            "method": "two heights, 4096 columns, GPU-drawn Student-t(5) weights; rounds 1..7 span / 7"}


def cold_warm_pass(torch, nv, W, outs, reps=25) -> dict:
    """One call per mode on the first matrix, timed with HIP events around the call: "cold" after a
    read-only pass over 1 GiB has evicted the Infinity Cache and the L2s (outside the timed region; a
    read leaves no dirty lines behind whose write-back would land in the timed call), "warm" for the
    same call repeated at once. Median of `reps` of each."""
    dev = W.device
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev).view(-1, 4096)
    flush.amax(dim=1)  # the fill's dirty lines leave before the first timed call
    torch.cuda.synchronize()
    res = {}
    for mode, iters in MODES:
        o = outs[mode]
        call = lambda: nv.quantize(W, mode, iters, codes=o["codes"], scales=o["scales"],  # noqa: E731
                                   alpha=o["alpha"], mchoice=o["mchoice"], workspace=o["workspace"])
        cold, warm = [], []
        for r in range(reps):
            flush.amax(dim=1)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            call()
            ev[1].record()
            ev[2].record()
            call()
            ev[3].record()
            torch.cuda.synchronize()
            cold.append(ev[0].elapsed_time(ev[1]))
            warm.append(ev[2].elapsed_time(ev[3]))
        c, w = float(np.median(cold)), float(np.median(warm))
        res[mode] = {"cold_ms": round(c, 5), "warm_ms": round(w, 5),
                     "cold_GBps": round(W.numel() * 2 / (c * 1e-3) / 1e9, 1),
                     "warm_GBps": round(W.numel() * 2 / (w * 1e-3) / 1e9, 1),
                     "cold_frac_hbm_peak": round(W.numel() * 2 / (c * 1e-3) / PEAK_HBM, 4),
                     "warm_frac_hbm_peak": round(W.numel() * 2 / (w * 1e-3) / PEAK_HBM, 4)}
    res["method"] = (f"HIP events around one call, median of {reps}; cold = after a read-only pass over 1 GiB, "
                     "warm = the same call repeated at once")
    del flush
    torch.cuda.empty_cache()
    return res


def graph_mode_pass(torch, nv, mats, outs, reps=24) -> dict:
    """Per-mode device time without host overhead: `reps` calls of one mode, on the resident matrices in
    turn (each visited twice, so most calls find their matrix in no cache), captured in one HIP graph;
    HIP events around a replay. A replay must reproduce the eager outputs of its last call."""
    res = {}
    for mode, iters in MODES:
        o = outs[mode]

        def call(W):
            nv.quantize(W, mode, iters, codes=o["codes"], scales=o["scales"], alpha=o["alpha"],
                        mchoice=o["mchoice"], workspace=o["workspace"])
        last = mats[(reps - 1) % len(mats)]
        call(last)
        torch.cuda.synchronize()
        want = (o["codes"].clone(), o["scales"].clone(), o["alpha"].clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                call(mats[r % len(mats)])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        if not (torch.equal(o["codes"], want[0]) and torch.equal(o["scales"], want[1]) and
                torch.equal(o["alpha"], want[2])):
            raise RuntimeError(f"{mode}: a graph replay differs from the eager call")
        ms = e0.elapsed_time(e1) / reps
        gbps = ROWS * COLS * 2 / (ms * 1e-3) / 1e9
        res[mode] = {"ms": round(ms, 5), "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps * 1e9 / PEAK_HBM, 4)}
        del g
    res["method"] = (f"{reps} calls per mode on the {len(mats)} resident matrices in turn, one HIP graph, "
                     "events around a replay")
    return res


def fp32_pass(torch, nv, W) -> dict:
    """The first matrix widened to fp32 (64 MiB; the same values), one warm call per mode timed with HIP
    events (median of 5): the binary32 input path. Its search has no exactness window (every block scans
    all 202 candidates), and its block sums run in binary64."""
    Wf = W.float().contiguous()
    res = {}
    for mode, iters in MODES:
        nv.quantize(Wf, mode, iters)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            nv.quantize(Wf, mode, iters)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        res[mode] = {"ms": round(ms, 5), "GBps": round(Wf.numel() * 4 / (ms * 1e-3) / 1e9, 1)}
    del Wf
    return res


def hbm_attainable(torch, dev) -> dict:
    """What a plain streaming kernel reaches on this machine: a 1 GiB device copy (torch's copy kernel;
    read + write bytes per second) and a read-only pass over 1 GiB (torch's max reduction over rows of
    4096 values, which keeps every CU streaming; bytes read per second). Median of 10 each."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    rows = src.view(-1, 4096)

    def med(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    t_copy = med(lambda: dst.copy_(src))
    t_read = med(lambda: rows.amax(dim=1))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * n * 4 / t_copy / 1e9, 1), "frac_of_peak": round(2 * n * 4 / t_copy / PEAK_HBM, 4),
            "read_GBps": round(n * 4 / t_read / 1e9, 1), "read_frac_of_peak": round(n * 4 / t_read / PEAK_HBM, 4),
            "kind": "1 GiB device copy (read + write bytes) and 1 GiB read-only row-max reduction, median of 10"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=3, help="HIP streams that consecutive steps rotate over")
    ap.add_argument("--no-c5", action="store_true", help="skip the whole-model (224 matrices) pass")
    ap.add_argument("--only-4096", action="store_true",
                    help="skip the passes on other shapes (MLP matrices, round anatomy), so that a profiler "
                         "averaging per kernel sees only 4096x4096 launches")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the quantizer runs on a single device and --gpus {args.gpus} is not "
              "supported (shard by matrix across processes instead)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}))
        return

    import nvfp4_block_scaled_elem_amd as nv
    import synth

    dev = torch.device("cuda:0")
    log("generating inputs")
    W0 = synth.c2(0)
    base = torch.from_numpy(W0.view(np.int16)).view(torch.bfloat16).to(dev)
    # the other matrices: row rotations of the first with alternating sign (same distribution, new bytes)
    mats = [base] + [(-1 if i % 2 else 1) * torch.roll(base, shifts=331 * i, dims=0) for i in range(1, N_MATS)]
    mats = [m.contiguous() for m in mats]
    n_streams = max(1, args.streams)
    streams = [torch.cuda.Stream(device=dev) for _ in range(n_streams)]
    outs = []
    for _ in range(n_streams):
        out = {}
        for mode, _ in MODES:
            out[mode] = dict(
                codes=torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=dev),
                scales=torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device=dev),
                alpha=torch.empty(1, dtype=torch.float32, device=dev),
                workspace=torch.empty(nv.workspace_bytes(ROWS, COLS, mode), dtype=torch.uint8, device=dev),
                mchoice=torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device=dev) if mode == "4o6" else None,
            )
        outs.append(out)
    out = outs[0]
    nk = {mode: nv.kernel_count(mode, iters) for mode, iters in MODES}

    def step(s, events=None, n=n_streams, modes=MODES, own_streams=True):
        # own_streams=False keeps the caller's current stream (graph capture, the instrumented pass)
        W = mats[s % N_MATS]
        k = s % n
        with torch.cuda.stream(streams[k]) if own_streams else contextlib.nullcontext():
            for mode, iters in modes:
                o = outs[k][mode]
                nv.quantize(W, mode, iters, codes=o["codes"], scales=o["scales"], alpha=o["alpha"],
                            mchoice=o["mchoice"], workspace=o["workspace"],
                            stage_events=events[mode] if events else None)

    def timed(n, modes=MODES):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(args.warmup + s, n=n, modes=modes)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    log("warmup")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # timed region: K steps, consecutive steps alternating over the streams
    log(f"timing {args.steps} steps on {n_streams} stream(s)")
    ms_per_step = timed(n_streams)
    single_ms_per_step = timed(1) if n_streams > 1 else ms_per_step
    # each mode alone on one stream, no events: the per-mode call time
    mode_ms = {mode: timed(1, ((mode, iters),)) for mode, iters in MODES}

    # per-kernel durations: the same steps again with HIP events recorded by the library around each of
    # its kernels on the stream they run on
    n_ev = max(20, min(args.steps, 100))
    evs = [{mode: [torch.cuda.Event(enable_timing=True) for _ in range(nk[mode] + 1)] for mode, _ in MODES}
           for _ in range(n_ev)]
    log(f"instrumented pass, {n_ev} steps")
    for s in range(n_ev):
        step(args.warmup + s, evs[s], n=1, own_streams=False)
    torch.cuda.synchronize()
    # CJSO calls with only two events, before round 1 and after round ITERS-1: the average round as the
    # rounds run back to back (per-kernel events add a gap in front of every kernel)
    o = outs[0]["cjso"]
    span_ev = []
    for s in range(n_ev):
        ev = [None] * (nk["cjso"] + 1)
        ev[2] = torch.cuda.Event(enable_timing=True)
        ev[2 + ITERS - 1] = torch.cuda.Event(enable_timing=True)
        nv.quantize(mats[(args.warmup + s) % N_MATS], "cjso", ITERS, codes=o["codes"], scales=o["scales"],
                    alpha=o["alpha"], workspace=o["workspace"], stage_events=ev)
        span_ev.append((ev[2], ev[2 + ITERS - 1]))
    torch.cuda.synchronize()
    # the SOAR call again with the 202-candidate search (same outputs), for its kernel time
    o = outs[0]["soar"]
    full_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk["soar"] + 1)] for _ in range(n_ev)]
    for s in range(n_ev):
        nv.quantize(mats[(args.warmup + s) % N_MATS], "soar", ITERS, codes=o["codes"], scales=o["scales"],
                    alpha=o["alpha"], workspace=o["workspace"], stage_events=full_ev[s], full_search=True)
    torch.cuda.synchronize()

    # the same step replayed from HIP graphs (one per resident matrix), for the launch overhead
    graphs = []
    for m in range(N_MATS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(m, n=1, own_streams=False)
        graphs.append(g)
    torch.cuda.synchronize()
    tg0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s % N_MATS].replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - tg0) * 1e3 / args.steps

    # per-mode call times and per-kernel durations from the stage events (GPU clock)
    per_mode = {}
    kern = {}
    for mode, iters in MODES:
        calls = [e[mode][0].elapsed_time(e[mode][-1]) for e in evs]
        dur = np.array([[e[mode][j].elapsed_time(e[mode][j + 1]) for j in range(nk[mode])] for e in evs])
        call_ms = mode_ms[mode]
        gbps = ROWS * COLS * 2 / (call_ms * 1e-3) / 1e9
        per_mode[mode] = {"ms": round(call_ms, 5), "GBps": round(gbps, 2), "frac_hbm_peak": round(gbps * 1e9 / PEAK_HBM, 4),
                          "ms_with_events": round(float(np.mean(calls)), 5), "kernels_ms": {}}
        for j, name in enumerate(KERNEL_NAMES[mode]):
            key = name if name != "k_cjso_iter" else "k_cjso_iter(avg)"
            per_mode[mode]["kernels_ms"].setdefault(key, []).append(float(dur[:, j].mean()))
        per_mode[mode]["kernels_ms"] = {k: round(float(np.mean(v)), 5) for k, v in per_mode[mode]["kernels_ms"].items()}
        kern[mode] = dur
    nblk = ROWS * COLS // 16
    nel = ROWS * COLS
    # CJSO rounds other than the last: the span of rounds 1 .. ITERS-1 over their number
    t_round = float(np.mean([a.elapsed_time(b) for a, b in span_ev])) / (ITERS - 1) * 1e-3
    rounds = np.concatenate([kern[m][:, 2:2 + ITERS - 1].reshape(-1) for m in ("cjso", "soar")])
    per_mode["cjso"]["round_ms_per_kernel_events"] = round(float(rounds.mean()), 5)
    round_gbps = nel * ROUND_BYTES_PER_ELEM / t_round / 1e9
    per_mode["cjso"]["round_ms"] = round(t_round * 1e3, 5)
    per_mode["cjso"]["round_algo_GBps"] = round(round_gbps, 2)
    per_mode["cjso"]["round_frac_hbm_peak"] = round(round_gbps * 1e9 / PEAK_HBM, 4)
    t_search = float(kern["soar"][:, -1].mean()) * 1e-3
    search_gbps = nel * SEARCH_BYTES_PER_ELEM / t_search / 1e9
    t_full = float(np.mean([e[-2].elapsed_time(e[-1]) for e in full_ev])) * 1e-3
    full_tflops = nblk * SEARCH_FLOPS_PER_BLOCK / t_full / 1e12
    per_mode["soar"].update({
        "search_ms": round(t_search * 1e3, 5), "search_algo_GBps": round(search_gbps, 2),
        "search_frac_hbm_peak": round(search_gbps * 1e9 / PEAK_HBM, 4),
        "full_search_ms": round(t_full * 1e3, 5), "full_search_TFLOPs": round(full_tflops, 3),
        "full_search_frac_fp32_peak": round(full_tflops * 1e12 / PEAK_FP32, 4),
    })
    m4 = int(out["4o6"]["mchoice"].sum().item())
    per_mode["4o6"]["m4_fraction"] = round(m4 / nblk, 4)
    # HBM view of the memory-bound single passes: algorithmic bytes of the whole call (read W once,
    # write codes and scales) over the call time
    algo_bytes = nel * (2 + 0.5 + 1.0 / 16)
    for mode in ("max", "4o6"):
        per_mode[mode]["algo_GBps"] = round(algo_bytes / (per_mode[mode]["ms"] * 1e-3) / 1e9, 2)

    # HBM bytes per launch of the CJSO round from the committed rocprofv3 counter summary, used only
    # while the kernel sources are the ones it was taken with
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_hash") == source_hash():
            traffic = int(float(fields["bytes_per_launch"]))
    roofline = {"bound": "hbm", "kernel": "k_cjso_iter (CJSO round other than the last)",
                "achieved": round(round_gbps, 2), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(round_gbps * 1e9 / PEAK_HBM, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(nel * ROUND_BYTES_PER_ELEM),
                "avg_launch_ms": round(t_round * 1e3, 5), "launches_per_step": 2 * (ITERS - 1)}

    cold_warm = cold_warm_pass(torch, nv, mats[0], outs[0])
    graph_modes = graph_mode_pass(torch, nv, mats, outs[0])
    for mode, _ in MODES:
        per_mode[mode]["graph_ms"] = graph_modes[mode]["ms"]
        per_mode[mode]["graph_GBps"] = graph_modes[mode]["GBps"]
        per_mode[mode]["graph_frac_hbm_peak"] = graph_modes[mode]["frac_hbm_peak"]
    fp32 = fp32_pass(torch, nv, mats[0])
    w4a16 = w4a16_pass(torch, nv, dev, mats[0])
    gptq = gptq_pass(torch, nv, dev, mats[0])
    quality = quality_pass(torch, nv, mats[0])
    c3 = None if args.only_4096 else c3_pass(torch, nv, dev)
    anatomy = None if args.only_4096 else round_anatomy(torch, nv, dev, nk["cjso"])
    attainable = hbm_attainable(torch, dev)
    # the same rate against what a plain copy reaches on this machine (context for the fraction of peak)
    roofline["frac_of_attainable"] = round(round_gbps / attainable["copy_GBps"], 4)
    roofline["frac_of_read_attainable"] = round(round_gbps / attainable["read_GBps"], 4)
    if anatomy is not None:
        anatomy["marginal_frac_of_attainable"] = round(anatomy["marginal_GBps"] / attainable["copy_GBps"], 4)
        roofline["anatomy"] = anatomy
    # the step as a whole: every kernel's algorithmic bytes over the timed step (streams overlapping)
    step_bytes = nel * sum(sum(v) for v in STEP_KERNEL_BYTES_PER_ELEM.values())
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    step_roofline = {"algorithmic_bytes_per_step": int(step_bytes), "passes_over_W": sum(
        len(v) for v in STEP_KERNEL_BYTES_PER_ELEM.values()), "GBps": round(step_gbps, 1),
        "frac_of_peak": round(step_gbps * 1e9 / PEAK_HBM, 4),
        "frac_of_attainable": round(step_gbps / attainable["copy_GBps"], 4)}
    c5 = None if args.no_c5 else c5_pass(torch, nv, dev, streams)

    value = len(MODES) * ROWS * COLS * 2 / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "4096x4096 bf16 attention-projection weights, Student-t(nu=4) std 0.02 with 0.1% "
                               "outlier columns x20; 12 resident matrices visited in turn; step = MAX, FourOverSix, "
                               "CJSO(8), SOAR(8) of one matrix; consecutive steps on alternating streams", "rows": ROWS, "cols": COLS, "input_dtype": "bf16",
                   "matrices": N_MATS, "cjso_iters": ITERS, "parallelism": "single GPU",
                   "input_sha256": hashlib.sha256(W0.tobytes()).hexdigest()},
        "modes": per_mode,
        "streams": n_streams,
        "single_stream_ms_per_step": round(single_ms_per_step, 5),
        "graph_replay_ms_per_step": round(graph_ms_per_step, 5),
        "roofline": roofline,
        "step_roofline": step_roofline,
    }
    line["cold_warm"] = cold_warm
    line["graph_modes"] = graph_modes
    line["fp32_input"] = fp32
    line["w4a16"] = w4a16
    line["gptq"] = gptq
    line["quality"] = quality
    if c3 is not None:
        line["c3_mlp"] = c3
    line["hbm_attainable"] = attainable
    if c5 is not None:
        line["c5_whole_model"] = c5
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(W0)
        line["speedup_vs_cpu"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
