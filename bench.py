#!/usr/bin/env python3
"""Benchmark of the packed-ternary x q8_K hot path on one MI355X.

One step = one pass of the decode hot path over one token: q8_K quantization
of a fresh fp32 activation vector and the 32768 x 8192 pq2_0 matrix-vector
product, in one launch (`tq_gemv_f32`: every workgroup quantizes the slice
of x it needs on chip).  The weights are resident in HBM; eight repacked
copies (570 MB) are rotated so that the 256 MB Infinity Cache cannot serve a
repeat call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials N]

Prints ONE JSON line.  Timing: W eager warm-up steps, then K steps captured
in one HIP graph; the graph is replayed once untimed and then N times (N >= 5),
each replay bracketed by stream synchronizations and timed with HIP events on
the stream the kernels run on.  `value` is Gweights/s from the median replay;
`ms_per_step` is that replay's time / K.  The decode step is one kernel, so
the roofline's `kernel_us` is the same per-launch figure: the kernel's
algorithmic HBM bytes divided by it give `achieved`.  `ceiling` holds the
read ceiling of this part measured in the same run (libtq_probe.so): one
streaming read of the same eight rotated 71 MB buffers, and of 1 GiB, plus the
shader clock.  `extra` carries the prompt-product (17408 x 5120, 4 and 64
tokens), 64-layer step, ptq1_0 and small-workload figures, each the median of
N graph replays; `cpu_baseline` times the CPU oracle on the host.

Other modes (no JSON line):
    python bench.py --probe all|decode|prefill|ptq1|step64|...
        the workload of the rocprofv3 counter runs: every timed kernel of the
        benchmark launched 20 times, plus three 1 GiB device copies whose known
        size calibrates the byte counters;
    python bench.py --summarize DIR [--kernel-trace DIR2]
        reads rocprofv3 CSV output (counter collection and/or kernel trace)
        and prints the per-kernel summary committed under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tq_inputs as TI  # noqa: E402

METRIC = "Gweights/s + % peak HBM GB/s, ternary GEMV 32768×8192; GMAC/s prefill 64 tok"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published (TOPS = 2 x MAC/s)
MALL_BYTES = 256 << 20
NUM_CU = 256
PEAK_SCLK_GHZ = 2.4  # MI355X peak shader clock
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "bit_quantized_matvec_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--trials", type=int, default=7, help="timed graph replays per figure (median reported; >= 5)")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed replays of each graph before its timed replays (clocks settle)")
    ap.add_argument("--no-extra", action="store_true", help="skip the prompt-product, ptq1_0 and step figures")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall budget of the CPU baseline")
    ap.add_argument("--probe", default=None,
                    help="run only the named workloads' kernels 20 times each (counter runs): all, decode, prefill, "
                         "ptq1, step64, tiny, quant, ceiling (comma-separated)")
    ap.add_argument("--summarize", default=None, help="summarize rocprofv3 counter CSVs under this directory")
    ap.add_argument("--kernel-trace", default=None, help="with --summarize: a rocprofv3 kernel-trace CSV directory")
    ap.add_argument("--write-counters", action="store_true",
                    help="with --summarize: also record the per-kernel figures in profiles/counters.json")
    return ap.parse_args()


# ----------------------------------------------------------------- timing
# Untimed replays before the timed ones, for at least this many seconds of
# wall time (--settle).  Measured on MI355X: the first few tens of
# milliseconds of work after the GPU was idle run about 3% slower (the same
# 32768 x 8192 ptq1_0 product: 15.44 us per launch when timed first in a
# process, 15.01 us when timed again in it), and a 20-step graph replays in
# 0.3 ms, so a short timed region would otherwise sit entirely in that phase.
SETTLE_S = 0.3


def graph_trials(torch, step, K, trials):
    """Capture K calls of step(i) in one graph; replay it untimed once and
    then for at least SETTLE_S seconds; then `trials` times, each replay
    between two stream synchronizations and timed with HIP events recorded on
    the replay stream.  Returns per-replay seconds (device time), the host
    wall time of each replay and the number of untimed settle replays."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)  # one eager call on the capture stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    settle = 0
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        g.replay()
        settle += 1
        if settle % 8 == 0:
            torch.cuda.synchronize()  # keep the queue of replays short
    torch.cuda.synchronize()
    dev_s, wall_s = [], []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(max(5, trials)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall_s.append(time.perf_counter() - t0)
        dev_s.append(e0.elapsed_time(e1) * 1e-3)
    del g
    return {"median_s": statistics.median(dev_s), "min_s": min(dev_s), "max_s": max(dev_s),
            "wall_median_s": statistics.median(wall_s), "trials": len(dev_s), "settle_replays": settle}


def per_call_us(t, K):
    """Median / min / max microseconds per call of a graph_trials result."""
    return {"us": t["median_s"] * 1e6 / K, "us_min": t["min_s"] * 1e6 / K, "us_max": t["max_s"] * 1e6 / K}


def rounded(d, nd=4):
    return {k: (round(v, nd) if isinstance(v, float) else v) for k, v in d.items()}


def copies_for(nbytes: int) -> int:
    """Enough distinct weight copies that the rotation exceeds twice the MALL."""
    return max(2, -(-2 * MALL_BYTES // nbytes))


def resident_copies(torch, tq, name):
    """Repacked weight copies of a named workload (rotated so that no repeat
    call is served by the Infinity Cache), and its activations."""
    fmt, Wc, x = TI.make(name)
    R, G, _ = Wc.shape
    C = G * 128
    wdev = torch.from_numpy(Wc.reshape(-1)).cuda()
    ncopy = copies_for(tq.repacked_bytes(fmt, R, C))
    Ws = [tq.repack(wdev, fmt, R, C) for _ in range(ncopy)]
    del wdev
    return fmt, R, C, Ws, x


# ----------------------------------------------------------------- workloads
def decode_bench(torch, tq, K, W, trials):
    fmt, R, C, Ws, _x = resident_copies(torch, tq, "decode_32768x8192")
    ncopy = len(Ws)
    # a fresh activation vector per step: rotate over a pool of distinct vectors
    xs = torch.from_numpy(TI.activations(TI.rng(TI.DECODE, 0, 0, 1), 64, C)).cuda()
    q = torch.empty((1, C), dtype=torch.int8, device="cuda")
    d = torch.empty((1, C // 256), dtype=torch.float32, device="cuda")
    bs = torch.empty((1, C // 16), dtype=torch.int16, device="cuda")
    y = torch.empty(R, dtype=torch.float32, device="cuda")

    def step(i):
        # one launch: every workgroup quantizes x itself, on chip
        tq.gemv_f32(fmt, Ws[i % ncopy], R, C, xs[i % 64], out=y)

    def step_two(i):
        tq.quantize_q8k(xs[i % 64: i % 64 + 1], out=(q, d, bs))
        tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y)

    for i in range(W):
        step(i)
        step_two(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    main = graph_trials(torch, step, K, trials)
    two = graph_trials(torch, step_two, K, trials)
    gemv = graph_trials(torch, lambda i: tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y), K, trials)
    quant = graph_trials(torch, lambda i: tq.quantize_q8k(xs[i % 64: i % 64 + 1], out=(q, d, bs)), K, trials)
    wbytes = tq.repacked_bytes(fmt, R, C)
    return {
        "R": R, "C": C, "Ws": Ws, "copies": ncopy, "main": main, "two": two, "gemv": gemv, "quant": quant,
        "eager_s": eager_s,
        # algorithmic bytes per launch: weights + fp32 x + fp32 y (fused); weights + q + d + y (stored-q8 product)
        "algo_bytes": wbytes + 4 * C + 4 * R, "algo_bytes_gemv": wbytes + C + 4 * (C // 256) + 4 * R,
        "weight_bytes": wbytes,
    }


def prefill_bench(torch, tq, T, K, trials, fmt_name="pq2_0"):
    prefix = "prefill" if fmt_name == "pq2_0" else "ptq1_prefill"
    fmt, R, C, Ws, x = resident_copies(torch, tq, f"{prefix}_17408x5120_t{T}")
    ncopy = len(Ws)
    q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
    y = torch.empty((T, R), dtype=torch.float32, device="cuda")
    call = lambda i: tq.gemm(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y)
    for i in range(20):
        call(i)
    torch.cuda.synchronize()
    r = per_call_us(graph_trials(torch, call, K, trials), K)
    us = r["us"]
    macs = R * C * T
    r.update({"tokens": T, "gmac_s": macs / us / 1e3,
              # int8 matrix-core share of the wall time (2 ops per MAC); the
              # counter-based figures are under "counters"
              "mfma_frac_wall": 2 * macs / (us * 1e-6) / (INT8_MFMA_PEAK_TOPS * 1e12)})
    bsum_bytes = 2 * T * (C // 16) if fmt == "ptq1_0" else 0
    algo = tq.repacked_bytes(fmt, R, C) + T * C + bsum_bytes + 4 * T * (C // 256) + 4 * T * R
    r["algo_bytes"] = algo
    r["hbm_gbs"] = algo / us / 1e3
    r["hbm_frac"] = r["hbm_gbs"] / HBM_PEAK_GBS
    return r


def ptq1_bench(torch, tq, K, trials):
    fmt, R, C, Ws, x = resident_copies(torch, tq, "ptq1_32768x8192")
    ncopy = len(Ws)
    q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
    y = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, R, C, 1)
    call = lambda i: tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y, ws=ws)
    for i in range(20):
        call(i)
    torch.cuda.synchronize()
    r = per_call_us(graph_trials(torch, call, K, trials), K)
    wb = tq.repacked_bytes(fmt, R, C)
    r.update({"gweights_s": R * C / r["us"] / 1e3, "weight_gbs": wb / r["us"] / 1e3,
              "hbm_frac": wb / r["us"] / 1e3 / HBM_PEAK_GBS})
    return r


def synth_pq2_gpu(torch, gen, rows, cols):
    """Canonical pq2_0 blocks drawn on the device from a seeded generator
    (timing does not depend on the values): each code byte is one of the 81
    bytes whose four 2-bit fields are all valid, each scale uniform in
    [0.01, 0.05] rounded to fp16, blocks laid out as fp16 d then 32 code bytes."""
    G = cols // 128
    table = torch.from_numpy(TI.VALID_PQ2_BYTES.astype(np.uint8)).cuda()
    idx = torch.randint(0, table.numel(), (rows, G, 32), device="cuda", generator=gen)
    codes = table[idx]
    del idx
    d = (torch.rand((rows, G), device="cuda", generator=gen) * 0.04 + 0.01).half()
    return torch.cat([d.view(torch.uint8).view(rows, G, 2), codes], dim=2).reshape(-1)


class Step64:
    """The 64-layer decode step for one token: for each layer the gate, up,
    down, qkv and out matrices (distinct weights, 5.7 GB in all), each with a
    fresh q8_K quantization of its own N(0,1) activation vector.  Gate and up
    share one launch (tq_gemv_f32_batch); the others are tq_gemv_f32."""

    def __init__(self, torch, tq):
        self.torch, self.tq = torch, tq
        fmt = self.fmt = "pq2_0"
        gen = torch.Generator(device="cuda")
        gen.manual_seed(TI.SEED_BASE + TI.STEP64)
        self.mats = []
        for _layer in range(64):
            for _name, R, C in TI.STEP64_SHAPES:
                canon = synth_pq2_gpu(torch, gen, R, C)
                self.mats.append((R, C, tq.repack(canon, fmt, R, C, check_codes=False)))
                del canon
        self.names = [name for _layer in range(64) for name, _R, _C in TI.STEP64_SHAPES]
        kmax = max(C for _, C, _ in self.mats)
        rmax = max(R for R, _, _ in self.mats)
        self.xs = torch.randn((len(self.mats), kmax), device="cuda", generator=gen)
        self.q = torch.empty(kmax, dtype=torch.int8, device="cuda")
        self.d = torch.empty(kmax // 256, dtype=torch.float32, device="cuda")
        self.bs = torch.empty(kmax // 16, dtype=torch.int16, device="cuda")
        self.y = torch.empty(rmax, dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(max(tq.workspace_bytes(fmt, R, C) for R, C, _ in self.mats), dtype=torch.uint8,
                              device="cuda")
        self.ys = [torch.empty(R, dtype=torch.float32, device="cuda") for R, _C, _W in self.mats[:2]]
        pair_rows = sum(-(-R // 64) * 64 for R, _C, _W in self.mats[:2])
        self.ws_pair = torch.zeros(max(16, tq.workspace_bytes(fmt, pair_rows, self.mats[0][1])), dtype=torch.uint8,
                                   device="cuda")

    def step(self, _i=0):
        tq, fmt, mats, names = self.tq, self.fmt, self.mats, self.names
        m = 0
        while m < len(mats):
            R, C, Wd = mats[m]
            if names[m] == "gate" and names[m + 1] == "up":
                # gate and up read the same layer input in a real model: one launch
                R2, _C2, Wd2 = mats[m + 1]
                tq.gemv_f32_batch(fmt, [Wd, Wd2], [R, R2], C, [self.xs[m, :C], self.xs[m + 1, :C]], outs=self.ys,
                                  ws=self.ws_pair)
                m += 2
                continue
            tq.gemv_f32(fmt, Wd, R, C, self.xs[m, :C], out=self.y[:R], ws=self.ws)
            m += 1

    def step_two(self, _i=0):
        tq, fmt = self.tq, self.fmt
        for m, (R, C, Wd) in enumerate(self.mats):
            tq.quantize_q8k(self.xs[m, :C].view(1, C), out=(self.q[:C].view(1, C), self.d[: C // 256].view(1, -1),
                                                             self.bs[: C // 16].view(1, -1)))
            tq.gemv(fmt, Wd, R, C, self.q[:C], self.d[: C // 256], self.bs[: C // 16], out=self.y[:R], ws=self.ws)


def step64_bench(torch, tq, reps, trials):
    s = Step64(torch, tq)
    s.step_two()
    s.step()
    torch.cuda.synchronize()
    t = graph_trials(torch, s.step, reps, trials)
    t2 = graph_trials(torch, s.step_two, reps, trials)
    weights = sum(R * C for R, C, _ in s.mats)
    wbytes = sum(tq.repacked_bytes(s.fmt, R, C) for R, C, _ in s.mats)
    ms = t["median_s"] * 1e3 / reps
    return {"matrices": len(s.mats), "step": "tq_gemv_f32_batch for gate + up, tq_gemv_f32 for down, qkv, out",
            "ms_per_token": ms, "ms_min": t["min_s"] * 1e3 / reps, "ms_max": t["max_s"] * 1e3 / reps,
            "gweights_s": weights / (ms * 1e-3) / 1e9,
            "weight_gbs": wbytes / (ms * 1e-3) / 1e9, "hbm_frac": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "weight_bytes": wbytes, "two_kernel_ms_per_token": t2["median_s"] * 1e3 / reps}


def tiny_bench(torch, tq, K, trials):
    """The 256x1024 workload: one fused call per step, replayed from a graph
    (launch-bound: its 70 KB of weights stay in the caches)."""
    fmt, Wc, x = TI.make("tiny_256x1024")
    R, G, _ = Wc.shape
    C = G * 128
    W = tq.repack(torch.from_numpy(Wc.reshape(-1)).cuda(), fmt, R, C)
    xd = torch.from_numpy(x[0].copy()).cuda()
    y = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, R, C, 1)
    r = per_call_us(graph_trials(torch, lambda i: tq.gemv_f32(fmt, W, R, C, xd, out=y, ws=ws), K, trials), K)
    r.update({"rows": R, "cols": C, "gweights_s": R * C / r["us"] / 1e3})
    return r


def quantize_bench(torch, tq, K, trials):
    C = 8192
    xs = torch.from_numpy(TI.activations(TI.rng(TI.DECODE, 0, 0, 2), 1, C)).cuda()
    out = (torch.empty((1, C), dtype=torch.int8, device="cuda"), torch.empty((1, 32), dtype=torch.float32, device="cuda"),
           torch.empty((1, 512), dtype=torch.int16, device="cuda"))
    r = per_call_us(graph_trials(torch, lambda i: tq.quantize_q8k(xs, out=out), K, trials), K)
    r["cols"] = C
    return r


# ----------------------------------------------------------------- ceiling probe
def probe_lib():
    import ctypes

    import bit_quantized_matvec_amd as tq  # noqa: F401  (loads torch's HIP runtime first)

    path = os.path.join(ROOT, "bit_quantized_matvec_amd", "libtq_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python bit_quantized_matvec_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.tqp_read.argtypes = [P, I64, I, I, I, P, P]
    lib.tqp_read.restype = I
    lib.tqp_clock.argtypes = [P, I, I, P, I64, P]
    lib.tqp_clock.restype = I
    lib.tqp_read_units.argtypes = [P, I, I, P, P]
    lib.tqp_read_units.restype = I
    return lib


READ_BLOCKS, READ_THREADS = 8192, 512  # the fastest shape of a sweep of the read kernel
DECODE_TILES, DECODE_UNITS = 512, 32  # 32768 x 8192: row tiles of 64, units of 256 columns


def ceiling_bench(torch, bufs, K, trials):
    """Streaming reads with libtq_probe's read kernel: one pass over each of the
    rotated 71 MB weight copies (the decode step's own buffers, so the same
    one-shot, cache-cold traffic), and over a 1 GiB buffer; the same copies
    read with the decode product's own pattern (its grid, waves, units and
    two-unit ring, no arithmetic); plus the shader clock (s_memtime against
    the 100 MHz s_memrealtime), idle and while streaming."""
    import ctypes

    lib = probe_lib()
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def read(buf, nt=1):
        st = lib.tqp_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), READ_BLOCKS,
                          READ_THREADS, nt, ctypes.c_void_p(sink.data_ptr()), stream())
        if st != 0:
            raise RuntimeError(f"tqp_read failed: hipError {st}")

    nb = bufs[0].numel()
    for i in range(16):
        read(bufs[i % len(bufs)])
    r71 = per_call_us(graph_trials(torch, lambda i: read(bufs[i % len(bufs)]), K, trials), K)
    r71_c = per_call_us(graph_trials(torch, lambda i: read(bufs[i % len(bufs)], 0), K, trials), K)

    def read_units(buf):
        # the decode's 512 row tiles of 32 units (4352 bytes each)
        st = lib.tqp_read_units(ctypes.c_void_p(buf.data_ptr()), DECODE_TILES, DECODE_UNITS,
                                ctypes.c_void_p(sink.data_ptr()), stream())
        if st != 0:
            raise RuntimeError(f"tqp_read_units failed: hipError {st}")

    if nb != DECODE_TILES * DECODE_UNITS * 4352:
        raise RuntimeError("the rotated copies are not the decode's 512 x 32 units")
    r71_p = per_call_us(graph_trials(torch, lambda i: read_units(bufs[i % len(bufs)]), K, trials), K)
    big = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        read(big)
    rbig = per_call_us(graph_trials(torch, lambda i: read(big), 10, trials), 10)
    # clock
    blocks = 2048
    out = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    mhz = {}
    for label, iters, buf in (("spin", 200000, None), ("streaming", 400, big)):
        for _ in range(2):
            st = lib.tqp_clock(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                               ctypes.c_void_p(buf.data_ptr()) if buf is not None else None,
                               buf.numel() * 4 if buf is not None else 0, stream())
            if st != 0:
                raise RuntimeError(f"tqp_clock failed: hipError {st}")
        torch.cuda.synchronize()
        h = out.cpu().numpy().reshape(blocks, 2).astype(np.float64)
        mhz[label] = float(np.median(100.0 * h[:, 0] / np.maximum(h[:, 1], 1)))
    del big
    return {"read_71MB_rotated_us": r71["us"], "read_71MB_rotated_gbs": nb / r71["us"] / 1e3,
            "read_71MB_rotated_cached_loads_gbs": nb / r71_c["us"] / 1e3,
            "read_71MB_decode_pattern_us": r71_p["us"], "read_71MB_decode_pattern_gbs": nb / r71_p["us"] / 1e3,
            "read_1GiB_gbs": (1 << 30) / rbig["us"] / 1e3,
            "read_shape": f"{READ_BLOCKS} workgroups x {READ_THREADS} threads, 4 x 16 B non-temporal loads in flight per thread",
            "sclk_mhz_spin": mhz["spin"], "sclk_mhz_streaming": mhz["streaming"]}


# ----------------------------------------------------------------- counters on record
def source_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# the sources each benchmarked kernel is compiled from: a recorded counter
# figure is reported only while their hash matches
# (with the build script, which holds the compiler flags)
KERNEL_SOURCES = {
    "gemv_pq2_kernel": ["k_gemv_pq2.hip", "q8k_block.h", "kernels.h", "layout.h", "../build.py"],
    "gemv_pq2_batch_kernel": ["k_gemv_pq2.hip", "q8k_block.h", "kernels.h", "layout.h", "../build.py"],
    "gemm_pq2_kernel": ["k_gemm_pq2.hip", "kernels.h", "layout.h", "../build.py"],
    "gemv_ptq1_kernel": ["k_gemv_ptq1.hip", "kernels.h", "layout.h", "../build.py"],
    "gemm_ptq1_kernel": ["k_gemm_ptq1.hip", "kernels.h", "layout.h", "../build.py"],
    "quantize_q8k_kernel": ["k_quant.hip", "q8k_block.h", "kernels.h", "../build.py"],
}


def kernel_family(name: str):
    for fam in KERNEL_SOURCES:
        if f"{fam}<" in name or f"{fam}(" in name or name.endswith(fam):
            return fam
    return None


def recorded_counters():
    """Per-kernel counter figures from the committed counter runs whose
    kernel sources still hash the same, keyed by label; {} if none."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for label, e in rec.get("kernels", {}).items():
        fam = e.get("family")
        if fam in KERNEL_SOURCES and e.get("source_sha256") == source_sha256(KERNEL_SOURCES[fam]):
            out[label] = e
    return out


# ----------------------------------------------------------------- counter-run workload
def probe_workloads(torch, tq, names):
    """Every benchmarked kernel 20 times (what the counter runs profile), then
    three device copies of 1 GiB that calibrate the byte counters."""
    names = set(names.split(","))
    every = "all" in names
    n = 20
    if every or "decode" in names:
        log("probe: decode")
        fmt, R, C, Ws, x = resident_copies(torch, tq, "decode_32768x8192")
        xd = torch.from_numpy(x).cuda()
        q, d, bs = tq.quantize_q8k(xd)
        y = torch.empty(R, dtype=torch.float32, device="cuda")
        for i in range(n):
            tq.gemv_f32(fmt, Ws[i % len(Ws)], R, C, xd[0], out=y)
        for i in range(n):
            tq.gemv(fmt, Ws[i % len(Ws)], R, C, q, d, bs, out=y)
        if every or "ceiling" in names:
            lib = probe_lib()
            import ctypes

            sink = torch.zeros(1, dtype=torch.int32, device="cuda")
            for i in range(n):
                lib.tqp_read(ctypes.c_void_p(Ws[i % len(Ws)].data_ptr()), Ws[0].numel(), READ_BLOCKS, READ_THREADS, 1,
                             ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            for i in range(n):
                lib.tqp_read_units(ctypes.c_void_p(Ws[i % len(Ws)].data_ptr()), DECODE_TILES, DECODE_UNITS,
                                   ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        del Ws
    if every or "quant" in names:
        log("probe: quantize")
        x = torch.from_numpy(TI.activations(TI.rng(TI.DECODE, 0, 0, 2), 1, 8192)).cuda()
        for _ in range(n):
            tq.quantize_q8k(x)
    if every or "prefill" in names:
        for T in (4, 64):
            log(f"probe: prefill t{T}")
            fmt, R, C, Ws, x = resident_copies(torch, tq, f"prefill_17408x5120_t{T}")
            q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
            y = torch.empty((T, R), dtype=torch.float32, device="cuda")
            for i in range(n):
                tq.gemm(fmt, Ws[i % len(Ws)], R, C, q, d, bs, out=y)
            torch.cuda.synchronize()
            del Ws
    if every or "ptq1" in names:
        log("probe: ptq1")
        fmt, R, C, Ws, x = resident_copies(torch, tq, "ptq1_32768x8192")
        q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
        y = torch.empty(R, dtype=torch.float32, device="cuda")
        ws = tq.workspace(fmt, R, C, 1)
        for i in range(n):
            tq.gemv(fmt, Ws[i % len(Ws)], R, C, q, d, bs, out=y, ws=ws)
        torch.cuda.synchronize()
        del Ws
        for T in (4, 64):
            log(f"probe: ptq1 prefill t{T}")
            fmt, R, C, Ws, x = resident_copies(torch, tq, f"ptq1_prefill_17408x5120_t{T}")
            q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
            y = torch.empty((T, R), dtype=torch.float32, device="cuda")
            for i in range(n):
                tq.gemm(fmt, Ws[i % len(Ws)], R, C, q, d, bs, out=y)
            torch.cuda.synchronize()
            del Ws
    if every or "tiny" in names:
        log("probe: tiny")
        fmt, Wc, x = TI.make("tiny_256x1024")
        R, G, _ = Wc.shape
        C = G * 128
        W = tq.repack(torch.from_numpy(Wc.reshape(-1)).cuda(), fmt, R, C)
        xd = torch.from_numpy(x[0].copy()).cuda()
        y = torch.empty(R, dtype=torch.float32, device="cuda")
        ws = tq.workspace(fmt, R, C, 1)
        for _ in range(n):
            tq.gemv_f32(fmt, W, R, C, xd, out=y, ws=ws)
    if every or "step64" in names:
        log("probe: step64")
        s = Step64(torch, tq)
        for _ in range(2):
            s.step()
        torch.cuda.synchronize()
        del s
    torch.cuda.synchronize()
    log("probe: 1 GiB copies")
    a = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


# ----------------------------------------------------------------- rocprofv3 summaries
def _read_csvs(d, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _dims(r):
    """(grid work-items, workgroup size) of a counter-collection or kernel-trace row."""
    def total(base):
        if base in r and r[base] not in (None, ""):
            return int(r[base])
        return int(r[base + "_X"]) * int(r.get(base + "_Y") or 1) * int(r.get(base + "_Z") or 1)
    return total("Grid_Size"), total("Workgroup_Size")


def short_name(name: str) -> str:
    if name.startswith("void "):
        name = name[5:]
    name = name.replace("tq::(anonymous namespace)::", "tq::").replace("(anonymous namespace)::", "")
    cut = name.find("(")
    return name[:cut] if cut > 0 else name


NUM_XCD = 8  # rocprofv3 sums GRBM_GUI_ACTIVE over the eight XCDs


def summarize(counter_dir, trace_dir=None):
    """Median counter value per (kernel, grid) from rocprofv3 counter-collection
    CSVs; byte counters scaled by what they read for the 1 GiB device copy;
    durations and back-to-back launch periods from a kernel-trace CSV; derived
    figures:
      mfma_ops        = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 (2 ops per int8 MAC)
      mfma_util       = mfma_ops / (trace duration x dense int8 peak)
      gui_cycles      = GRBM_GUI_ACTIVE / 8 (one XCD's busy cycles)
      valu_busy       = SQ_ACTIVE_INST_VALU x 4 / (SIMDs x gui_cycles): the
                        share of SIMD cycles issuing VALU (the counter is in
                        quad-cycles, summed over waves)
      mfma_busy       = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x gui_cycles)
      valu_issue_us   = SQ_ACTIVE_INST_VALU x 4 / SIMDs / 2.4 GHz: one SIMD's
                        VALU issue time at the peak clock
      valu_frac_trace = valu_issue_us / trace_avg_us (a lower bound of the
                        SIMDs' VALU-busy share over the kernel's own run:
                        GRBM_GUI_ACTIVE also counts cycles around it)"""
    rows = _read_csvs(counter_dir, "counter_collection.csv") if counter_dir else []
    vals = {}
    lds = {}
    for r in rows:
        key = (short_name(r["Kernel_Name"]),) + _dims(r)
        lds[key] = int(r["LDS_Block_Size"])
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}
    # calibration: the 1 GiB copy reads and writes exactly 2^30 bytes
    copy = [cs for k, cs in med.items() if "copyBuffer" in k[0]]  # the largest reading is the 1 GiB copy
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        got = [cs[c] for cs in copy if c in cs]
        if got:
            scale[c] = (1 << 30) / (max(got) * 1024.0)
    durations, periods = {}, {}
    if trace_dir:
        trace = []
        for r in _read_csvs(trace_dir, "kernel_trace.csv"):
            key = (short_name(r["Kernel_Name"]),) + _dims(r)
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            trace.append((t0, t1, key))
            durations.setdefault(key, []).append((t1 - t0) * 1e-3)
        trace.sort()
        # start-to-start interval of consecutive launches of one kernel with
        # nothing between them (a graph replay): the per-launch time that a
        # replay timed with events measures
        for (s0, _e0, k0), (s1, _e1, k1) in zip(trace, trace[1:]):
            if k0 == k1:
                periods.setdefault(k0, []).append((s1 - s0) * 1e-3)
    out = {}
    for key in sorted(set(med) | set(durations), key=lambda k: (k[0], k[1])):
        fam = kernel_family(key[0])
        if fam is None and "copyBuffer" not in key[0] and "read_kernel" not in key[0] and "units_kernel" not in key[0]:
            continue
        cs = med.get(key, {})
        e = {"kernel": key[0], "grid": key[1], "block": key[2], "lds": lds.get(key), "family": fam}
        for c, v in cs.items():
            e[c] = v
        if "FETCH_SIZE" in cs and "FETCH_SIZE" in scale:
            e["fetch_bytes"] = cs["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        if "WRITE_SIZE" in cs and "WRITE_SIZE" in scale:
            e["write_bytes"] = cs["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
        if key in durations:
            ds = durations[key]
            e["trace_launches"] = len(ds)
            e["trace_avg_us"] = sum(ds) / len(ds)
            e["trace_median_us"] = statistics.median(ds)
        if len(periods.get(key, [])) >= 5:
            e["trace_period_us"] = statistics.median(periods[key])
        if "SQ_INSTS_VALU_MFMA_MOPS_I8" in cs:
            e["mfma_ops"] = cs["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512
            if "trace_avg_us" in e:
                e["mfma_util"] = e["mfma_ops"] / (e["trace_avg_us"] * 1e-6 * INT8_MFMA_PEAK_TOPS * 1e12)
        if "SQ_ACTIVE_INST_VALU" in cs:
            e["valu_issue_us"] = cs["SQ_ACTIVE_INST_VALU"] * 4 / (NUM_CU * 4) / (PEAK_SCLK_GHZ * 1e3)
            if "trace_avg_us" in e:
                e["valu_frac_trace"] = e["valu_issue_us"] / e["trace_avg_us"]
        gui = cs.get("GRBM_GUI_ACTIVE")
        if gui:
            cyc = gui / NUM_XCD
            e["gui_cycles"] = cyc
            if "SQ_ACTIVE_INST_VALU" in cs:
                e["valu_busy"] = cs["SQ_ACTIVE_INST_VALU"] * 4 / (NUM_CU * 4 * cyc)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
                e["mfma_busy"] = cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (NUM_CU * 4 * cyc)
        if fam:
            e["source_sha256"] = source_sha256(KERNEL_SOURCES[fam])
        out[f"{key[0]} grid={key[1]} block={key[2]}"] = e
    return {"scale": scale, "kernels": out}


def print_summary(s):
    cols = ["trace_launches", "trace_avg_us", "trace_period_us", "fetch_bytes", "write_bytes", "mfma_ops", "mfma_util",
            "mfma_busy", "valu_issue_us", "valu_frac_trace", "valu_busy", "VALUBusy", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_WAIT_INST_LDS",
            "SQ_LDS_BANK_CONFLICT", "gui_cycles"]
    present = [c for c in cols if any(c in e for e in s["kernels"].values())]
    print("byte-counter scale (bytes per KiB read):", {k: round(v, 6) for k, v in s["scale"].items()})
    print()
    print("| kernel | grid / block / LDS | " + " | ".join(present) + " |")
    print("|---|---|" + "---|" * len(present))
    for e in s["kernels"].values():
        cells = []
        for c in present:
            v = e.get(c)
            cells.append("" if v is None else (f"{v:.4g}" if isinstance(v, float) else str(v)))
        print(f"| {e['kernel']} | {e['grid']} / {e['block']} / {e['lds']} | " + " | ".join(cells) + " |")


# ----------------------------------------------------------------- CPU oracle
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float):
    """The CPU oracle on the host cores: quantize + product over the full
    32768 x 8192 matrix, repeated while the wall budget lasts.  Beside it, in
    about a third of that budget each: the same on one core, the ptq1_0
    32768 x 8192 product and the 17408 x 5120 prompt product at 64 tokens on
    all cores (row samples, scaled to the whole matrix)."""
    import oracle

    oracle.build(force=False)
    fmt, Wc, x = TI.make("decode_32768x8192")
    R, G, _ = Wc.shape
    cores = len(os.sched_getaffinity(0))

    def run(call, budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            call()
            n += 1
            if time.perf_counter() - t0 >= budget:
                return n, time.perf_counter() - t0

    def full_pass():
        q, d, _ = oracle.quantize_q8k(x)
        oracle.matmul(fmt, Wc, q, d, threads=cores)

    passes, dt = run(full_pass, seconds)
    out = {"value": passes * R * G * 128 / dt / 1e9, "unit": "Gweights/s", "cores": cores, "kind": "oracle",
           "sample": f"{passes} full passes (q8_K quantize + 32768x8192 pq2_0 product, fp64 epilogue) over {dt:.1f} s, "
                     f"row ranges split over {cores} threads",
           "cpu": _cpu_model(), "cflags": " ".join(oracle.CFLAGS)}
    side = seconds / 3
    q1, d1, _ = oracle.quantize_q8k(x)
    n, dt = run(lambda: oracle.matmul(fmt, Wc, q1, d1, rows=(0, 4096), threads=1), side)
    out["one_core_gweights_s"] = n * 4096 * G * 128 / dt / 1e9
    pfmt, Pc, px = TI.make("ptq1_32768x8192")
    pq, pd, _ = oracle.quantize_q8k(px)
    n, dt = run(lambda: oracle.matmul(pfmt, Pc, pq, pd, threads=cores), side)
    out["ptq1_gweights_s"] = n * Pc.shape[0] * Pc.shape[1] * 128 / dt / 1e9
    del Pc
    gfmt, Gc, gx = TI.make("prefill_17408x5120_t64")
    gq, gd, _ = oracle.quantize_q8k(gx)
    sub = np.ascontiguousarray(Gc[:1024])
    n, dt = run(lambda: oracle.matmul(gfmt, sub, gq, gd, threads=cores), side)
    out["prefill_t64_gmac_s"] = n * 1024 * Gc.shape[1] * 128 * gx.shape[0] / dt / 1e9
    return out


# ----------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize:
        s = summarize(args.summarize, args.kernel_trace)
        print_summary(s)
        if args.write_counters:
            s["command_note"] = "see the profiles/*.md summaries for the rocprofv3 commands"
            with open(COUNTERS_FILE, "w") as f:
                json.dump(s, f, indent=1, sort_keys=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bit_quantized_matvec_amd as tq

    if args.probe:
        probe_workloads(torch, tq, args.probe)
        return
    trials = max(5, args.trials)
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle)
    K = args.steps
    log("decode bench")
    dec = decode_bench(torch, tq, K, args.warmup, trials)
    R, C = dec["R"], dec["C"]
    main_t = dec["main"]
    step_s = main_t["median_s"]
    value = K * R * C / step_s / 1e9
    kernel_us = step_s * 1e6 / K  # the step is one kernel launch
    achieved = dec["algo_bytes"] / (kernel_us * 1e-6) / 1e9
    log("ceiling probe")
    ceil = ceiling_bench(torch, dec["Ws"], min(K, 1000), trials)
    del dec["Ws"]
    counters = recorded_counters()
    # the timed kernel: gemv_pq2_kernel<RING, IDOTS=false, NT, LDSQ, FX=true, XB> on 512 workgroups of 256
    fused = {k: v for k, v in counters.items() if v.get("family") == "gemv_pq2_kernel" and v.get("grid") == 131072
             and "false, true, true, true," in v.get("kernel", "")}
    traffic = None
    for v in fused.values():
        if "fetch_bytes" in v and "write_bytes" in v:
            traffic = round(v["fetch_bytes"] + v["write_bytes"])
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3 / K, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode_32768x8192", "format": "pq2_0", "rows": R, "cols": C, "tokens": 1,
                   "step": "tq_gemv_f32 (q8_K quantization inside the product kernel)",
                   "weight_copies_rotated": dec["copies"],
                   "timing": f"hip graph of K steps, median of {main_t['trials']} replays timed with HIP events, "
                             f"after {SETTLE_S:g} s of untimed replays ({main_t['settle_replays']})"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "gemv_pq2_kernel (fused q8_K)", "kernel_us": round(kernel_us, 3),
                     "kernel_us_min": round(main_t["min_s"] * 1e6 / K, 3),
                     "kernel_us_max": round(main_t["max_s"] * 1e6 / K, 3),
                     "algo_bytes": dec["algo_bytes"],
                     "frac_of_measured_ceiling": round(ceil["read_71MB_rotated_us"] / kernel_us, 4)},
    }
    extra = {"decode_wall_gweights_s": round(K * R * C / main_t["wall_median_s"] / 1e9, 2),
             "decode_eager_gweights_s": round(K * R * C / dec["eager_s"] / 1e9, 2),
             "decode_two_kernel_step": rounded({
                 "step": "tq_quantize_q8k + tq_gemv",
                 "gweights_s": K * R * C / dec["two"]["median_s"] / 1e9,
                 "us_per_step": dec["two"]["median_s"] * 1e6 / K,
                 "gemv_us": dec["gemv"]["median_s"] * 1e6 / K,
                 "quant_us": dec["quant"]["median_s"] * 1e6 / K,
                 "gemv_hbm_frac": dec["algo_bytes_gemv"] / (dec["gemv"]["median_s"] / K) / 1e9 / HBM_PEAK_GBS}),
             "decode_weight_gbs": round(dec["weight_bytes"] / (kernel_us * 1e-6) / 1e9, 1),
             "ceiling": rounded(ceil, 3)}
    if not args.no_extra:
        log("prefill")
        for T in (4, 64):
            extra[f"prefill_t{T}"] = rounded(prefill_bench(torch, tq, T, 200, trials))
        log("64-layer step")
        extra["step64"] = rounded(step64_bench(torch, tq, 5, trials))
        log("ptq1")
        extra["ptq1_decode"] = rounded(ptq1_bench(torch, tq, 200, trials))
        for T in (4, 64):
            extra[f"ptq1_prefill_t{T}"] = rounded(prefill_bench(torch, tq, T, 100, trials, "ptq1_0"))
        extra["quantize_8192"] = rounded(quantize_bench(torch, tq, 200, trials), 3)
        extra["tiny_256x1024"] = rounded(tiny_bench(torch, tq, 1000, trials), 3)
    if counters:
        extra["counters"] = {k: rounded({c: v[c] for c in ("fetch_bytes", "write_bytes", "mfma_util", "mfma_busy",
                                                          "valu_frac_trace", "trace_avg_us", "trace_period_us")
                                         if c in v}, 4)
                             for k, v in counters.items()}
    out["extra"] = extra
    if not args.no_cpu:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
