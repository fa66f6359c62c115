#!/usr/bin/env python3
"""Benchmark of the packed-ternary x q8_K hot path on one MI355X.

One step = one pass of the decode hot path over one token: q8_K quantization
of a fresh fp32 activation vector, then the 32768 x 8192 pq2_0 matrix-vector
product (tq_quantize_q8k + tq_gemv through the C ABI).  The weights are
resident in HBM; eight repacked copies (570 MB) are rotated so that the
256 MB Infinity Cache cannot serve a repeat call.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  `value` is Gweights/s of the whole timed region (K
steps captured in one HIP graph and replayed once, bracketed by
synchronizations).  `roofline` is the matrix-vector kernel's algorithmic HBM
bytes per launch divided by its mean duration, measured with one HIP event
pair around K back-to-back launches of that kernel on the stream it runs on.
`extra` carries the prompt-product (17408 x 5120, 4 and 64 tokens), 64-layer
step and ptq1_0 figures; `cpu_baseline` times the CPU oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true", help="skip the prompt-product and ptq1_0 figures")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall budget of the CPU baseline")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run 20 decode matrix-vector launches and three 1 GiB device copies "
                         "(the workload of the FETCH_SIZE / WRITE_SIZE counter runs), print nothing")
    return ap.parse_args()


def copies_for(nbytes: int) -> int:
    """Enough distinct weight copies that the rotation exceeds twice the MALL."""
    return max(2, -(-2 * MALL_BYTES // nbytes))


def batch_us(torch, call, K):
    """Mean duration of K back-to-back launches of call(i) on the current
    stream: one HIP event pair around the whole batch (no host gaps between
    the kernels, so this is the kernels' own average as a tracer sees it)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / K


def graph_time(torch, step, K):
    """Capture K calls of step() in one graph, replay once; returns seconds."""
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
    g.replay()  # warm replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def decode_bench(torch, tq, K, W):
    fmt, Wc, x = TI.make("decode_32768x8192")
    R, G, _ = Wc.shape
    C = G * 128
    wdev = torch.from_numpy(Wc.reshape(-1)).cuda()
    ncopy = copies_for(tq.repacked_bytes(fmt, R, C))
    Ws = [tq.repack(wdev, fmt, R, C) for _ in range(ncopy)]
    del wdev
    # a fresh activation vector per step: rotate over a pool of distinct vectors
    xs = torch.from_numpy(TI.activations(TI.rng(TI.DECODE, 0, 0, 1), 64, C)).cuda()
    q = torch.empty((1, C), dtype=torch.int8, device="cuda")
    d = torch.empty((1, C // 256), dtype=torch.float32, device="cuda")
    bs = torch.empty((1, C // 16), dtype=torch.int16, device="cuda")
    y = torch.empty(R, dtype=torch.float32, device="cuda")

    def step_two(i):
        tq.quantize_q8k(xs[i % 64: i % 64 + 1], out=(q, d, bs))
        tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y)

    def step(i):
        # one launch: every workgroup quantizes x itself, on chip
        tq.gemv_f32(fmt, Ws[i % ncopy], R, C, xs[i % 64], out=y)

    for i in range(W):
        step_two(i)
        step(i)
    torch.cuda.synchronize()
    # eager pass of whole steps (host-launched, for reference)
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    # the product kernel alone, K launches back to back on this stream
    fused_us = batch_us(torch, step, K)
    gemv_us = batch_us(torch, lambda i: tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y), K)
    quant_us = batch_us(torch, lambda i: tq.quantize_q8k(xs[i % 64: i % 64 + 1], out=(q, d, bs)), K)
    # graph passes: the timed region of `value` (fused step), and the two-kernel step
    graph_s = graph_time(torch, step, K)
    graph_two_s = graph_time(torch, step_two, K)
    wbytes = tq.repacked_bytes(fmt, R, C)
    return {
        "R": R, "C": C, "copies": ncopy, "graph_s": graph_s, "graph_two_s": graph_two_s, "eager_s": eager_s,
        "fused_us": fused_us, "gemv_us": gemv_us, "quant_us": quant_us,
        # algorithmic bytes per launch: weights + fp32 x + fp32 y (fused); weights + q + d + y (two-kernel GEMV)
        "algo_bytes": wbytes + 4 * C + 4 * R, "algo_bytes_gemv": wbytes + C + 4 * (C // 256) + 4 * R,
        "weight_bytes": wbytes,
    }


def prefill_bench(torch, tq, T, K, fmt_name="pq2_0"):
    prefix = "prefill" if fmt_name == "pq2_0" else "ptq1_prefill"
    fmt, Wc, x = TI.make(f"{prefix}_17408x5120_t{T}")
    R, G, _ = Wc.shape
    C = G * 128
    wdev = torch.from_numpy(Wc.reshape(-1)).cuda()
    ncopy = copies_for(tq.repacked_bytes(fmt, R, C))
    Ws = [tq.repack(wdev, fmt, R, C) for _ in range(ncopy)]
    del wdev
    q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
    y = torch.empty((T, R), dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, R, C, T)
    call = lambda i: tq.gemm(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y, ws=ws)
    for i in range(20):
        call(i)
    torch.cuda.synchronize()
    us = graph_time(torch, call, K) * 1e6 / K  # replayed from a graph: device time, no host launch cost
    macs = R * C * T
    r = {"tokens": T, "us": us, "gmac_s": macs / us / 1e3}
    if fmt == "pq2_0":  # int8 matrix cores; ptq1_0 takes its dot products on the vector units
        r["mfma_frac"] = 2 * macs / (us * 1e-6) / (INT8_MFMA_PEAK_TOPS * 1e12)
    bsum_bytes = 2 * T * (C // 16) if fmt == "ptq1_0" else 0
    r["hbm_gbs"] = (tq.repacked_bytes(fmt, R, C) + T * C + bsum_bytes + 4 * T * (C // 256) + 4 * T * R) / us / 1e3
    return r


def ptq1_bench(torch, tq, K):
    fmt, Wc, x = TI.make("ptq1_32768x8192")
    R, G, _ = Wc.shape
    C = G * 128
    wdev = torch.from_numpy(Wc.reshape(-1)).cuda()
    ncopy = copies_for(tq.repacked_bytes(fmt, R, C))
    Ws = [tq.repack(wdev, fmt, R, C) for _ in range(ncopy)]
    del wdev
    q, d, bs = tq.quantize_q8k(torch.from_numpy(x).cuda())
    y = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, R, C, 1)
    call = lambda i: tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y, ws=ws)
    for i in range(20):
        call(i)
    torch.cuda.synchronize()
    us = graph_time(torch, call, K) * 1e6 / K  # replayed from a graph
    wb = tq.repacked_bytes(fmt, R, C)
    return {"us": us, "gweights_s": R * C / us / 1e3, "weight_gbs": wb / us / 1e3, "hbm_frac": wb / us / 1e3 / HBM_PEAK_GBS}


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


def step64_bench(torch, tq, reps):
    """The 64-layer decode step for one token: for each layer the gate, up,
    down, qkv and out matrices (distinct weights, 5.7 GB in all), each
    preceded by a fresh q8_K quantization of its own N(0,1) activation vector.
    The 320 quantize + matrix-vector pairs are captured in one graph."""
    fmt = "pq2_0"
    gen = torch.Generator(device="cuda")
    gen.manual_seed(TI.SEED_BASE + TI.STEP64)
    mats = []
    for layer in range(64):
        for _name, R, C in TI.STEP64_SHAPES:
            canon = synth_pq2_gpu(torch, gen, R, C)
            mats.append((R, C, tq.repack(canon, fmt, R, C, check_codes=False)))
            del canon
    kmax = max(C for _, C, _ in mats)
    rmax = max(R for R, _, _ in mats)
    xs = torch.randn((len(mats), kmax), device="cuda", generator=gen)
    q = torch.empty(kmax, dtype=torch.int8, device="cuda")
    d = torch.empty(kmax // 256, dtype=torch.float32, device="cuda")
    bs = torch.empty(kmax // 16, dtype=torch.int16, device="cuda")
    y = torch.empty(rmax, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(tq.workspace_bytes(fmt, R, C) for R, C, _ in mats), dtype=torch.uint8, device="cuda")

    def step_two(_i):
        for m, (R, C, Wd) in enumerate(mats):
            tq.quantize_q8k(xs[m, :C].view(1, C), out=(q[:C].view(1, C), d[: C // 256].view(1, -1), bs[: C // 16].view(1, -1)))
            tq.gemv(fmt, Wd, R, C, q[:C], d[: C // 256], bs[: C // 16], out=y[:R], ws=ws)

    names = [name for _layer in range(64) for name, _R, _C in TI.STEP64_SHAPES]
    ys = [torch.empty(R, dtype=torch.float32, device="cuda") for R, _C, _W in mats[:2]]
    ws_pair = torch.zeros(max(16, tq.workspace_bytes(fmt, sum(-(-R // 64) * 64 for R, _C, _W in mats[:2]), mats[0][1])),
                          dtype=torch.uint8, device="cuda")

    def step(_i):
        m = 0
        while m < len(mats):
            R, C, Wd = mats[m]
            if names[m] == "gate" and names[m + 1] == "up":
                # gate and up read the same layer input in a real model: one launch
                R2, _C2, Wd2 = mats[m + 1]
                tq.gemv_f32_batch(fmt, [Wd, Wd2], [R, R2], C, [xs[m, :C], xs[m + 1, :C]], outs=ys, ws=ws_pair)
                m += 2
                continue
            tq.gemv_f32(fmt, Wd, R, C, xs[m, :C], out=y[:R], ws=ws)
            m += 1

    step_two(0)
    step(0)
    torch.cuda.synchronize()
    g_s = graph_time(torch, step, reps)
    g2_s = graph_time(torch, step_two, reps)
    weights = sum(R * C for R, C, _ in mats)
    wbytes = sum(tq.repacked_bytes(fmt, R, C) for R, C, _ in mats)
    ms = g_s * 1e3 / reps
    return {"matrices": len(mats), "step": "tq_gemv_f32_batch for gate + up, tq_gemv_f32 for down, qkv, out",
            "ms_per_token": ms,
            "gweights_s": weights / (ms * 1e-3) / 1e9,
            "weight_gbs": wbytes / (ms * 1e-3) / 1e9, "hbm_frac": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "weight_bytes": wbytes, "two_kernel_ms_per_token": g2_s * 1e3 / reps}


def tiny_bench(torch, tq, K):
    """The 256x1024 workload: one fused call per step, replayed from a graph
    (launch-bound: its 70 KB of weights stay in the caches)."""
    fmt, Wc, x = TI.make("tiny_256x1024")
    R, G, _ = Wc.shape
    C = G * 128
    W = tq.repack(torch.from_numpy(Wc.reshape(-1)).cuda(), fmt, R, C)
    xd = torch.from_numpy(x[0].copy()).cuda()
    y = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, R, C, 1)
    step = lambda i: tq.gemv_f32(fmt, W, R, C, xd, out=y, ws=ws)
    t = graph_time(torch, step, K)
    return {"rows": R, "cols": C, "us_per_step": t * 1e6 / K, "gweights_s": R * C * K / t / 1e9}


def quantize_bench(torch, tq, K):
    C = 8192
    xs = torch.from_numpy(TI.activations(TI.rng(TI.DECODE, 0, 0, 2), 1, C)).cuda()
    out = (torch.empty((1, C), dtype=torch.int8, device="cuda"), torch.empty((1, 32), dtype=torch.float32, device="cuda"),
           torch.empty((1, 512), dtype=torch.int16, device="cuda"))
    for _ in range(20):
        tq.quantize_q8k(xs, out=out)
    torch.cuda.synchronize()
    us = batch_us(torch, lambda i: tq.quantize_q8k(xs, out=out), K)
    # replayed from a graph: the kernel's cadence without the host's launch cost
    graph_us = graph_time(torch, lambda i: tq.quantize_q8k(xs, out=out), K) * 1e6 / K
    return {"cols": C, "us": us, "graph_us": graph_us}


def ceiling_probe(torch):
    """Plain streaming kernels of known size: torch's sum (read) and copy."""
    n = (2 << 30) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    for _ in range(3):
        a.sum()
        b.copy_(a[: n // 2])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a.sum()
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 10 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record()
    for _ in range(10):
        b.copy_(a[: n // 2])
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * 4 * (n // 2) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return {"read_sum_2GiB_gbs": read_gbs, "copy_1GiB_gbs": copy_gbs}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_32768x8192.json")
# the sources the decode kernel is compiled from: the recorded traffic holds while their hash matches
GEMV_SOURCES = [os.path.join(ROOT, "bit_quantized_matvec_amd", "csrc", f) for f in ("k_gemv_pq2.hip", "q8k_block.h")]


def traffic_probe(torch, tq):
    """The workload of the HBM-traffic counter runs: 20 launches of the
    decode product with quantization inside (the timed step), then 20 of the
    matrix-vector kernel on a stored q8_K vector (rotating weight copies, as
    in the timed run), and three device-to-device copies of 1 GiB, whose
    known byte count calibrates the counters."""
    fmt, Wc, x = TI.make("decode_32768x8192")
    R, G, _ = Wc.shape
    C = G * 128
    wdev = torch.from_numpy(Wc.reshape(-1)).cuda()
    ncopy = copies_for(tq.repacked_bytes(fmt, R, C))
    Ws = [tq.repack(wdev, fmt, R, C) for _ in range(ncopy)]
    del wdev
    xd = torch.from_numpy(x).cuda()
    q, d, bs = tq.quantize_q8k(xd)
    y = torch.empty(R, dtype=torch.float32, device="cuda")
    for i in range(20):
        tq.gemv_f32(fmt, Ws[i % ncopy], R, C, xd[0], out=y)
    for i in range(20):
        tq.gemv(fmt, Ws[i % ncopy], R, C, q, d, bs, out=y)
    torch.cuda.synchronize()
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty(n, dtype=torch.float32, device="cuda")
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def kernel_source_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for path in GEMV_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter
    runs, or None if the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        sha = kernel_source_sha256()
    except (OSError, ValueError):
        return None
    return rec.get("traffic_bytes") if rec.get("kernel_source_sha256") == sha else None


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
    # one core, the first 4096 rows of the same product
    q1, d1, _ = oracle.quantize_q8k(x)
    n, dt = run(lambda: oracle.matmul(fmt, Wc, q1, d1, rows=(0, 4096), threads=1), side)
    out["one_core_gweights_s"] = n * 4096 * G * 128 / dt / 1e9
    # ptq1_0 32768 x 8192 on all cores
    pfmt, Pc, px = TI.make("ptq1_32768x8192")
    pq, pd, _ = oracle.quantize_q8k(px)
    n, dt = run(lambda: oracle.matmul(pfmt, Pc, pq, pd, threads=cores), side)
    out["ptq1_gweights_s"] = n * Pc.shape[0] * Pc.shape[1] * 128 / dt / 1e9
    del Pc
    # prompt product 17408 x 5120, 64 tokens, a block of 1024 rows on all cores
    gfmt, Gc, gx = TI.make("prefill_17408x5120_t64")
    gq, gd, _ = oracle.quantize_q8k(gx)
    sub = np.ascontiguousarray(Gc[:1024])
    n, dt = run(lambda: oracle.matmul(gfmt, sub, gq, gd, threads=cores), side)
    out["prefill_t64_gmac_s"] = n * 1024 * Gc.shape[1] * 128 * gx.shape[0] / dt / 1e9
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bit_quantized_matvec_amd as tq

    if args.traffic_probe:
        traffic_probe(torch, tq)
        return
    log("decode bench")
    dec = decode_bench(torch, tq, args.steps, args.warmup)
    R, C, K = dec["R"], dec["C"], args.steps
    value = K * R * C / dec["graph_s"] / 1e9
    achieved = dec["algo_bytes"] / (dec["fused_us"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(dec["graph_s"] * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode_32768x8192", "format": "pq2_0", "rows": R, "cols": C, "tokens": 1,
                   "step": "tq_gemv_f32 (q8_K quantization inside the product kernel)",
                   "weight_copies_rotated": dec["copies"], "timing": "hip graph of K steps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": "gemv_pq2_kernel (fused q8_K)", "kernel_us": round(dec["fused_us"], 3),
                     "algo_bytes": dec["algo_bytes"]},
    }
    extra = {"decode_eager_gweights_s": round(K * R * C / dec["eager_s"] / 1e9, 2),
             "decode_two_kernel_step": {"step": "tq_quantize_q8k + tq_gemv",
                                        "gweights_s": round(K * R * C / dec["graph_two_s"] / 1e9, 2),
                                        "us_per_step": round(dec["graph_two_s"] * 1e6 / K, 3),
                                        "gemv_us": round(dec["gemv_us"], 3), "quant_us": round(dec["quant_us"], 3),
                                        "gemv_hbm_frac": round(dec["algo_bytes_gemv"] / (dec["gemv_us"] * 1e-6) / 1e9
                                                               / HBM_PEAK_GBS, 4)},
             "decode_weight_gbs": round(dec["weight_bytes"] / (dec["fused_us"] * 1e-6) / 1e9, 1),
             "decode_kernel_gweights_s": round(R * C / dec["fused_us"] / 1e3, 1)}
    if not args.no_extra:
        log("prefill / ptq1 / quantize / ceiling")
        for T in (4, 64):
            p = prefill_bench(torch, tq, T, 200)
            extra[f"prefill_t{T}"] = {k: round(v, 4) if isinstance(v, float) else v for k, v in p.items()}
        log("64-layer step")
        extra["step64"] = {k: round(v, 4) if isinstance(v, float) else v for k, v in step64_bench(torch, tq, 5).items()}
        p = ptq1_bench(torch, tq, 200)
        extra["ptq1_decode"] = {k: round(v, 4) for k, v in p.items()}
        for T in (4, 64):
            p = prefill_bench(torch, tq, T, 100, "ptq1_0")
            extra[f"ptq1_prefill_t{T}"] = {k: round(v, 4) if isinstance(v, float) else v for k, v in p.items()}
        extra["quantize_8192"] = {k: round(v, 3) if isinstance(v, float) else v for k, v in quantize_bench(torch, tq, 200).items()}
        extra["tiny_256x1024"] = {k: round(v, 3) if isinstance(v, float) else v for k, v in tiny_bench(torch, tq, 1000).items()}
        extra["ceiling"] = {k: round(v, 1) for k, v in ceiling_probe(torch).items()}
    out["extra"] = extra
    if not args.no_cpu:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
