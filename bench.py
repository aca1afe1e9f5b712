"""Benchmark: effective weight-stream GB/s of the affine group-quantized
product on one MI355X, for the 27B-style dense MLP up projection
(K = 5120, N = 17408, 4-bit codes, G = 32) at M = 1, 4 and 16 activation rows.

One step = one qmm_forward call at each of M = 1, 4, 16 (three launches),
every call reading its own copy of the packed weights, scales and biases:
the copies rotate over more than 512 MB so that no call is served from the
256 MB Infinity Cache. Inputs are resident in HBM before timing starts.

value = weight bytes streamed per step / step time, where weight bytes per
call = N*K*(bits/8 + 4/G) (codes plus fp16 scale and bias per group).

Prints one JSON line. Synthetic data (seeded; no trained weights).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

import numpy as np
import torch

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import qmm_inputs  # noqa: E402
from qmm_inputs import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
ROTATION_BYTES = 512 * 2 ** 20
CELLS_M = (1, 4, 16)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="output rows of the CPU oracle sample (0: all rows)")
    return ap.parse_args()


def make_copies(shape, dev, seed=0):
    """Packed weights, scales, biases (C copies, > 512 MB in total) and x [16, K]."""
    p = qmm_inputs.make_problem(seed=seed, M=max(CELLS_M), K=shape.K, N=shape.N, bits=shape.bits,
                                G=shape.G, packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s = torch.from_numpy(p.scales).to(dev)
    b = torch.from_numpy(p.biases).to(dev)
    copies = max(2, -(-ROTATION_BYTES // shape.weight_bytes))
    sets = [(wq, s, b)] + [(wq.clone(), s.clone(), b.clone()) for _ in range(copies - 1)]
    x = torch.from_numpy(p.x).to(dev)
    return p, sets, x


def time_launches(fn, reps: int, stream) -> float:
    """Average ms per call of fn(i) over `reps` back-to-back calls (HIP events on `stream`)."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(reps):
        fn(i)
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps


def cpu_baseline(p, shape, rows: int):
    """The fp64 oracle on the host cores, on a bounded sample of output rows."""
    import oracle
    o = oracle.get()
    threads = oracle.default_threads()
    rng = np.random.default_rng(1)
    rows = shape.N if rows <= 0 else min(rows, shape.N)
    sel = np.sort(rng.choice(shape.N, size=rows, replace=False))
    t0 = time.perf_counter()
    for M in CELLS_M:
        o.forward_rows(p.x[:M], p.words, p.scales, p.biases, shape.bits, shape.G, sel,
                       nthreads=threads)
    dt = time.perf_counter() - t0
    sample_bytes = len(CELLS_M) * sel.size * (shape.weight_bytes / shape.N)
    return {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{sel.size} of {shape.N} output rows of {shape.name}, one pass at each of "
                   f"M={list(CELLS_M)}; fp64 dequantize-then-dot; {dt:.2f} s"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the product shards along N "
              "with no exchange, so there is no multi-GPU measurement to make here", file=sys.stderr)
        sys.exit(2)
    import affine_group_quantized_qmm_amd as qmm

    dev = torch.device("cuda:0")
    shape = W.DENSE_UP
    p, sets, x = make_copies(shape, dev)
    xs = {M: x[:M].contiguous() for M in CELLS_M}
    ys = {M: torch.empty((M, shape.N), dtype=torch.float32, device=dev) for M in CELLS_M}
    stream = torch.cuda.current_stream(dev)
    C = len(sets)

    def call(M, j):
        wq, s, b = sets[j % C]
        qmm.qmm_forward(xs[M], wq, s, b, shape.bits, shape.G, out=ys[M])

    counter = [0]

    def step():
        for M in CELLS_M:
            call(M, counter[0])
            counter[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / args.steps

    # per-cell launch durations (same rotation), for the roofline and the breakdown
    cells = {}
    reps = max(50, 2 * C)
    for M in CELLS_M:
        ms = time_launches(lambda i, M=M: call(M, i), reps, stream)
        algo = shape.weight_bytes + 2 * M * shape.K + 4 * M * shape.N
        cells[f"M{M}"] = {
            "kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G),
            "us_per_call": round(ms * 1e3, 3),
            "weight_GBps": round(shape.weight_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * shape.weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "algorithmic_bytes": algo,
            "rows_outputs_per_s": round(M * shape.N / (ms * 1e-3), 1),
        }
    dominant = max(cells, key=lambda k: cells[k]["us_per_call"])
    dom = cells[dominant]
    achieved = dom["algorithmic_bytes"] / (dom["us_per_call"] * 1e-6) / 1e9

    weight_bytes_per_step = len(CELLS_M) * shape.weight_bytes
    value = weight_bytes_per_step / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "effective weight GB/s (% HBM peak) for W4 g32 qmm at M=1,4,16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes, fp16 x/scale/bias, fp32 accumulate",
        "data": "synthetic (seeded uniform codes, U(0.005,0.02) scales, U(-0.1,0.1) biases, N(0,1) x)",
        "config": {
            "workload": f"{shape.name}, one qmm_forward at each of M={list(CELLS_M)} per step",
            "K": shape.K, "N": shape.N, "bits": shape.bits, "G": shape.G,
            "weight_copies_rotated": C,
            "weight_bytes_per_call": shape.weight_bytes,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "cells": cells,
        "m16_over_m1_time": round(cells["M16"]["us_per_call"] / cells["M1"]["us_per_call"], 3),
        "roofline": {
            "kernel": f"{dom['kernel']} (M={dominant[1:]})",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, shape, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
