"""Benchmark: effective weight-stream GB/s of the affine group-quantized
product on one MI355X, for the 27B-style dense MLP up projection
(K = 5120, N = 17408, 4-bit codes, G = 32) at M = 1, 4 and 16 activation rows.

One step = one qmm_forward call at each of M = 1, 4, 16 (three launches),
every call reading its own copy of the packed weights, scales and biases:
the copies rotate over more than 512 MB so that no call is served from the
256 MB Infinity Cache. Inputs are resident in HBM before timing starts. The
timed steps are captured once into a HIP graph (untimed) and replayed, so the
host's per-call cost does not leave the GPU idle between launches.

value = weight bytes streamed per step / step time, where weight bytes per
call = N*K*(bits/8 + 4/G) (codes plus fp16 scale and bias per group).

Prints one JSON line. Synthetic data (seeded; no trained weights). Besides
the headline cells the line carries `layer_sweep`: the 64-layer sweep
(13.63 GB of 4-bit weights resident in HBM, 448 projections per pass) at
M = 1 and 8, one launch per projection and fused; `long_k`: the 17408 x 5120
down projection at M = 16 through qmm_forward_splitk, S = 1, 2, 4, 8;
`layer`: one decoder layer
of the layer sweep at M = 1 and 8, its seven projections launched one by one and with
q/k/v and gate/up fused (qmm_forward_fused); `other_workloads`: the
dense up projection with 2- and 3-bit codes and the mixed 5/6/8-bit G=64
projections, timed like the headline cells; and `tiled_layout`: the
headline cells read from the tiled layout (qmm_forward_tiled); and `bf16`:
the headline cells with bfloat16 x, scales and biases (qmm_forward_bf16).

The roofline object covers the kernel that takes most of a step. Its
`traffic` (HBM bytes per launch) comes from the rocprofv3 FETCH_SIZE and
WRITE_SIZE summary committed under profiles/, scaled by the counts the same
counters give for a plain elementwise copy of known size, and is reported
only while the kernel's sources still match the fingerprint recorded with
the counters. Helper modes (used with rocprofv3, see profiles/):
  --profile-run             a few launches of every cell plus the copy
                            calibration, no timing;
  --summarize-pmc F W OUT   counters CSV directories (FETCH_SIZE run, then
                            WRITE_SIZE run) -> text summary OUT;
  --summarize-trace D OUT   kernel-trace stats directory -> text summary OUT.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
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
CSRC = ROOT / "affine_group_quantized_qmm_amd" / "csrc"
# sources that determine each kernel's memory traffic
KERNEL_SOURCES = {
    "mfma": ["qmm_mfma_xr.hip", "qmm_device.hpp", "qmm_kernels.hpp"],
    "mfma_lds": ["qmm_mfma.hip", "qmm_device.hpp", "qmm_kernels.hpp"],
    "qmv": ["qmm_qmv.hip", "qmm_device.hpp", "qmm_kernels.hpp"],
}
# rocprofv3 kernel-name fragments of the library's kernels
KERNEL_SYMBOLS = {"mfma": "mfma_xr_kernel", "mfma_lds": "mfma_kernel<", "qmv": "qmv_kernel"}
PMC_SUMMARY = ROOT / "profiles" / "dense_up_w4g32_hbm_traffic.txt"
COPY_ELEMS = 64 * 2 ** 20  # fp32 elements of the calibration copy (256 MiB read, 256 MiB written)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the decoder-layer cell and the other workloads")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="output rows of the CPU oracle sample (0: all rows)")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"))
    return ap.parse_args()


def fingerprint(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        h.update((CSRC / name).read_bytes())
    return h.hexdigest()[:16]


def _counter_rows(directory: str):
    """(dispatch index, kernel name, counter, value) from a rocprofv3 counter CSV."""
    files = sorted(Path(directory).rglob("*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                             float(r["Counter_Value"])))
    return rows


def _per_dispatch(rows, counter):
    """Counter value per dispatch (summed over instances), in dispatch order."""
    acc = {}
    for d, name, c, v in rows:
        if c == counter:
            k = acc.setdefault(d, [name, 0.0])
            k[1] += v
    return [(d, acc[d][0], acc[d][1]) for d in sorted(acc)]


def _repo_relative(path: str) -> str:
    """`path` relative to the repository root when it lies inside it."""
    p = Path(path).resolve()
    try:
        return str(p.relative_to(ROOT))
    except ValueError:
        return str(path)


def summarize_pmc(fetch_dir: str, write_dir: str, out: str):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the profile run -> text summary."""
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    # the profile run launches, in order: PROFILE_REPS rounds of the three cells, then
    # PROFILE_REPS calibration copies
    def classify(seq):
        ours = [(n, v) for _, n, v in seq if "qmm::" in n]
        other = [(n, v) for _, n, v in seq if "qmm::" not in n]
        return ours, other
    f_ours, f_copy = classify(fetch)
    w_ours, w_copy = classify(write)
    # the calibration copies are the last PROFILE_REPS non-library dispatches (earlier
    # ones are the uploads of the inputs); the first of them runs on cold caches
    f_copy, w_copy = f_copy[-PROFILE_REPS + 1:], w_copy[-PROFILE_REPS + 1:]
    copy_bytes = 4 * COPY_ELEMS
    f_copy_kib = sum(v for _, v in f_copy) / len(f_copy)
    w_copy_kib = sum(v for _, v in w_copy) / len(w_copy)
    f_scale = copy_bytes / (f_copy_kib * 1024)
    w_scale = copy_bytes / (w_copy_kib * 1024)
    cells = {}
    for idx, ((fn, fv), (wn, wv)) in enumerate(zip(f_ours, w_ours)):
        M = CELLS_M[idx % len(CELLS_M)]
        kind = next(k for k, sym in KERNEL_SYMBOLS.items() if sym in fn)
        if idx < len(CELLS_M):  # first round: cold caches, not used
            continue
        c = cells.setdefault(M, {"kernel": kind, "fetch": [], "write": []})
        c["fetch"].append(fv)
        c["write"].append(wv)
    lines = [
        "# HBM traffic of the dense-up W4 g32 cells (K=5120, N=17408), rocprofv3 counters",
        "# commands (from the repository root on the GPU host):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o run -- python3 bench.py --profile-run",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o run -- python3 bench.py --profile-run",
        f"#   python3 bench.py --summarize-pmc <F> <W> {_repo_relative(out)}",
        f"copy_calibration kernel={f_copy[0][0].split('(')[0][:60].replace(' ', '_')} "
        f"bytes={copy_bytes} fetch_kib={f_copy_kib:.1f} write_kib={w_copy_kib:.1f} "
        f"fetch_scale={f_scale:.4f} write_scale={w_scale:.4f}",
    ]
    for M, c in sorted(cells.items()):
        fk = sum(c["fetch"]) / len(c["fetch"])
        wk = sum(c["write"]) / len(c["write"])
        hbm = fk * 1024 * f_scale + wk * 1024 * w_scale
        lines.append(f"cell M={M} kernel={c['kernel']} fingerprint={fingerprint(c['kernel'])} "
                     f"fetch_kib={fk:.1f} write_kib={wk:.1f} hbm_bytes={hbm:.0f} dispatches={len(c['fetch'])}")
    Path(out).write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(kernel: str, Ms):
    """Average HBM bytes per launch of `kernel` over cells Ms, or None (no summary, or
    the kernel changed since the counters were taken)."""
    if not PMC_SUMMARY.exists():
        return None
    got = {}
    for line in PMC_SUMMARY.read_text().splitlines():
        if not line.startswith("cell "):
            continue
        kv = dict(t.split("=", 1) for t in line.split()[1:])
        if kv["kernel"] == kernel and kv["fingerprint"] == fingerprint(kernel):
            got[int(kv["M"])] = float(kv["hbm_bytes"])
    if any(M not in got for M in Ms):
        return None
    return sum(got[M] for M in Ms) / len(Ms)


def summarize_trace(trace_dir: str, out: str):
    """Kernel-trace stats of a bench run -> text summary (library kernels first)."""
    files = sorted(Path(trace_dir).rglob("*kernel_stats.csv"))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0], newline="")))
    lines = [
        "# rocprofv3 kernel-trace stats of a bench run (dense-up W4 g32, M = 1, 4, 16)",
        "# commands (from the repository root on the GPU host):",
        "#   rocprofv3 --kernel-trace --stats --output-format csv -d <D> -o run -- "
        "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-layer",
        f"#   python3 bench.py --summarize-trace <D> {out}",
        "# name | calls | average_us | min_us | max_us | total_percent",
    ]
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    for r in rows:
        name = r["Name"]
        short = next((k for k, sym in KERNEL_SYMBOLS.items() if sym in name), None)
        label = f"{short}: {name}" if short else name
        lines.append(f"{label[:140]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                     f"{float(r['Percentage']):.2f}")
    Path(out).write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


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


def cpu_baseline(p, shape, rows: int, min_seconds: float = 10.0):
    """The fp64 oracle on the host cores, on a bounded sample of output rows."""
    import oracle
    o = oracle.get()
    threads = oracle.default_threads()
    rng = np.random.default_rng(1)
    rows = shape.N if rows <= 0 else min(rows, shape.N)
    sel = np.sort(rng.choice(shape.N, size=rows, replace=False))
    # whole passes (one call at each M over the sampled rows) until about 10 s of work
    passes = 0
    t0 = time.perf_counter()
    while True:
        for M in CELLS_M:
            o.forward_rows(p.x[:M], p.words, p.scales, p.biases, shape.bits, shape.G, sel,
                           nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 1000:
            break
    sample_bytes = passes * len(CELLS_M) * sel.size * (shape.weight_bytes / shape.N)
    return {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{passes} passes over {sel.size} of {shape.N} output rows of {shape.name}, "
                   f"each pass one call at each of M={list(CELLS_M)}; fp64 dequantize-then-dot; "
                   f"{dt:.1f} s"),
    }


# Other workloads, timed like the headline cells (not part of `value`):
# the dense up projection with 2- and 3-bit codes, and the mixed 5/6/8-bit
# G=64 projections.
# the headline projection at the verify widths outside the headline cells, then other widths
EXTRA_SHAPES = ((W.DENSE_UP, tuple(m for m in W.DENSE_UP_M if m not in CELLS_M)),
                (W.Shape("dense_up_5120x17408_w2g32", K=5120, N=17408, bits=2, G=32), (1, 16)),
                (W.Shape("dense_up_5120x17408_w3g32", K=5120, N=17408, bits=3, G=32), (1, 16)),
                *((sh, W.MIXED_M) for sh in W.MIXED))


def kernel_label(qmm, M, shape, dtype):
    """The kernel qmm_forward (or qmm_forward_bf16) takes for M rows of `shape`."""
    return qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G)


def measure_cells(qmm, shape, Ms, dev, stream, capture, dtype="f16"):
    """Per-M launch times of qmm_forward (qmm_forward_bf16 for dtype "bf16") on
    `shape` (rotated weight copies, graph replay)."""
    p = qmm_inputs.make_problem(seed=5, M=max(Ms), K=shape.K, N=shape.N, bits=shape.bits,
                                G=shape.G, packed_words=True, dtype=dtype)

    def operand(a):
        if dtype == "bf16":  # uint16 bit patterns
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s = operand(p.scales)
    b = operand(p.biases)
    copies = max(2, -(-ROTATION_BYTES // shape.weight_bytes))
    sets = [(wq, s, b)] + [(wq.clone(), s.clone(), b.clone()) for _ in range(copies - 1)]
    x = operand(p.x)
    fwd = qmm.qmm_forward_bf16 if dtype == "bf16" else qmm.qmm_forward
    out = {"K": shape.K, "N": shape.N, "bits": shape.bits, "G": shape.G,
           "weight_bytes_per_call": shape.weight_bytes, "weight_copies_rotated": copies}
    for M in Ms:
        xm = x[:M].contiguous()
        y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)

        def call(i, xm=xm, y=y):
            fwd(xm, *sets[i % copies], shape.bits, shape.G, out=y)

        reps = max(50, 2 * copies)
        g = capture(call, reps)
        g.replay()
        torch.cuda.synchronize()
        ms = time_launches(lambda i, g=g: g.replay(), 1, stream) / reps
        del g
        out[f"M{M}"] = {
            "kernel": kernel_label(qmm, M, shape, dtype),
            "us_per_call": round(ms * 1e3, 3),
            "weight_GBps": round(shape.weight_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * shape.weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        }
    return out


def measure_tiled(qmm, shape, Ms, dev, stream, capture):
    """The headline projection read from the tiled (matrix-core) layout:
    qmm_repack_tiled once per weight copy (untimed), qmm_forward_tiled timed."""
    p = qmm_inputs.make_problem(seed=0, M=max(Ms), K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s = torch.from_numpy(p.scales).to(dev)
    b = torch.from_numpy(p.biases).to(dev)
    copies = max(2, -(-ROTATION_BYTES // shape.weight_bytes))
    first = qmm.qmm_repack_tiled(wq, s, b, shape.bits, shape.G)
    sets = [first] + [(first[0].clone(), first[1].clone()) for _ in range(copies - 1)]
    del wq, s, b
    x = torch.from_numpy(p.x).to(dev)
    out = {"workload": f"{shape.name} from the tiled layout (qmm_forward_tiled)",
           "weight_copies_rotated": copies}
    for M in Ms:
        xm = x[:M].contiguous()
        y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)

        def call(i, xm=xm, y=y):
            tw, tsb = sets[i % copies]
            qmm.qmm_forward_tiled(xm, tw, tsb, shape.N, shape.bits, shape.G, out=y)

        reps = max(50, 2 * copies)
        g = capture(call, reps)
        g.replay()
        torch.cuda.synchronize()
        ms = time_launches(lambda i, g=g: g.replay(), 1, stream) / reps
        del g
        out[f"M{M}"] = {
            "us_per_call": round(ms * 1e3, 3),
            "weight_GBps": round(shape.weight_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * shape.weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        }
    return out


def measure_layer(qmm, dev, stream, capture):
    """One decoder layer of the layer sweep (q, k, v, o, gate, up, down; 4-bit
    G=32) at each sweep M: the seven projections one launch each, and with
    q/k/v and gate/up fused (qmm_forward_fused: four launches). Weight copies
    rotate over more than 512 MB as in the headline cells; graph replay."""
    shapes = [(name, W.Shape(f"L0.{name}", K=K, N=N, bits=4, G=32), j)
              for j, (name, K, N) in enumerate(W.LAYER_PROJECTIONS)]
    layer_bytes = sum(sh.weight_bytes for _, sh, _ in shapes)
    base = {}
    for name, sh, seed in shapes:
        pr = qmm_inputs.make_problem(seed=seed, M=max(W.SWEEP_M), K=sh.K, N=sh.N, bits=4, G=32,
                                     packed_words=True)
        base[name] = (torch.from_numpy(pr.words.view(np.int32)).to(dev),
                      torch.from_numpy(pr.scales).to(dev), torch.from_numpy(pr.biases).to(dev),
                      torch.from_numpy(pr.x).to(dev))
    copies = max(2, -(-ROTATION_BYTES // layer_bytes))
    sets = [{n: t[:3] for n, t in base.items()}]
    sets += [{n: tuple(u.clone() for u in t[:3]) for n, t in base.items()} for _ in range(copies - 1)]
    out = {"workload": (f"one dense decoder layer of the sweep ({', '.join(n for n, _, _ in shapes)}; "
                        f"4-bit G=32), {layer_bytes / 1e6:.2f} MB of weights"),
           "weight_copies_rotated": copies}
    for M in W.SWEEP_M:
        xs = {n: t[3][:M].contiguous() for n, t in base.items()}
        ys = {n: torch.empty((M, sh.N), dtype=torch.float32, device=dev) for n, sh, _ in shapes}

        def separate(i):
            st = sets[i % copies]
            for n, _, _ in shapes:
                qmm.qmm_forward(xs[n], *st[n], 4, 32, out=ys[n])

        def fused(i):
            st = sets[i % copies]
            qmm.qmm_forward_fused(xs["q"], [st["q"], st["k"], st["v"]], 4, 32,
                                  outs=[ys["q"], ys["k"], ys["v"]])
            qmm.qmm_forward(xs["o"], *st["o"], 4, 32, out=ys["o"])
            qmm.qmm_forward_fused(xs["gate"], [st["gate"], st["up"]], 4, 32,
                                  outs=[ys["gate"], ys["up"]])
            qmm.qmm_forward(xs["down"], *st["down"], 4, 32, out=ys["down"])

        cell = {}
        reps = 4 * copies
        for label, fn in (("separate", separate), ("fused", fused)):
            g = capture(fn, reps)
            g.replay()
            torch.cuda.synchronize()
            ms = time_launches(lambda i, g=g: g.replay(), 1, stream) / reps
            del g
            cell[f"{label}_us"] = round(ms * 1e3, 2)
            cell[f"{label}_weight_GBps"] = round(layer_bytes / (ms * 1e-3) / 1e9, 1)
        out[f"M{M}"] = cell
    return out


def measure_long_k(qmm, dev, stream, capture):
    """The long-K down projection (K = 17408, N = 5120, 4-bit G=32) at M = 16
    through qmm_forward_splitk at each split factor (S = 1 is one launch
    without a workspace; S > 1 writes S fp32 partials and sums them in a
    second launch), weight copies rotated as in the headline cells."""
    shape, M = W.LONG_K, W.LONG_K_M
    p = qmm_inputs.make_problem(seed=11, M=M, K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s = torch.from_numpy(p.scales).to(dev)
    b = torch.from_numpy(p.biases).to(dev)
    copies = max(2, -(-ROTATION_BYTES // shape.weight_bytes))
    sets = [(wq, s, b)] + [(wq.clone(), s.clone(), b.clone()) for _ in range(copies - 1)]
    x = torch.from_numpy(p.x).to(dev)
    y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)
    out = {"workload": f"{shape.name} at M = {M}, qmm_forward_splitk", "weight_bytes_per_call": shape.weight_bytes,
           "weight_copies_rotated": copies}
    for S in W.LONG_K_SPLITS:
        need = qmm.qmm_splitk_workspace_bytes(M, shape.N, S)
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)

        def call(i, S=S, ws=ws):
            qmm.qmm_forward_splitk(x, *sets[i % copies], shape.bits, shape.G, S, workspace=ws, out=y)

        reps = max(50, 2 * copies)
        g = capture(call, reps)
        g.replay()
        torch.cuda.synchronize()
        ms = time_launches(lambda i, g=g: g.replay(), 1, stream) / reps
        del g
        out[f"S{S}"] = {
            "kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G) if S == 1 else "split",
            "us_per_call": round(ms * 1e3, 3),
            "weight_GBps": round(shape.weight_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * shape.weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "partial_bytes": 8 * S * M * shape.N if S > 1 else 0,
        }
    return out


def measure_sweep(qmm, dev, stream, capture, layers: int = W.SWEEP_LAYERS):
    """The layer-stack sweep: `layers` dense decoder layers (q, k, v, o, gate,
    up, down; 4-bit G=32; 13.63 GB of weights at 64 layers), all resident in
    HBM, every projection once per pass, back to back on one stream at each
    sweep M: 448 launches one per projection, 256 with q/k/v and gate/up
    fused, and 320 with the down projection through split-K (S = 4: a slice
    launch and the in-order reduction). Layers are independent (each projection reads its own layer
    input; no chaining). One pass is captured into a HIP graph and replayed.

    The weights are drawn on the device with torch's generator (uniform
    words, scales U(0.005, 0.02), biases U(-0.1, 0.1), x N(0, 1); seed
    1000*layer + projection): drawing 13.6 GB on the host would take minutes.
    Parity at these shapes is covered by the one-layer GPU tests."""
    gen = torch.Generator(device=dev)
    mats = []
    for layer, j, sh, seed in W.sweep_shapes(layers):
        gen.manual_seed(seed)
        wq = torch.randint(-2 ** 31, 2 ** 31 - 1, (sh.N, sh.K * sh.bits // 32), dtype=torch.int32,
                           device=dev, generator=gen)
        lo, hi = qmm_inputs.SCALE_RANGE
        s = (torch.rand((sh.N, sh.K // sh.G), device=dev, generator=gen) * (hi - lo) + lo).half()
        lo, hi = qmm_inputs.BIAS_RANGE
        b = (torch.rand((sh.N, sh.K // sh.G), device=dev, generator=gen) * (hi - lo) + lo).half()
        mats.append((layer, j, sh, wq, s, b))
    total = sum(sh.weight_bytes for _, _, sh, _, _, _ in mats)
    names = [n for n, _, _ in W.LAYER_PROJECTIONS]
    out = {"workload": (f"{layers} dense decoder layers (q, k, v, o, gate, up, down; 4-bit G=32), "
                        f"{total / 1e9:.3f} GB of weights resident in HBM, one pass per step"),
           "weight_bytes": total}
    for M in W.SWEEP_M:
        gen.manual_seed(7 + M)
        # one input per layer input: q/k/v and gate/up share theirs (fused launches need it)
        xin = {}
        for layer in range(layers):
            for key, K in (("qkv", 5120), ("o", 6144), ("gu", 5120), ("down", 17408)):
                xin[layer, key] = torch.randn((M, K), device=dev, generator=gen).half()
        key_of = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gu", "up": "gu", "down": "down"}
        ys = {(layer, j): torch.empty((M, sh.N), dtype=torch.float32, device=dev)
              for layer, j, sh, _, _, _ in mats}
        by = {(layer, names[j]): (wq, s, b) for layer, j, _, wq, s, b in mats}

        def separate(_i):
            for layer, j, sh, wq, s, b in mats:
                qmm.qmm_forward(xin[layer, key_of[names[j]]], wq, s, b, 4, 32, out=ys[layer, j])

        def fused(_i):
            for layer in range(layers):
                qmm.qmm_forward_fused(xin[layer, "qkv"], [by[layer, "q"], by[layer, "k"], by[layer, "v"]], 4, 32,
                                      outs=[ys[layer, 0], ys[layer, 1], ys[layer, 2]])
                qmm.qmm_forward(xin[layer, "o"], *by[layer, "o"], 4, 32, out=ys[layer, 3])
                qmm.qmm_forward_fused(xin[layer, "gu"], [by[layer, "gate"], by[layer, "up"]], 4, 32,
                                      outs=[ys[layer, 4], ys[layer, 5]])
                qmm.qmm_forward(xin[layer, "down"], *by[layer, "down"], 4, 32, out=ys[layer, 6])

        # the down projection (K = 17408) through split-K, S = 4, as a caller would run it
        ws = torch.empty(qmm.qmm_splitk_workspace_bytes(M, 5120, 4) // 4, dtype=torch.float32, device=dev)

        def fused_splitk(_i):
            for layer in range(layers):
                qmm.qmm_forward_fused(xin[layer, "qkv"], [by[layer, "q"], by[layer, "k"], by[layer, "v"]], 4, 32,
                                      outs=[ys[layer, 0], ys[layer, 1], ys[layer, 2]])
                qmm.qmm_forward(xin[layer, "o"], *by[layer, "o"], 4, 32, out=ys[layer, 3])
                qmm.qmm_forward_fused(xin[layer, "gu"], [by[layer, "gate"], by[layer, "up"]], 4, 32,
                                      outs=[ys[layer, 4], ys[layer, 5]])
                qmm.qmm_forward_splitk(xin[layer, "down"], *by[layer, "down"], 4, 32, 4, workspace=ws,
                                       out=ys[layer, 6])

        cell = {}
        for label, fn, launches in (("separate", separate, 7 * layers), ("fused", fused, 4 * layers),
                                    ("fused_splitk_down", fused_splitk, 5 * layers)):
            g = capture(fn, 1)
            g.replay()
            torch.cuda.synchronize()
            times = [time_launches(lambda i, g=g: g.replay(), 1, stream) for _ in range(5)]
            ms = sorted(times)[len(times) // 2]
            del g
            cell[f"{label}_launches"] = launches
            cell[f"{label}_ms"] = round(ms, 3)
            cell[f"{label}_weight_GBps"] = round(total / (ms * 1e-3) / 1e9, 1)
            cell[f"{label}_pct_hbm_peak"] = round(100 * total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
        out[f"M{M}"] = cell
        del xin, ys
    del mats
    torch.cuda.empty_cache()
    return out


PROFILE_REPS = 4


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
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

    if args.profile_run:
        for _ in range(PROFILE_REPS):
            step()
        src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(PROFILE_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"profile run: {PROFILE_REPS} rounds of M={list(CELLS_M)}, {PROFILE_REPS} copies", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The launches are replayed from HIP graphs: a Python call of the binding
    # costs about as much host time as a one-row product takes on the GPU, so
    # eager launches would measure the host. Capture is untimed.
    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        torch.cuda.synchronize()
        return g

    step_graph = capture(lambda i: step(), args.steps)

    # timed region: exactly `steps` steps (one replay of the captured steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    step_graph.replay()
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / args.steps
    del step_graph

    # per-cell launch durations (same rotation, graph replay), for the roofline
    # and the breakdown
    cells = {}
    reps = max(50, 2 * C)
    for M in CELLS_M:
        g = capture(lambda i, M=M: call(M, i), reps)
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        ms = time_launches(lambda i, g=g: g.replay(), 1, stream) / reps
        del g
        algo = shape.weight_bytes + 2 * M * shape.K + 4 * M * shape.N
        cells[f"M{M}"] = {
            "kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G),
            "us_per_call": round(ms * 1e3, 3),
            "weight_GBps": round(shape.weight_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * shape.weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "algorithmic_bytes": algo,
            "rows_outputs_per_s": round(M * shape.N / (ms * 1e-3), 1),
        }
    # the kernel with the largest share of a step, over all of its launches
    by_kernel = {}
    for key, c in cells.items():
        by_kernel.setdefault(c["kernel"], []).append(int(key[1:]))
    dominant = max(by_kernel, key=lambda k: sum(cells[f"M{M}"]["us_per_call"] for M in by_kernel[k]))
    dom_Ms = by_kernel[dominant]
    dom_us = sum(cells[f"M{M}"]["us_per_call"] for M in dom_Ms) / len(dom_Ms)
    dom_bytes = sum(cells[f"M{M}"]["algorithmic_bytes"] for M in dom_Ms) / len(dom_Ms)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = read_traffic(dominant, dom_Ms)

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
            "kernel": f"{dominant} (M={','.join(str(M) for M in dom_Ms)}; per-launch averages)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": round(dom_bytes),
            "us_per_launch": round(dom_us, 3),
            "traffic": None if traffic is None else round(traffic),
        },
    }
    if not args.no_layer:
        out["layer"] = measure_layer(qmm, dev, stream, capture)
        out["layer_sweep"] = measure_sweep(qmm, dev, stream, capture)
        out["long_k"] = measure_long_k(qmm, dev, stream, capture)
        out["other_workloads"] = {sh.name: measure_cells(qmm, sh, Ms, dev, stream, capture)
                                  for sh, Ms in EXTRA_SHAPES}
        out["tiled_layout"] = measure_tiled(qmm, shape, CELLS_M, dev, stream, capture)
        out["bf16"] = {"workload": f"{shape.name} with bfloat16 x, scales and biases (qmm_forward_bf16)",
                       **measure_cells(qmm, shape, CELLS_M, dev, stream, capture, dtype="bf16")}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, shape, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
