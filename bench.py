"""Benchmark: effective weight-stream GB/s of the affine group-quantized
product on one MI355X, for the 27B-style dense MLP up projection
(K = 5120, N = 17408, 4-bit codes, G = 32) at M = 1, 4 and 16 activation rows.

One step = one qmm_forward call at each of M = 1, 4, 16 (three launches),
every call reading its own copy of the packed weights, scales and biases:
the copies rotate over more than 512 MB so that no call is served from the
256 MB Infinity Cache. Inputs are resident in HBM before timing starts. The
timed steps are captured once into a HIP graph (untimed), replayed once
untimed (the first replay uploads the graph), then replayed once timed, so
the host's per-call cost does not leave the GPU idle between launches.

value = weight bytes streamed per step / step time, where weight bytes per
call = N*K*(bits/8 + 4/G) (codes plus fp16 scale and bias per group).

Prints one JSON line. Synthetic data (seeded; no trained weights). Besides
the headline the line carries:
  cells           per-M launch times of the headline cells, three trials in
                  alternating order (forward, reverse, forward; median used);
  parity          the headline GPU outputs against the fp64 oracle on every
                  one of the 17408 output rows (max error / bound per M);
  tiny            the 512 x 512 projection at M = 1: latency of one call and
                  time per call back to back, with full oracle parity;
  read_ceiling    the streaming-read kernel over the headline call's weight
                  bytes (the most a one-row product can reach);
  layer           one decoder layer of the sweep at M = 1 and 8, projections
                  one by one and with q/k/v and gate/up fused;
  layer_sweep     64 decoder layers (13.63 GB of 4-bit weights resident in
                  HBM) at M = 1 and 8, with every output column of layer 0
                  checked against the oracle;
  long_k          the 17408 x 5120 down projection at M = 16 through
                  qmm_forward_splitk, S = 1, 2, 4, 8;
  other_workloads the headline projection at M = 2 and 8, with 2- and 3-bit
                  codes, and the mixed 5/6/8-bit G = 64 projections;
  tiled_layout    the headline cells from the tiled layout;
  bf16            the headline cells with bfloat16 x, scales and biases;
  machine         GPU clocks, temperatures and power before and after;
  cpu_baseline    the fp64 oracle on the host cores.

The roofline object covers the kernel that takes most of a step. Its
`traffic` (HBM bytes per launch) comes from the rocprofv3 FETCH_SIZE and
WRITE_SIZE summary committed under profiles/, scaled by the counts the same
counters give for a plain elementwise copy of known size, and is reported
only while the kernel's sources still match the fingerprint recorded with
the counters. Helper modes (used with rocprofv3, see profiles/):
  --profile-run SET --manifest F   a few eager launches of every cell of SET
                            (headline, ab, mixed, longk, layer, read, tiny or
                            all) plus the copy calibration, no timing; F gets
                            the label of every library dispatch in order;
  --summarize-pmc F W DIR --manifest M   counter CSV directories (FETCH_SIZE
                            run, then WRITE_SIZE run) -> one text summary per
                            set under DIR;
  --summarize-dispatches T DIR --manifest M   kernel-trace CSV directory of a
                            profile run -> per-label durations, one summary
                            per set under DIR;
  --summarize-counters D1 .. Dn DIR --manifest M   any counters of profile
                            runs (e.g. the SQ instruction and cycle counts)
                            -> one summary per set under DIR;
  --summarize-trace D OUT   kernel-trace stats directory of a bench run ->
                            text summary OUT.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import subprocess
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
TRIALS = 3  # timing trials per cell, in alternating order
CSRC = ROOT / "affine_group_quantized_qmm_amd" / "csrc"
# sources that determine each kernel's memory traffic
_COMMON = ["qmm_device.hpp", "qmm_kernels.hpp"]
KERNEL_SOURCES = {
    "mfma": ["qmm_mfma_xr.hip", *_COMMON],
    "mfma_lds": ["qmm_mfma.hip", *_COMMON],
    "qmv": ["qmm_qmv.hip", *_COMMON],
    "reduce": ["qmm_pack.hip", *_COMMON],
    "read": ["qmm_stream.hip", *_COMMON],
}
# rocprofv3 kernel-name fragments of the library's kernels
KERNEL_SYMBOLS = {"mfma": "mfma_xr_kernel", "mfma_lds": "mfma_kernel<", "qmv": "qmv_kernel",
                  "reduce": "splitk_reduce_kernel", "read": "stream_read_kernel"}
ZERO_SYMBOL = "zero_kernel"  # clears y for the long-K launches
PROFILES = ROOT / "profiles"
PMC_SUMMARY = PROFILES / "dense_up_w4g32_hbm_traffic.txt"
COPY_ELEMS = 64 * 2 ** 20  # fp32 elements of the calibration copy (256 MiB read, 256 MiB written)
PROFILE_REPS = 4           # rounds of every cell in a profile run (the first runs on cold caches)
PROFILE_SETS = ("headline", "ab", "mixed", "longk", "layer", "read", "tiny")
# summary file stem of each profile set (named for its workload)
SET_FILES = {
    "headline": "dense_up_w4g32",
    "ab": "dense_up_w4g32_valu_vs_mfma_M2-8",
    "mixed": "mixed_5120x5120_w5-6-8g64",
    "longk": "long_k_17408x5120_w4g32_M16",
    "layer": "sweep_layer0_w4g32",
    "read": "stream_read_55.7MB",
    "tiny": "tiny_512x512_w4g32",
}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer, sweep, long-K and other-workload cells")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="output rows of the CPU oracle sample (0: all rows)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="about this much oracle work for the CPU baseline")
    ap.add_argument("--profile-run", choices=(*PROFILE_SETS, "all"))
    ap.add_argument("--manifest", help="profile manifest (JSON) written by --profile-run")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_DIR"))
    ap.add_argument("--summarize-dispatches", nargs=2, metavar=("TRACE_DIR", "OUT_DIR"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="counter CSV directories of profile runs, then the output directory")
    return ap.parse_args(argv)


def fingerprint(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        h.update((CSRC / name).read_bytes())
    return h.hexdigest()[:16]


def kernel_short(name: str) -> str | None:
    return next((k for k, sym in KERNEL_SYMBOLS.items() if sym in name), None)


def _repo_relative(path) -> str:
    """`path` relative to the repository root when it lies inside it."""
    p = Path(path).resolve()
    try:
        return str(p.relative_to(ROOT))
    except ValueError:
        return str(path)


# ---------------------------------------------------------------------------
# rocprofv3 output -> summaries
# ---------------------------------------------------------------------------

def _csv_rows(directory: str, suffix: str):
    files = sorted(Path(directory).rglob(f"*{suffix}"))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(directory: str, counter: str):
    """[(dispatch id, kernel name, counter value summed over instances)] in dispatch order."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            k = acc.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
            k[1] += float(r["Counter_Value"])
    return [(d, acc[d][0], acc[d][1]) for d in sorted(acc)]


def _split_library(seq, manifest):
    """Library dispatches matched to the manifest's labels, and the copy
    calibration (the last PROFILE_REPS non-library dispatches; the first of
    them, on cold caches, is dropped). The fill that clears y ahead of a
    long-K launch (its two K halves add into y) is counted with that launch."""
    ours, pending = [], 0
    for _, n, v in seq:
        if "qmm::" not in n:
            continue
        if ZERO_SYMBOL in n:
            pending += v
            continue
        ours.append((n, v + pending))
        pending = 0
    other = [(n, v) for _, n, v in seq if "qmm::" not in n]
    labels = manifest["dispatches"]
    if len(ours) != len(labels):
        raise SystemExit(f"{len(ours)} library dispatches but {len(labels)} manifest labels")
    return list(zip(labels, ours)), other[-PROFILE_REPS + 1:]


def _group(pairs):
    """{(set, label): {"kernel": name, "values": [...], "algo": bytes}} over warm rounds."""
    cells = {}
    for lab, (name, v) in pairs:
        if lab["round"] == 0:  # cold caches
            continue
        c = cells.setdefault((lab["set"], lab["label"]), {"kernel": name, "values": [],
                                                          "algo": lab["algorithmic_bytes"]})
        c["values"].append(v)
    return cells


def summarize_pmc(fetch_dir: str, write_dir: str, out_dir: str, manifest_path: str):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of a profile run -> one
    text summary per profile set under out_dir."""
    manifest = json.loads(Path(manifest_path).read_text())
    f_pairs, f_copy = _split_library(_per_dispatch(fetch_dir, "FETCH_SIZE"), manifest)
    w_pairs, w_copy = _split_library(_per_dispatch(write_dir, "WRITE_SIZE"), manifest)
    copy_bytes = 4 * COPY_ELEMS
    f_copy_kib = sum(v for _, v in f_copy) / len(f_copy)
    w_copy_kib = sum(v for _, v in w_copy) / len(w_copy)
    f_scale = copy_bytes / (f_copy_kib * 1024)
    w_scale = copy_bytes / (w_copy_kib * 1024)
    fetch, write = _group(f_pairs), _group(w_pairs)
    written = []
    for set_name in manifest["sets"]:
        stem = SET_FILES[set_name]
        out = Path(out_dir) / f"{stem}_hbm_traffic.txt"
        lines = [
            f"# HBM traffic per dispatch, profile set '{set_name}' ({manifest['workloads'][set_name]}),"
            " rocprofv3 counters",
            "# commands (from the repository root on the GPU host):",
            f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o run -- python3 bench.py "
            f"--profile-run {manifest['run']} --manifest <MAN>",
            f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o run -- python3 bench.py "
            f"--profile-run {manifest['run']} --manifest <MAN>",
            f"#   python3 bench.py --summarize-pmc <F> <W> {_repo_relative(out_dir)} --manifest <MAN>",
            "# hbm_bytes = fetch_kib*1024*fetch_scale + write_kib*1024*write_scale (copy calibration);"
            " ratio = hbm_bytes / algorithmic_bytes",
            f"copy_calibration bytes={copy_bytes} fetch_kib={f_copy_kib:.1f} write_kib={w_copy_kib:.1f} "
            f"fetch_scale={f_scale:.4f} write_scale={w_scale:.4f}",
        ]
        for (s, label), c in fetch.items():
            if s != set_name:
                continue
            wc = write[(s, label)]
            fk = sum(c["values"]) / len(c["values"])
            wk = sum(wc["values"]) / len(wc["values"])
            hbm = fk * 1024 * f_scale + wk * 1024 * w_scale
            kind = kernel_short(c["kernel"]) or "other"
            fp = fingerprint(kind) if kind in KERNEL_SOURCES else "-"
            ratio = hbm / c["algo"] if c["algo"] else float("nan")
            lines.append(f"cell set={set_name} label={label} kernel={kind} fingerprint={fp} "
                         f"fetch_kib={fk:.1f} write_kib={wk:.1f} hbm_bytes={hbm:.0f} "
                         f"algorithmic_bytes={c['algo']} ratio={ratio:.4f} dispatches={len(c['values'])}")
        out.write_text("\n".join(lines) + "\n")
        written.append(out)
        print("\n".join(lines))
    return written


def read_traffic(kernel: str, Ms):
    """Average HBM bytes per launch of `kernel` over headline cells Ms, or None
    (no summary, or the kernel changed since the counters were taken)."""
    if not PMC_SUMMARY.exists():
        return None
    got = {}
    for line in PMC_SUMMARY.read_text().splitlines():
        if not line.startswith("cell "):
            continue
        kv = dict(t.split("=", 1) for t in line.split()[1:])
        if kv.get("set") == "headline" and kv["kernel"] == kernel and kv["fingerprint"] == fingerprint(kernel):
            got[int(kv["label"].lstrip("M"))] = float(kv["hbm_bytes"])
    if any(M not in got for M in Ms):
        return None
    return sum(got[M] for M in Ms) / len(Ms)


def _trace_dispatches(trace_dir: str):
    """[(dispatch id, kernel name, duration ns)] of a kernel-trace CSV, in dispatch order."""
    out = []
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        out.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out.sort()
    return out


def summarize_dispatches(trace_dir: str, out_dir: str, manifest_path: str):
    """Kernel trace of a profile run -> average duration per label, one summary
    per profile set, with the achieved rate on its algorithmic bytes."""
    manifest = json.loads(Path(manifest_path).read_text())
    pairs, _ = _split_library(_trace_dispatches(trace_dir), manifest)
    cells = _group(pairs)
    written = []
    for set_name in manifest["sets"]:
        out = Path(out_dir) / f"{SET_FILES[set_name]}_dispatch_trace.txt"
        lines = [
            f"# rocprofv3 kernel trace, profile set '{set_name}' ({manifest['workloads'][set_name]});"
            " eager launches, warm rounds only",
            "# commands (from the repository root on the GPU host):",
            f"#   rocprofv3 --kernel-trace --output-format csv -d <T> -o run -- python3 bench.py "
            f"--profile-run {manifest['run']} --manifest <MAN>",
            f"#   python3 bench.py --summarize-dispatches <T> {_repo_relative(out_dir)} --manifest <MAN>",
            "# label | kernel | dispatches | average_us | min_us | max_us | algorithmic_bytes | GB/s | % of 8 TB/s",
        ]
        for (s, label), c in cells.items():
            if s != set_name:
                continue
            us = [v / 1e3 for v in c["values"]]
            avg = sum(us) / len(us)
            rate = c["algo"] / (avg * 1e-6) / 1e9 if c["algo"] else float("nan")
            kind = kernel_short(c["kernel"]) or "other"
            lines.append(f"{label} | {kind}: {c['kernel'][:110]} | {len(us)} | {avg:.3f} | {min(us):.3f} | "
                         f"{max(us):.3f} | {c['algo']} | {rate:.1f} | {100 * rate / HBM_PEAK_GBPS:.2f}")
        out.write_text("\n".join(lines) + "\n")
        written.append(out)
        print("\n".join(lines))
    return written


def summarize_counters(dirs, out_dir: str, manifest_path: str):
    """Any rocprofv3 counters of profile runs (one or more counter CSV
    directories, each a run of the same manifest) -> per-label averages, one
    summary per profile set under out_dir ("<stem>_sq_counters.txt")."""
    manifest = json.loads(Path(manifest_path).read_text())
    table = {}  # (set, label) -> {"kernel": name, counter: [values]}
    names = []
    for d in dirs:
        rows = _csv_rows(d, "counter_collection.csv")
        counters = sorted({r["Counter_Name"] for r in rows})
        for c in counters:
            if c not in names:
                names.append(c)
            pairs, _ = _split_library(_per_dispatch(d, c), manifest)
            for lab, (kname, v) in pairs:
                if lab["round"] == 0:  # cold caches
                    continue
                e = table.setdefault((lab["set"], lab["label"]), {"kernel": kname})
                e.setdefault(c, []).append(v)
    written = []
    for set_name in manifest["sets"]:
        out = Path(out_dir) / f"{SET_FILES[set_name]}_sq_counters.txt"
        lines = [
            f"# rocprofv3 SQ counters per dispatch (averages over warm rounds), profile set '{set_name}' "
            f"({manifest['workloads'][set_name]})",
            "# commands (from the repository root on the GPU host), one run per counter group:",
            f"#   rocprofv3 --pmc <counters> --output-format csv -d <D_i> -o run -- python3 bench.py "
            f"--profile-run {manifest['run']} --manifest <MAN>",
            f"#   python3 bench.py --summarize-counters <D_1> ... <D_n> {_repo_relative(out_dir)} --manifest <MAN>",
            "# SQ_INSTS_* count wave instructions; *_CYCLES are summed over the counter instances",
            "label | kernel | " + " | ".join(names),
        ]
        for (s_, label), e in table.items():
            if s_ != set_name:
                continue
            kind = kernel_short(e["kernel"]) or "other"
            vals = [f"{sum(e[c]) / len(e[c]):.0f}" if c in e else "-" for c in names]
            lines.append(f"{label} | {kind} | " + " | ".join(vals))
        out.write_text("\n".join(lines) + "\n")
        written.append(out)
        print("\n".join(lines))
    return written


def summarize_trace(trace_dir: str, out: str):
    """Kernel-trace stats of a bench run -> text summary (library kernels first)."""
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = [
        "# rocprofv3 kernel-trace stats of a bench run (dense-up W4 g32 cells M = 1, 4, 16; the read-ceiling "
        "and tiny cells follow them)",
        "# commands (from the repository root on the GPU host):",
        "#   rocprofv3 --kernel-trace --stats --output-format csv -d <D> -o run -- "
        "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-layer",
        f"#   python3 bench.py --summarize-trace <D> {_repo_relative(out)}",
        "# name | calls | average_us | min_us | max_us | total_percent",
    ]
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    for r in rows:
        name = r["Name"]
        short = kernel_short(name)
        label = f"{short}: {name}" if short else name
        lines.append(f"{label[:140]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                     f"{float(r['Percentage']):.2f}")
    Path(out).write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# host and machine state
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> dict:
    """CPUs this process may run on: its affinity set, capped by a cgroup CPU quota."""
    logical = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = logical
    quota = None
    try:
        q, period = Path("/sys/fs/cgroup/cpu.max").read_text().split()[:2]
        if q != "max":
            quota = max(1, math.ceil(int(q) / int(period)))
    except (OSError, ValueError):
        pass
    usable = min(affinity, quota) if quota else affinity
    return {"logical_cpus": logical, "affinity_cpus": affinity, "cgroup_cpu_limit": quota,
            "usable": usable}


def machine_state() -> dict:
    """GPU clocks, temperatures and power from rocm-smi (a child process)."""
    cmd = ["rocm-smi", "--showtemp", "--showclocks", "--showpower", "--json"]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=60)
        data = json.loads(res.stdout)
    except (OSError, subprocess.SubprocessError, ValueError) as e:
        return {"error": f"{' '.join(cmd)}: {type(e).__name__}"}
    keep = ("temp", "clock", "power", "sclk", "mclk", "fclk", "socclk")
    out = {}
    for card, fields in data.items():
        if isinstance(fields, dict):
            out[card] = {k: v for k, v in fields.items() if any(t in k.lower() for t in keep)}
    return out


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

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


def capture_graph(fn, count):
    """Capture fn(0), ..., fn(count-1) into one HIP graph (untimed)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    torch.cuda.synchronize()
    return g


def timed_cells(cells, stream):
    """cells: [(key, fn, reps)]. Each cell's `reps` calls are captured into a
    graph and replayed once untimed; then TRIALS timed replays of every cell,
    the cell order alternating forward and reverse. Returns {key: [us per
    call, one per trial]}."""
    graphs = []
    for key, fn, reps in cells:
        g = capture_graph(fn, reps)
        g.replay()  # the first replay uploads the graph
        torch.cuda.synchronize()
        graphs.append((key, g, reps))
    res = {key: [] for key, _, _ in cells}
    for t in range(TRIALS):
        for key, g, reps in (graphs if t % 2 == 0 else graphs[::-1]):
            res[key].append(time_launches(lambda i, g=g: g.replay(), 1, stream) / reps * 1e3)
    del graphs
    return res


def log(msg: str):
    """Progress on stderr (the JSON line is the only stdout output)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def median(v):
    return sorted(v)[len(v) // 2]


def rate_fields(nbytes: int, us: float) -> dict:
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 3), "weight_GBps": round(gbps, 1),
            "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}


def rotated(p, dev, weight_bytes: int, dtype: str = "f16"):
    """C device copies of (wq, scales, biases) of problem p, over more than
    ROTATION_BYTES in total, and x."""
    def operand(a):
        if dtype == "bf16":  # uint16 bit patterns
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s, b = operand(p.scales), operand(p.biases)
    copies = max(2, -(-ROTATION_BYTES // weight_bytes))
    sets = [(wq, s, b)] + [(wq.clone(), s.clone(), b.clone()) for _ in range(copies - 1)]
    return sets, operand(p.x)


def parity_ratio(o, y_gpu: np.ndarray, ref: np.ndarray, absum: np.ndarray) -> float:
    """max |y - ref| / bound (bound = 1e-5 * sum|w x| + 1e-6); inf if non-finite."""
    y = np.asarray(y_gpu, dtype=np.float64)
    if not np.isfinite(y).all():
        return float("inf")
    bound = 1e-5 * absum + 1e-6
    return float((np.abs(y - ref) / bound).max())


# ---------------------------------------------------------------------------
# measured cells
# ---------------------------------------------------------------------------

def measure_cells(qmm, shape, Ms, dev, stream, dtype="f16"):
    """Per-M launch times of qmm_forward (qmm_forward_bf16 for dtype "bf16") on
    `shape` (rotated weight copies, graph replay, alternating trials)."""
    p = qmm_inputs.make_problem(seed=5, M=max(Ms), K=shape.K, N=shape.N, bits=shape.bits,
                                G=shape.G, packed_words=True, dtype=dtype)
    sets, x = rotated(p, dev, shape.weight_bytes, dtype)
    C = len(sets)
    fwd = qmm.qmm_forward_bf16 if dtype == "bf16" else qmm.qmm_forward
    out = {"K": shape.K, "N": shape.N, "bits": shape.bits, "G": shape.G,
           "weight_bytes_per_call": shape.weight_bytes, "weight_copies_rotated": C}
    cells = []
    for M in Ms:
        xm = x[:M].contiguous()
        y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)

        def call(i, xm=xm, y=y):
            fwd(xm, *sets[i % C], shape.bits, shape.G, out=y)
        cells.append((M, call, max(50, 2 * C)))
    times = timed_cells(cells, stream)
    for M in Ms:
        out[f"M{M}"] = {"kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G),
                        **rate_fields(shape.weight_bytes, median(times[M])),
                        "trials_us": [round(t, 3) for t in times[M]]}
    return out


def measure_tiled(qmm, shape, Ms, dev, stream):
    """The headline projection read from the tiled (matrix-core) layout:
    qmm_repack_tiled once per weight copy (untimed), qmm_forward_tiled timed."""
    p = qmm_inputs.make_problem(seed=0, M=max(Ms), K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s, b = torch.from_numpy(p.scales).to(dev), torch.from_numpy(p.biases).to(dev)
    copies = max(2, -(-ROTATION_BYTES // shape.weight_bytes))
    first = qmm.qmm_repack_tiled(wq, s, b, shape.bits, shape.G)
    sets = [first] + [(first[0].clone(), first[1].clone()) for _ in range(copies - 1)]
    del wq, s, b
    x = torch.from_numpy(p.x).to(dev)
    out = {"workload": f"{shape.name} from the tiled layout (qmm_forward_tiled)",
           "weight_copies_rotated": copies}
    cells = []
    for M in Ms:
        xm = x[:M].contiguous()
        y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)

        def call(i, xm=xm, y=y):
            tw, tsb = sets[i % copies]
            qmm.qmm_forward_tiled(xm, tw, tsb, shape.N, shape.bits, shape.G, out=y)
        cells.append((M, call, max(50, 2 * copies)))
    times = timed_cells(cells, stream)
    for M in Ms:
        out[f"M{M}"] = {**rate_fields(shape.weight_bytes, median(times[M])),
                        "trials_us": [round(t, 3) for t in times[M]]}
    return out


def measure_tiny(qmm, dev, stream, o):
    """The tiny projection (K = N = 512, 4-bit G = 32, M = 1, seed 0): time per
    call back to back (graph of many calls) and the latency of one call (a
    graph of one call, each replay timed alone), and full oracle parity."""
    shape = W.TINY
    p = qmm_inputs.make_problem(seed=0, M=1, K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s, b, x = (torch.from_numpy(a).to(dev) for a in (p.scales, p.biases, p.x))
    y = torch.empty((1, shape.N), dtype=torch.float32, device=dev)

    def call(_i):
        qmm.qmm_forward(x, wq, s, b, shape.bits, shape.G, out=y)
    back = timed_cells([("b2b", call, 200)], stream)["b2b"]
    g = capture_graph(call, 1)
    g.replay()
    torch.cuda.synchronize()
    single = []
    for _ in range(50):
        single.append(time_launches(lambda i: g.replay(), 1, stream) * 1e3)
        torch.cuda.synchronize()
    del g
    out = {"workload": f"{shape.name}, M = 1, qmm_forward",
           "kernel": qmm.qmm_kernel_name(1, shape.K, shape.N, shape.bits, shape.G),
           "latency_us_one_call": round(median(single), 3),
           "us_per_call_back_to_back": round(median(back), 3),
           "trials_us_back_to_back": [round(t, 3) for t in back]}
    if o is not None:
        ref, absum = o.forward(p.x, p.words, p.scales, p.biases, shape.bits, shape.G)
        out["parity_max_err_over_bound"] = round(parity_ratio(o, y.cpu().numpy(), ref, absum), 4)
    return out


def measure_read_ceiling(qmm, dev, stream, nbytes: int):
    """The streaming-read kernel over `nbytes` (one headline call's weight
    bytes), buffers rotated over more than 512 MB like the product cells."""
    words = nbytes // 4
    copies = max(2, -(-ROTATION_BYTES // nbytes))
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), dtype=torch.int32, device=dev)
            for _ in range(copies)]
    sink = torch.empty(qmm.qmm_stream_read_sink_words(nbytes), dtype=torch.int32, device=dev)

    def call(i):
        qmm.qmm_stream_read(bufs[i % copies], sink)
    times = timed_cells([("read", call, max(50, 2 * copies))], stream)["read"]
    us = median(times)
    gbps = nbytes / (us * 1e-6) / 1e9
    del bufs
    return {"workload": f"qmm_stream_read over {nbytes} bytes (one dense-up call's weight bytes)",
            "bytes": nbytes, "buffers_rotated": copies, "us_per_call": round(us, 3),
            "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "trials_us": [round(t, 3) for t in times]}


def measure_layer(qmm, dev, stream):
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

        def separate(i, xs=xs, ys=ys):
            st = sets[i % copies]
            for n, _, _ in shapes:
                qmm.qmm_forward(xs[n], *st[n], 4, 32, out=ys[n])

        def fused(i, xs=xs, ys=ys):
            st = sets[i % copies]
            qmm.qmm_forward_fused(xs["q"], [st["q"], st["k"], st["v"]], 4, 32,
                                  outs=[ys["q"], ys["k"], ys["v"]])
            qmm.qmm_forward(xs["o"], *st["o"], 4, 32, out=ys["o"])
            qmm.qmm_forward_fused(xs["gate"], [st["gate"], st["up"]], 4, 32,
                                  outs=[ys["gate"], ys["up"]])
            qmm.qmm_forward(xs["down"], *st["down"], 4, 32, out=ys["down"])

        times = timed_cells([("separate", separate, 4 * copies), ("fused", fused, 4 * copies)], stream)
        cell = {}
        for label in ("separate", "fused"):
            us = median(times[label])
            cell[f"{label}_us"] = round(us, 2)
            cell[f"{label}_weight_GBps"] = round(layer_bytes / (us * 1e-6) / 1e9, 1)
            cell[f"{label}_trials_us"] = [round(t, 2) for t in times[label]]
        out[f"M{M}"] = cell
    return out


def measure_long_k(qmm, dev, stream):
    """The long-K down projection (K = 17408, N = 5120, 4-bit G=32) at M = 16
    through qmm_forward_splitk at each split factor (S = 1 is one launch
    without a workspace; S > 1 writes S fp32 partials and sums them in a
    second launch), weight copies rotated as in the headline cells."""
    shape, M = W.LONG_K, W.LONG_K_M
    p = qmm_inputs.make_problem(seed=11, M=M, K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    sets, x = rotated(p, dev, shape.weight_bytes)
    C = len(sets)
    y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)
    out = {"workload": f"{shape.name} at M = {M}, qmm_forward_splitk", "weight_bytes_per_call": shape.weight_bytes,
           "weight_copies_rotated": C}
    cells = []
    for S in W.LONG_K_SPLITS:
        need = qmm.qmm_splitk_workspace_bytes(M, shape.N, S)
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev)

        def call(i, S=S, ws=ws):
            qmm.qmm_forward_splitk(x, *sets[i % C], shape.bits, shape.G, S, workspace=ws, out=y)
        cells.append((S, call, max(50, 2 * C)))
    times = timed_cells(cells, stream)
    for S in W.LONG_K_SPLITS:
        out[f"S{S}"] = {
            "kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G) if S == 1 else "split",
            **rate_fields(shape.weight_bytes, median(times[S])),
            "trials_us": [round(t, 3) for t in times[S]],
            "partial_bytes": 8 * S * M * shape.N if S > 1 else 0,
        }
    return out


def measure_sweep(qmm, dev, stream, o, layers: int = W.SWEEP_LAYERS):
    """The layer-stack sweep: `layers` dense decoder layers (q, k, v, o, gate,
    up, down; 4-bit G=32; 13.63 GB of weights at 64 layers), all resident in
    HBM, every projection once per pass, back to back on one stream at each
    sweep M: 448 launches one per projection, 256 with q/k/v and gate/up
    fused, and 320 with the down projection through split-K (S = 4: a slice
    launch and the in-order reduction). Layers are independent (each
    projection reads its own layer input; no chaining). One pass is captured
    into a HIP graph and replayed.

    Layer 0's weights are drawn by the seeded generator (seed = projection
    index, as W.sweep_shapes gives); every other layer holds its own device
    copy of them (drawing 13.6 GB on the host would take minutes, and the
    values do not change the timing). Each layer input is drawn by the seeded
    generator (W.sweep_x_seed). After each timed mode every output column of
    layer 0 is checked against the oracle (`o`)."""
    base = []
    for layer, j, sh, seed in W.sweep_shapes(1):
        p = qmm_inputs.make_problem(seed=seed, M=1, K=sh.K, N=sh.N, bits=4, G=32, packed_words=True)
        base.append((j, sh, p))
    mats = []
    for layer in range(layers):
        for j, sh, p in base:
            if layer == 0:
                t = (torch.from_numpy(p.words.view(np.int32)).to(dev), torch.from_numpy(p.scales).to(dev),
                     torch.from_numpy(p.biases).to(dev))
            else:
                t = tuple(u.clone() for u in mats[j][3:])
            mats.append((layer, j, sh, *t))
    total = sum(sh.weight_bytes for _, _, sh, _, _, _ in mats)
    names = [n for n, _, _ in W.LAYER_PROJECTIONS]
    out = {"workload": (f"{layers} dense decoder layers (q, k, v, o, gate, up, down; 4-bit G=32), "
                        f"{total / 1e9:.3f} GB of weights resident in HBM, one pass per step"),
           "weight_bytes": total,
           "data": "layer 0 drawn by the seeded generator, other layers device copies of it; "
                   "inputs drawn per layer"}
    key_of = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gu", "up": "gu", "down": "down"}
    in_keys = (("qkv", 5120), ("o", 6144), ("gu", 5120), ("down", 17408))
    for M in W.SWEEP_M:
        xin_host = {}
        xin = {}
        for layer in range(layers):
            for ki, (key, K) in enumerate(in_keys):
                a = qmm_inputs.draw_x(qmm_inputs.rng_for(W.sweep_x_seed(layer, ki, M)), M, K)
                if layer == 0:
                    xin_host[key] = a
                xin[layer, key] = torch.from_numpy(a).to(dev)
        ys = {(layer, j): torch.empty((M, sh.N), dtype=torch.float32, device=dev)
              for layer, j, sh, _, _, _ in mats}
        by = {(layer, names[j]): (wq, s, b) for layer, j, _, wq, s, b in mats}
        refs = {}
        if o is not None:
            for j, sh, p in base:
                refs[j] = o.forward(xin_host[key_of[names[j]]], p.words, p.scales, p.biases, 4, 32,
                                    nthreads=host_cores()["usable"])

        def separate(_i):
            for layer, j, sh, wq, s, b in mats:
                qmm.qmm_forward(xin[layer, key_of[names[j]]], wq, s, b, 4, 32, out=ys[layer, j])

        def fused(_i, splitk=False):
            for layer in range(layers):
                qmm.qmm_forward_fused(xin[layer, "qkv"], [by[layer, "q"], by[layer, "k"], by[layer, "v"]], 4, 32,
                                      outs=[ys[layer, 0], ys[layer, 1], ys[layer, 2]])
                qmm.qmm_forward(xin[layer, "o"], *by[layer, "o"], 4, 32, out=ys[layer, 3])
                qmm.qmm_forward_fused(xin[layer, "gu"], [by[layer, "gate"], by[layer, "up"]], 4, 32,
                                      outs=[ys[layer, 4], ys[layer, 5]])
                if splitk:
                    qmm.qmm_forward_splitk(xin[layer, "down"], *by[layer, "down"], 4, 32, 4, workspace=ws,
                                           out=ys[layer, 6])
                else:
                    qmm.qmm_forward(xin[layer, "down"], *by[layer, "down"], 4, 32, out=ys[layer, 6])

        # the down projection (K = 17408) through split-K, S = 4, as a caller would run it
        ws = torch.empty(qmm.qmm_splitk_workspace_bytes(M, 5120, 4) // 4, dtype=torch.float32, device=dev)
        cell = {}
        for label, fn, launches in (("separate", separate, 7 * layers), ("fused", fused, 4 * layers),
                                    ("fused_splitk_down", lambda i: fused(i, True), 5 * layers)):
            times = timed_cells([(label, fn, 1)], stream)[label]
            ms = median(times) / 1e3
            cell[f"{label}_launches"] = launches
            cell[f"{label}_ms"] = round(ms, 3)
            cell[f"{label}_trials_ms"] = [round(t / 1e3, 3) for t in times]
            cell[f"{label}_weight_GBps"] = round(total / (ms * 1e-3) / 1e9, 1)
            cell[f"{label}_pct_hbm_peak"] = round(100 * total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
            if refs:
                torch.cuda.synchronize()
                cell[f"{label}_layer0_max_err_over_bound"] = round(max(
                    parity_ratio(o, ys[0, j].cpu().numpy(), *refs[j]) for j, _, _ in base), 4)
        out[f"M{M}"] = cell
        del xin, ys
    out["layer0_columns_checked"] = sum(sh.N for _, sh, _ in base) if o is not None else 0
    del mats
    torch.cuda.empty_cache()
    return out


def cpu_baseline(p, shape, rows: int, gpu_y: dict, min_seconds: float):
    """The fp64 oracle on the host cores, on a bounded sample of output rows
    (all of them by default); its first pass is also the parity check of the
    GPU's headline outputs `gpu_y` ({M: [M, N] array})."""
    import oracle
    o = oracle.get()
    cores = host_cores()
    threads = cores["usable"]
    rng = np.random.default_rng(1)
    rows = shape.N if rows <= 0 else min(rows, shape.N)
    sel = np.sort(rng.choice(shape.N, size=rows, replace=False))
    parity = {}
    passes = 0
    t0 = time.perf_counter()
    while True:
        for M in CELLS_M:
            ref, absum = o.forward_rows(p.x[:M], p.words, p.scales, p.biases, shape.bits, shape.G, sel,
                                        nthreads=threads)
            if passes == 0:
                parity[f"M{M}"] = round(parity_ratio(o, gpu_y[M][:, sel], ref, absum), 4)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 1000:
            break
    sample_bytes = passes * len(CELLS_M) * sel.size * (shape.weight_bytes / shape.N)
    base = {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{passes} passes over {sel.size} of {shape.N} output rows of {shape.name}, "
                   f"each pass one call at each of M={list(CELLS_M)}; fp64 dequantize-then-dot; "
                   f"{dt:.1f} s"),
        "cpu_model": cpu_model(),
        **{k: v for k, v in cores.items() if k != "usable"},
    }
    check = {"rows_checked": int(sel.size), "max_err_over_bound": parity,
             "ok": all(v <= 1.0 for v in parity.values())}
    return base, check


# ---------------------------------------------------------------------------
# profile runs: eager launches with a manifest of every library dispatch
# ---------------------------------------------------------------------------

class Manifest:
    def __init__(self, run: str):
        self.run = run
        self.sets, self.workloads, self.dispatches = [], {}, []
        self.round = 0

    def begin(self, set_name: str, workload: str):
        self.sets.append(set_name)
        self.workloads[set_name] = workload

    def add(self, set_name: str, label: str, algorithmic_bytes: int):
        self.dispatches.append({"set": set_name, "label": label, "round": self.round,
                                "algorithmic_bytes": int(algorithmic_bytes)})

    def write(self, path):
        Path(path).parent.mkdir(parents=True, exist_ok=True)
        Path(path).write_text(json.dumps({"run": self.run, "sets": self.sets, "workloads": self.workloads,
                                          "dispatches": self.dispatches}))


def product_bytes(shape, M: int) -> int:
    """Algorithmic bytes of one product launch: weights once, x, fp32 y."""
    return shape.weight_bytes + 2 * M * shape.K + 4 * M * shape.N


def profile_run(qmm, which: str, manifest_path: str, dev):
    man = Manifest(which)
    sets = PROFILE_SETS if which == "all" else (which,)
    for set_name in sets:
        log(f"profile set {set_name}")
        globals()[f"_profile_{set_name}"](qmm, man, dev)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(PROFILE_REPS):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    if manifest_path:
        man.write(manifest_path)
    print(f"profile run {which}: {len(man.dispatches)} library dispatches, {PROFILE_REPS} copies", flush=True)


def _rounds(man, fn):
    for r in range(PROFILE_REPS):
        man.round = r
        fn(r)
    man.round = 0


def _profile_forward_cells(qmm, man, dev, set_name, shape, Ms, kernels=(None,), seed=5):
    p = qmm_inputs.make_problem(seed=seed, M=max(Ms), K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    sets, x = rotated(p, dev, shape.weight_bytes)
    C = len(sets)
    xs = {M: x[:M].contiguous() for M in Ms}
    ys = {M: torch.empty((M, shape.N), dtype=torch.float32, device=dev) for M in Ms}
    prefix = "" if set_name != "mixed" else f"w{shape.bits}."
    n = [0]

    def one_round(_r):
        for kern in kernels:
            for M in Ms:
                w = sets[n[0] % C]
                n[0] += 1
                if kern is None:
                    qmm.qmm_forward(xs[M], *w, shape.bits, shape.G, out=ys[M])
                else:
                    qmm.qmm_forward_kernel(kern, xs[M], *w, shape.bits, shape.G, out=ys[M])
                man.add(set_name, f"{prefix}{kern + '.' if kern else ''}M{M}", product_bytes(shape, M))
    _rounds(man, one_round)


def _profile_headline(qmm, man, dev):
    man.begin("headline", f"{W.DENSE_UP.name}, qmm_forward at M={list(CELLS_M)}")
    _profile_forward_cells(qmm, man, dev, "headline", W.DENSE_UP, CELLS_M, seed=0)


def _profile_ab(qmm, man, dev):
    man.begin("ab", f"{W.DENSE_UP.name}, the VALU kernel (qmv) against the register-resident "
                    "matrix-core kernel (mfma) at M = 2..8, both forced")
    _profile_forward_cells(qmm, man, dev, "ab", W.DENSE_UP, tuple(range(2, 9)), kernels=("qmv", "mfma"))


def _profile_mixed(qmm, man, dev):
    man.begin("mixed", "mixed 5/6/8-bit G=64 projections, 5120 x 5120, qmm_forward at M = 1, 8, 16")
    for sh in W.MIXED:
        _profile_forward_cells(qmm, man, dev, "mixed", sh, W.MIXED_M)


def _profile_longk(qmm, man, dev):
    shape, M = W.LONG_K, W.LONG_K_M
    man.begin("longk", f"{shape.name} at M = {M}, qmm_forward_splitk at S = {list(W.LONG_K_SPLITS)}")
    p = qmm_inputs.make_problem(seed=11, M=M, K=shape.K, N=shape.N, bits=shape.bits, G=shape.G,
                                packed_words=True)
    sets, x = rotated(p, dev, shape.weight_bytes)
    C = len(sets)
    y = torch.empty((M, shape.N), dtype=torch.float32, device=dev)
    n = [0]

    def one_round(_r):
        for S in W.LONG_K_SPLITS:
            ws = torch.empty(max(qmm.qmm_splitk_workspace_bytes(M, shape.N, S) // 4, 1), dtype=torch.float32,
                             device=dev)
            qmm.qmm_forward_splitk(x, *sets[n[0] % C], shape.bits, shape.G, S, workspace=ws, out=y)
            n[0] += 1
            if S == 1:
                man.add("longk", "S1", product_bytes(shape, M))
            else:
                part = 4 * S * M * shape.N
                man.add("longk", f"S{S}.slices", shape.weight_bytes + 2 * M * shape.K + part)
                man.add("longk", f"S{S}.reduce", part + 4 * M * shape.N)
    _rounds(man, one_round)


def _profile_layer(qmm, man, dev):
    man.begin("layer", "layer 0 of the sweep (q, k, v, o, gate, up, down; 4-bit G=32) at M = 1 and 8: "
                       "one launch per projection, q/k/v and gate/up fused, down through split-K S = 4")
    shapes = {name: W.Shape(f"L0.{name}", K=K, N=N, bits=4, G=32) for name, K, N in W.LAYER_PROJECTIONS}
    layer_bytes = sum(sh.weight_bytes for sh in shapes.values())
    base = {}
    for j, (name, sh) in enumerate(shapes.items()):
        pr = qmm_inputs.make_problem(seed=j, M=max(W.SWEEP_M), K=sh.K, N=sh.N, bits=4, G=32, packed_words=True)
        base[name] = (torch.from_numpy(pr.words.view(np.int32)).to(dev), torch.from_numpy(pr.scales).to(dev),
                      torch.from_numpy(pr.biases).to(dev), torch.from_numpy(pr.x).to(dev))
    copies = max(2, -(-ROTATION_BYTES // layer_bytes))
    sets = [{n: t[:3] for n, t in base.items()}]
    sets += [{n: tuple(u.clone() for u in t[:3]) for n, t in base.items()} for _ in range(copies - 1)]
    n = [0]

    def one_round(_r):
        for M in W.SWEEP_M:
            xs = {k: t[3][:M].contiguous() for k, t in base.items()}
            ys = {k: torch.empty((M, sh.N), dtype=torch.float32, device=dev) for k, sh in shapes.items()}
            st = sets[n[0] % copies]
            n[0] += 1
            for k, sh in shapes.items():
                qmm.qmm_forward(xs[k], *st[k], 4, 32, out=ys[k])
                man.add("layer", f"{k}.M{M}", product_bytes(sh, M))
            qmm.qmm_forward_fused(xs["q"], [st["q"], st["k"], st["v"]], 4, 32, outs=[ys["q"], ys["k"], ys["v"]])
            man.add("layer", f"qkv_fused.M{M}", sum(product_bytes(shapes[k], M) for k in "qkv")
                    - 2 * 2 * M * 5120)
            qmm.qmm_forward_fused(xs["gate"], [st["gate"], st["up"]], 4, 32, outs=[ys["gate"], ys["up"]])
            man.add("layer", f"gate_up_fused.M{M}", product_bytes(shapes["gate"], M) +
                    product_bytes(shapes["up"], M) - 2 * M * 5120)
            sh = shapes["down"]
            ws = torch.empty(qmm.qmm_splitk_workspace_bytes(M, sh.N, 4) // 4, dtype=torch.float32, device=dev)
            qmm.qmm_forward_splitk(xs["down"], *st["down"], 4, 32, 4, workspace=ws, out=ys["down"])
            part = 4 * 4 * M * sh.N
            man.add("layer", f"down_splitk4.slices.M{M}", sh.weight_bytes + 2 * M * sh.K + part)
            man.add("layer", f"down_splitk4.reduce.M{M}", part + 4 * M * sh.N)
    _rounds(man, one_round)


def _profile_read(qmm, man, dev):
    nbytes = W.DENSE_UP.weight_bytes
    man.begin("read", f"qmm_stream_read over {nbytes} bytes (one dense-up call's weight bytes)")
    copies = max(2, -(-ROTATION_BYTES // nbytes))
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
            for _ in range(copies)]
    sink = torch.empty(qmm.qmm_stream_read_sink_words(nbytes), dtype=torch.int32, device=dev)

    def one_round(r):
        qmm.qmm_stream_read(bufs[r % copies], sink)
        man.add("read", "read", nbytes + 4 * sink.numel())
    _rounds(man, one_round)


def _profile_tiny(qmm, man, dev):
    shape = W.TINY
    man.begin("tiny", f"{shape.name}, qmm_forward at M = 1")
    p = qmm_inputs.make_problem(seed=0, M=1, K=shape.K, N=shape.N, bits=shape.bits, G=shape.G, packed_words=True)
    wq = torch.from_numpy(p.words.view(np.int32)).to(dev)
    s, b, x = (torch.from_numpy(a).to(dev) for a in (p.scales, p.biases, p.x))
    y = torch.empty((1, shape.N), dtype=torch.float32, device=dev)

    def one_round(_r):
        qmm.qmm_forward(x, wq, s, b, shape.bits, shape.G, out=y)
        man.add("tiny", "M1", product_bytes(shape, 1))
    _rounds(man, one_round)


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main(argv=None):
    args = parse(argv)
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.manifest)
        return
    if args.summarize_dispatches:
        summarize_dispatches(*args.summarize_dispatches, args.manifest)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[:-1], args.summarize_counters[-1], args.manifest)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the product shards along N "
              "with no exchange, so there is no multi-GPU measurement to make here", file=sys.stderr)
        sys.exit(2)
    state_before = None if args.profile_run else machine_state()
    import affine_group_quantized_qmm_amd as qmm

    dev = torch.device("cuda:0")
    if args.profile_run:
        profile_run(qmm, args.profile_run, args.manifest, dev)
        return

    shape = W.DENSE_UP
    p = qmm_inputs.make_problem(seed=0, M=max(CELLS_M), K=shape.K, N=shape.N, bits=shape.bits,
                                G=shape.G, packed_words=True)
    sets, x = rotated(p, dev, shape.weight_bytes)
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

    # The launches are replayed from HIP graphs: a Python call of the binding
    # costs about as much host time as a one-row product takes on the GPU, so
    # eager launches would measure the host. Capture is untimed, and so is the
    # first replay (it uploads the graph).
    step_graph = capture_graph(lambda i: step(), args.steps)
    step_graph.replay()
    torch.cuda.synchronize()

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
    gpu_y = {M: ys[M].cpu().numpy() for M in CELLS_M}

    # per-cell launch durations (same rotation, graph replay, alternating
    # trials), for the roofline and the breakdown
    reps = max(50, 2 * C)
    times = timed_cells([(M, lambda i, M=M: call(M, i), reps) for M in CELLS_M], stream)
    cells = {}
    for M in CELLS_M:
        us = median(times[M])
        cells[f"M{M}"] = {
            "kernel": qmm.qmm_kernel_name(M, shape.K, shape.N, shape.bits, shape.G),
            **rate_fields(shape.weight_bytes, us),
            "trials_us": [round(t, 3) for t in times[M]],
            "algorithmic_bytes": product_bytes(shape, M),
            "rows_outputs_per_s": round(M * shape.N / (us * 1e-6), 1),
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
    del sets, x, xs, ys
    torch.cuda.empty_cache()
    o = None
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.get()
    log(f"headline done: {ms_per_step * 1e3:.2f} us per step")
    out["read_ceiling"] = measure_read_ceiling(qmm, dev, stream, shape.weight_bytes)
    out["read_ceiling"]["M1_frac_of_ceiling"] = round(out["read_ceiling"]["us_per_call"] /
                                                      cells["M1"]["us_per_call"], 4)
    log("read ceiling done")
    out["tiny"] = measure_tiny(qmm, dev, stream, o)
    log("tiny done")
    if not args.no_layer:
        out["layer"] = measure_layer(qmm, dev, stream)
        log("layer done")
        out["layer_sweep"] = measure_sweep(qmm, dev, stream, o)
        log("layer sweep done")
        out["long_k"] = measure_long_k(qmm, dev, stream)
        log("long K done")
        extra = ((W.DENSE_UP, tuple(m for m in W.DENSE_UP_M if m not in CELLS_M)),
                 (W.Shape("dense_up_5120x17408_w2g32", K=5120, N=17408, bits=2, G=32), (1, 16)),
                 (W.Shape("dense_up_5120x17408_w3g32", K=5120, N=17408, bits=3, G=32), (1, 16)),
                 *((sh, W.MIXED_M) for sh in W.MIXED))
        out["other_workloads"] = {sh.name: measure_cells(qmm, sh, Ms, dev, stream) for sh, Ms in extra}
        log("other workloads done")
        out["tiled_layout"] = measure_tiled(qmm, shape, CELLS_M, dev, stream)
        out["bf16"] = {"workload": f"{shape.name} with bfloat16 x, scales and biases (qmm_forward_bf16)",
                       **measure_cells(qmm, shape, CELLS_M, dev, stream, dtype="bf16")}
    out["machine"] = {"before": state_before, "after": machine_state()}
    if not args.no_cpu_baseline:
        log("CPU baseline and full-row parity")
        out["cpu_baseline"], out["parity"] = cpu_baseline(p, shape, args.cpu_rows, gpu_y, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
