"""Host logic of the benchmark's profile summaries (no GPU): the HBM traffic
of a launch is its FETCH_SIZE and WRITE_SIZE counts (KiB per dispatch)
scaled by what the same counters read for a copy of known size, and a
summary is only used while the kernel's sources match its fingerprint."""
import csv
import json

import pytest

import bench


def _write_counters(directory, rows):
    directory.mkdir(parents=True)
    with open(directory / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, counter, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def _profile_run(counter, kib_of):
    """Dispatches in the order of bench.py --profile-run headline: uploads,
    PROFILE_REPS rounds of the three cells, then PROFILE_REPS calibration
    copies; and the manifest that run writes."""
    names = {1: "void qmm::(anonymous namespace)::qmv_kernel<4>(x)",
             4: "void qmm::(anonymous namespace)::mfma_xr_kernel<4>(x)",
             16: "void qmm::(anonymous namespace)::mfma_xr_kernel<4>(x)"}
    rows, d, labels = [], 0, []
    for _ in range(3):  # input uploads (not library kernels)
        rows.append((d, "void at::native::upload(x)", counter, 10.0)); d += 1
    for r in range(bench.PROFILE_REPS):
        for M in bench.CELLS_M:
            rows.append((d, names[M], counter, kib_of(M))); d += 1
            labels.append({"set": "headline", "label": f"M{M}", "round": r, "algorithmic_bytes": 1000 * M})
    for _ in range(bench.PROFILE_REPS):
        rows.append((d, "void at::native::vectorized_elementwise_kernel<4>(copy)", counter, kib_of("copy"))); d += 1
    manifest = {"run": "headline", "sets": ["headline"], "workloads": {"headline": "dense up"},
                "dispatches": labels}
    return rows, manifest


def test_traffic_scaled_by_the_copy_calibration(tmp_path, monkeypatch):
    copy_bytes = 4 * bench.COPY_ELEMS
    # FETCH_SIZE reads half the bytes of the copy (scale 2), WRITE_SIZE all (scale 1)
    fetch = {1: 27000.0, 4: 28000.0, 16: 28400.0, "copy": copy_bytes / 2 / 1024}
    write = {1: 68.0, 4: 272.0, 16: 1088.0, "copy": copy_bytes / 1024}
    frows, manifest = _profile_run("FETCH_SIZE", fetch.__getitem__)
    wrows, _ = _profile_run("WRITE_SIZE", write.__getitem__)
    _write_counters(tmp_path / "f", frows)
    _write_counters(tmp_path / "w", wrows)
    man = tmp_path / "manifest.json"
    man.write_text(json.dumps(manifest))
    out_dir = tmp_path / "out"
    out_dir.mkdir()
    written = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out_dir), str(man))
    assert [w.name for w in written] == ["dense_up_w4g32_hbm_traffic.txt"]
    monkeypatch.setattr(bench, "PMC_SUMMARY", written[0])
    for M in bench.CELLS_M:
        want = fetch[M] * 1024 * 2 + write[M] * 1024
        kernel = "qmv" if M == 1 else "mfma"
        assert bench.read_traffic(kernel, [M]) == pytest.approx(want, rel=1e-9)
    assert bench.read_traffic("mfma", [4, 16]) == pytest.approx(
        (fetch[4] + fetch[16]) * 1024 + (write[4] + write[16]) * 512, rel=1e-9)
    # warm rounds only: the cold first round is dropped
    text = written[0].read_text()
    assert f"dispatches={bench.PROFILE_REPS - 1}" in text


def test_manifest_must_match_the_library_dispatches(tmp_path):
    frows, manifest = _profile_run("FETCH_SIZE", lambda k: 1.0)
    manifest["dispatches"] = manifest["dispatches"][:-1]
    _write_counters(tmp_path / "f", frows)
    man = tmp_path / "manifest.json"
    man.write_text(json.dumps(manifest))
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "f"), str(tmp_path), str(man))


def test_traffic_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    summary = tmp_path / "summary.txt"
    summary.write_text(f"cell set=headline label=M1 kernel=qmv fingerprint=0000000000000000 fetch_kib=1 "
                       f"write_kib=1 hbm_bytes=123 dispatches=3\n"
                       f"cell set=headline label=M4 kernel=mfma fingerprint={bench.fingerprint('mfma')} "
                       f"fetch_kib=1 write_kib=1 hbm_bytes=456 dispatches=3\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", summary)
    assert bench.read_traffic("qmv", [1]) is None      # stale fingerprint
    assert bench.read_traffic("mfma", [4]) == 456.0
    assert bench.read_traffic("mfma", [4, 16]) is None  # a cell missing


def test_host_cores_and_cpu_model():
    c = bench.host_cores()
    assert 1 <= c["usable"] <= c["affinity_cpus"] <= c["logical_cpus"]
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_alternating_trial_order(monkeypatch):
    """timed_cells replays the cells forward, reverse, forward."""
    order = []

    class G:
        def __init__(self, key):
            self.key = key

        def replay(self):
            order.append(self.key)

    monkeypatch.setattr(bench, "capture_graph", lambda fn, reps: G(fn))
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda *a: None)
    monkeypatch.setattr(bench, "time_launches", lambda fn, reps, stream: (fn(0), 1.0)[1])
    res = bench.timed_cells([("a", "a", 1), ("b", "b", 1), ("c", "c", 1)], None)
    assert order == ["a", "b", "c"] + ["a", "b", "c", "c", "b", "a", "a", "b", "c"]
    assert all(len(v) == bench.TRIALS for v in res.values())


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    """bench.py measures one GPU: --gpus N with N != 1 exits before any GPU work."""
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU only" in capsys.readouterr().err


def test_counter_summary_averages_warm_rounds(tmp_path):
    rows, manifest = _profile_run("SQ_INSTS_VALU", {1: 100.0, 4: 400.0, 16: 1600.0, "copy": 1.0}.__getitem__)
    # the cold first round reads differently and must be dropped
    rows = [(d, n, c, (v * 3 if d < 3 + len(bench.CELLS_M) and "qmm::" in n else v)) for d, n, c, v in rows]
    _write_counters(tmp_path / "a", rows)
    man = tmp_path / "manifest.json"
    man.write_text(json.dumps(manifest))
    out = tmp_path / "out"
    out.mkdir()
    written = bench.summarize_counters([str(tmp_path / "a")], str(out), str(man))
    text = written[0].read_text()
    assert written[0].name == "dense_up_w4g32_sq_counters.txt"
    assert "M1 | qmv | 100" in text and "M4 | mfma | 400" in text and "M16 | mfma | 1600" in text


def test_y_fill_counted_with_the_long_k_launch():
    """The fill that clears y ahead of a long-K launch carries no manifest
    label of its own: its counts are added to the launch that follows it."""
    mfma = "void qmm::(anonymous namespace)::mfma_xr_kernel<4>(x)"
    fill = "qmm::(anonymous namespace)::zero_kernel(float*, unsigned long)"
    seq = [(0, "void at::native::upload(x)", 5.0), (1, fill, 2.0), (2, mfma, 30.0), (3, mfma, 20.0),
           (4, "void at::native::copy(x)", 7.0)]
    labels = [{"set": "longk", "label": "S1", "round": 0, "algorithmic_bytes": 1},
              {"set": "headline", "label": "M4", "round": 0, "algorithmic_bytes": 1}]
    pairs, other = bench._split_library(seq, {"dispatches": labels})
    assert [(lab["label"], v) for lab, (_, v) in pairs] == [("S1", 32.0), ("M4", 20.0)]
    assert all("zero_kernel" not in n for _, (n, _) in pairs)
