"""Host logic of the benchmark's profile summaries (no GPU): the HBM traffic
of a launch is its FETCH_SIZE and WRITE_SIZE counts (KiB per dispatch)
scaled by what the same counters read for a copy of known size, and a
summary is only used while the kernel's sources match its fingerprint."""
import csv

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
    """Dispatches in the order of bench.py --profile-run: uploads, PROFILE_REPS
    rounds of the three cells, then PROFILE_REPS calibration copies."""
    names = {1: "void qmm::(anonymous namespace)::qmv_kernel<4>(x)",
             4: "void qmm::(anonymous namespace)::mfma_xr_kernel<4>(x)",
             16: "void qmm::(anonymous namespace)::mfma_xr_kernel<4>(x)"}
    rows, d = [], 0
    for _ in range(3):  # input uploads (not library kernels)
        rows.append((d, "void at::native::upload(x)", counter, 10.0)); d += 1
    for _ in range(bench.PROFILE_REPS):
        for M in bench.CELLS_M:
            rows.append((d, names[M], counter, kib_of(M))); d += 1
    for _ in range(bench.PROFILE_REPS):
        rows.append((d, "void at::native::vectorized_elementwise_kernel<4>(copy)", counter, kib_of("copy"))); d += 1
    return rows


def test_traffic_scaled_by_the_copy_calibration(tmp_path, monkeypatch):
    copy_bytes = 4 * bench.COPY_ELEMS
    # FETCH_SIZE reads half the bytes of the copy (scale 2), WRITE_SIZE all (scale 1)
    fetch = {1: 27000.0, 4: 28000.0, 16: 28400.0, "copy": copy_bytes / 2 / 1024}
    write = {1: 68.0, 4: 272.0, 16: 1088.0, "copy": copy_bytes / 1024}
    _write_counters(tmp_path / "f", _profile_run("FETCH_SIZE", fetch.__getitem__))
    _write_counters(tmp_path / "w", _profile_run("WRITE_SIZE", write.__getitem__))
    out = tmp_path / "summary.txt"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out))
    monkeypatch.setattr(bench, "PMC_SUMMARY", out)
    for M in bench.CELLS_M:
        want = fetch[M] * 1024 * 2 + write[M] * 1024
        kernel = "qmv" if M == 1 else "mfma"
        assert bench.read_traffic(kernel, [M]) == pytest.approx(want, rel=1e-9)
    assert bench.read_traffic("mfma", [4, 16]) == pytest.approx(
        (fetch[4] + fetch[16]) * 1024 + (write[4] + write[16]) * 512, rel=1e-9)


def test_traffic_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    summary = tmp_path / "summary.txt"
    summary.write_text(f"cell M=1 kernel=qmv fingerprint=0000000000000000 fetch_kib=1 write_kib=1 "
                       f"hbm_bytes=123 dispatches=3\n"
                       f"cell M=4 kernel=mfma fingerprint={bench.fingerprint('mfma')} fetch_kib=1 "
                       f"write_kib=1 hbm_bytes=456 dispatches=3\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", summary)
    assert bench.read_traffic("qmv", [1]) is None      # stale fingerprint
    assert bench.read_traffic("mfma", [4]) == 456.0
    assert bench.read_traffic("mfma", [4, 16]) is None  # a cell missing


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    """bench.py measures one GPU: --gpus N with N != 1 exits before any GPU work."""
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU only" in capsys.readouterr().err
