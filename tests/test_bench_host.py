"""bench.py's host-side logic, checked on the CPU: the HBM-traffic records (rocprofv3
counter CSVs scaled by the copy calibration and keyed to the kernel source they were
taken on), the settle phase's no-op setting, and the one-GPU guard."""
import csv
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, grid, value in rows:
            w.writerow({"Kernel_Name": kernel, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_write_traffic_scales_each_counter_by_the_copy_and_keys_the_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("the kernel as measured")
    rec_file = tmp_path / "record.json"
    monkeypatch.setattr(bench, "TRAFFIC", {"k": {"file": str(rec_file), "src": str(src),
                                                 "kernel": "my_kernel<128, false>", "grid": 1024}})
    # FETCH_SIZE reads the 1 GiB copy as 0.5 GiB (factor 2), WRITE_SIZE as 1 GiB (factor 1); a
    # dispatch of the same kernel on another grid and other kernels are left out
    fetch = [("void copyBuffer(...)", 4096, 524288.0),
             ("void my_kernel<128, false>(Args)", 1024, 100.0),
             ("void my_kernel<128, false>(Args)", 1024, 300.0),
             ("void my_kernel<128, false>(Args)", 512, 99999.0),
             ("void other_kernel(Args)", 1024, 7.0)]
    write = [("void copyBuffer(...)", 4096, 1048576.0),
             ("void my_kernel<128, false>(Args)", 1024, 50.0)]
    fcsv, wcsv = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_counter_csv(fcsv, "FETCH_SIZE", fetch)
    write_counter_csv(wcsv, "WRITE_SIZE", write)
    bench.write_traffic(str(fcsv), str(wcsv), "the command")
    rec = json.load(open(rec_file))
    assert rec["fetch_size_dispatches"] == 2 and rec["fetch_size_kib_avg"] == 200.0
    assert rec["calibration"]["FETCH_SIZE"]["factor"] == 2.0
    assert rec["calibration"]["WRITE_SIZE"]["factor"] == 1.0
    assert rec["fetch_size_bytes"] == 200.0 * 1024 * 2
    assert rec["write_size_bytes"] == 50.0 * 1024
    assert rec["hbm_bytes_per_launch"] == 200.0 * 1024 * 2 + 50.0 * 1024
    assert rec["kernel"] == "my_kernel<128, false>" and rec["command"] == "the command"
    assert rec["kernel_source_sha256"] == hashlib.sha256(b"the kernel as measured").hexdigest()
    # read back while the source is unchanged; null once it changes
    assert bench.measured_traffic("k") == rec["hbm_bytes_per_launch"]
    src.write_text("the kernel, edited")
    assert bench.measured_traffic("k") is None


def test_measured_traffic_without_a_record_is_null(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("x")
    monkeypatch.setattr(bench, "TRAFFIC", {"k": {"file": str(tmp_path / "missing.json"), "src": str(src),
                                                 "kernel": "k"}})
    assert bench.measured_traffic("k") is None


def test_traffic_table_names_existing_sources_and_profile_files():
    for which, t in bench.TRAFFIC.items():
        assert os.path.isfile(t["src"]), which
        assert os.path.dirname(t["file"]).endswith("profiles"), which


def test_settle_of_zero_milliseconds_runs_nothing():
    calls = []
    bench.settle(lambda: calls.append(1), 0.0)
    assert calls == []


def test_several_gpus_are_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_sizes_its_sample_to_the_target(monkeypatch):
    """The oracle leg's row sample lands near its time target when each oracle call
    carries a fixed cost (the output allocation) on top of work-proportional time:
    the two calibration runs cancel the fixed part.  A stand-in oracle sleeps 50 ms
    plus 3e-7 s per visible (row, key) pair of the rows it is asked for."""
    import time
    import types

    import numpy as np
    import oracle

    N = 4096
    x = types.SimpleNamespace(q=np.zeros((1, 2, N, 8)), k=np.zeros((1, 1, N, 8)), v=np.zeros((1, 1, N, 8)),
                              scale=1.0)

    def fake_prefill(q, k, v, causal, scale, row_step=1, **kw):
        rows = np.arange(0, N, row_step, dtype=np.float64)
        time.sleep(0.05 + 3e-7 * float((rows + 1).sum()))

    monkeypatch.setattr(oracle, "prefill", fake_prefill)
    for target in (0.4, 1.0):
        r = bench.cpu_baseline(x, target)
        wall = float(r["sample"].rsplit(", ", 1)[1].split(" s wall")[0])
        assert 0.5 * target <= wall <= 1.6 * target, (target, r["sample"])  # the row step is an integer
