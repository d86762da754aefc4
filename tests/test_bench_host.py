"""CPU: bench.py's host-side logic (no GPU): the one-GPU guard, and the HBM
traffic figure built from rocprofv3 FETCH_SIZE / WRITE_SIZE counter files,
scaled by what the same counters read for the 1 GiB calibration copy."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def write_counters(path, counter, rows):
    """rows: (dispatch id, kernel name, grid size, value KiB)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, name, grid, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": v})


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    path = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_JSON", path)
    return path


def test_traffic_scaled_by_the_calibration_copy(tmp_path, traffic_file):
    kern = "void moe::gateup_q8_kernel<2>(moe::ExpertArgs, int, int, moe::SharedRows)"
    copy = "void at::native::vectorized_elementwise_kernel<neg_kernel ...>"
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half of what was read (the copy's 1 GiB shows as 0.5 GiB), two
    # dispatches of the kernel (per-instance rows summed per dispatch), a smaller copy
    # launch that is not the calibration one
    write_counters(tmp_path / "f.csv", "FETCH_SIZE", [
        (1, copy, 1 << 20, gib_kib / 2), (2, copy, 4096, 123.0),
        (3, kern, 512, 10000.0), (3, kern, 512, 5000.0), (4, kern, 512, 16000.0)])
    write_counters(tmp_path / "w.csv", "WRITE_SIZE", [
        (1, copy, 1 << 20, gib_kib), (3, kern, 512, 40.0), (4, kern, 512, 60.0)])
    bench.traffic_from(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "decode")
    rec = json.load(open(traffic_file))["decode"]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_bytes_per_launch"] == int(15500.0 * 1024 * 2)     # (15000 + 16000) / 2 KiB, x 2
    assert rec["write_bytes_per_launch"] == int(50.0 * 1024)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert bench.stored_traffic("decode") == rec["bytes_per_launch"]


def test_traffic_of_other_sources_is_not_used(traffic_file):
    with open(traffic_file, "w") as f:
        json.dump({"decode": {"bytes_per_launch": 123, "source_hash": "0" * 16}}, f)
    assert bench.stored_traffic("decode") is None
    assert bench.stored_traffic("prefill") is None


def test_traffic_needs_the_kernel_and_the_copy(tmp_path, traffic_file):
    write_counters(tmp_path / "f.csv", "FETCH_SIZE", [(1, "void moe::other_kernel()", 64, 1.0),
                                                      (2, "neg_kernel", 1024, 2.0)])
    write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(1, "void moe::other_kernel()", 64, 1.0),
                                                      (2, "neg_kernel", 1024, 2.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "decode")
    assert not os.path.exists(traffic_file)
