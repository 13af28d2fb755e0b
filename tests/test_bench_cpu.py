"""Host logic of bench.py (no GPU): the one-GPU contract, the calibration of
the rocprofv3 byte counters against the probe of known traffic, and the
guard that voids stored traffic once the kernel source changes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DECODE = "void kda::decode_kernel<float, 128, 1, 16, 4, 0, true, true, 0, true>(kda::Ptrs, int)"
RMW = "(anonymous namespace)::rmw_kernel(float __vector(4)*, float)"


def _write_counters(d, counter, rows):
    """A rocprofv3 --pmc CSV (the columns bench.py reads) under d/host/pid/."""
    sub = os.path.join(d, "host", "123")
    os.makedirs(sub)
    with open(os.path.join(sub, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_calibrated_on_the_probe(tmp_path):
    # the probe moves grid x 16 bytes each way; its counters read half the
    # fetched bytes and all the written bytes (in KiB), as FETCH_SIZE and
    # WRITE_SIZE do on gfx950
    grid = 8_388_608
    probe_bytes = grid * 16
    fetch = [(RMW, grid, probe_bytes / 2 / 1024), (RMW, grid, probe_bytes / 2 / 1024),
             (DECODE, 2_097_152, 70_000.0), (DECODE, 2_097_152, 70_002.0), ("other", 64, 5.0)]
    write = [(RMW, grid, probe_bytes / 1024), (DECODE, 2_097_152, 136_192.0)]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    rec = bench.traffic_from_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), out=str(out))
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(70_001.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(136_192.0 * 1024)
    assert rec["decode_dispatches"] == [2, 1]
    assert json.loads(out.read_text())["traffic_bytes_per_launch"] == pytest.approx(
        rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"])
    # the stored figure is reported while the kernel source is unchanged ...
    assert bench.stored_traffic(str(out)) == pytest.approx(rec["traffic_bytes_per_launch"])
    # ... and voided once it changes
    stale = dict(rec, kernel_source_sha256_16="0" * 16)
    out.write_text(json.dumps(stale))
    assert bench.stored_traffic(str(out)) is None
    assert bench.stored_traffic(str(tmp_path / "missing.json")) is None


def test_traffic_needs_one_decode_kernel(tmp_path):
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", [(RMW, 16, 1.0)])
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", [(RMW, 16, 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(tmp_path / "fetch"), str(tmp_path / "write"),
                                    out=str(tmp_path / "t.json"))
