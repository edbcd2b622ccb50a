"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the
traffic arithmetic (counter CSVs -> bytes per launch, scaled by the copy
kernel's reading) and the rule that a traffic record counts only for the
kernel sources it was taken on."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for did, name, value in rows:
            w.writerow(dict(Dispatch_Id=did, Kernel_Name=name, Counter_Name=counter, Counter_Value=value))


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    copy = "void at::native::vectorized_elementwise_kernel<4, copy>(...)"
    fwd = "void kd::fwd_kernel<true, 1>(kd::LogitArgs)"
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1); the
    # counter is split over two rows of one dispatch for the forward kernel (summed), and the
    # median over its dispatches is taken
    _counters(tmp_path / "f.csv", "FETCH_SIZE", [(1, copy, gib_kib / 2), (2, fwd, 1000.0), (2, fwd, 500.0),
                                                 (3, fwd, 1500.0), (4, fwd, 9000.0)])
    _counters(tmp_path / "w.csv", "WRITE_SIZE", [(1, copy, gib_kib), (2, fwd, 10.0), (3, fwd, 10.0),
                                                 (4, fwd, 10.0)])
    out = tmp_path / "t.json"
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out))
    rec = json.loads(out.read_text())
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["fetch_kib"] == 1500.0 and rec["write_kib"] == 10.0
    assert rec["bytes_per_launch"] == 1500.0 * 1024 * 2 + 10.0 * 1024
    assert rec["kernel_source_hash"] == bench.kernel_hash()


def test_traffic_record_counts_only_for_its_sources(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    rec = tmp_path / "t.json"
    rec.write_text(json.dumps({"bytes_per_launch": 123.0, "kernel_source_hash": bench.kernel_hash()}))
    assert bench.recorded_traffic(str(rec)) == 123.0
    rec.write_text(json.dumps({"bytes_per_launch": 123.0, "kernel_source_hash": "0" * 16}))
    assert bench.recorded_traffic(str(rec)) is None
    rec.write_text("not json")
    assert bench.recorded_traffic(str(rec)) is None
    assert bench.recorded_traffic(str(tmp_path / "missing.json")) is None
