"""Host-side checks of the benchmark driver (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_is_consistent():
    """The committed HBM-traffic record: fetched + written bytes per launch, its ratio to the
    algorithmic bytes of the 163840 x 2304 GEMV, and the copy-kernel scale factors."""
    with open(os.path.join(ROOT, "profiles", "traffic_gemv_163840x2304.json")) as f:
        t = json.load(f)
    assert t["algorithmic_bytes_per_launch"] == 163840 * 2304 // 2 + 163840 * 18 * 2 + 2304 * 2
    fetched = t["fetch_size_kib_per_dispatch"] * 1024 * t["fetch_scale"]
    written = t["write_size_kib_per_dispatch"] * 1024 * t["write_scale"]
    assert abs(fetched + written - t["bytes_per_launch"]) <= 2
    assert abs(t["bytes_per_launch"] / t["algorithmic_bytes_per_launch"]
               - t["ratio_to_algorithmic"]) < 1e-3
    assert abs(t["copy_reference_bytes"] - t["copy_fetch_size_kib"] * 1024 * t["fetch_scale"]) \
        < 0.001 * t["copy_reference_bytes"]
    assert t["copy_write_size_kib"] * 1024 * t["write_scale"] == t["copy_reference_bytes"]
    assert len(t["kernel_source_digest"]) == 16
