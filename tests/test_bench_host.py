"""Host-side pieces of bench.py (no GPU): the one-GPU rule, percentiles, and
the HBM traffic summary being used only for the kernel source it was taken
on (otherwise the roofline's traffic is null)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_percentile_nearest_rank():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 0) == 1.0
    assert bench.percentile(xs, 100) == 5.0


def test_traffic_summary_applies_only_to_its_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_digest": bench.kernel_digest(), "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for_launch() == 123
    f.write_text(json.dumps({"kernel_digest": "0" * 16, "bytes_per_launch": 123}))
    assert bench.traffic_for_launch() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for_launch() is None

