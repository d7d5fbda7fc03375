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



def _counter_csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, counter, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_sweep_kernel_keys():
    assert bench.fused_sweep_key(
        "at::fwd_fused_bf16_direct_kernel<128, 8, 64, true, 2, false, 2, 0, true>(x)") == (256, 64)
    assert bench.fused_sweep_key("at::fwd_fused_bf16_direct_kernel<256, 4, 32>(x)") is None
    assert bench.smallcache_sweep_key("void at::sc_scores_exp<256, 128>(a)") == 128
    assert bench.smallcache_sweep_key("_ZN2at16sc_value_productILi256ELi64EEEvPKDF16b") == 64
    assert bench.smallcache_sweep_key("_ZN2at16sc_value_productILi128ELi64EEEvPKDF16b") is None


def test_mfma_busy_sums_the_kernels_of_one_key(tmp_path):
    # two kernels of one tile: busy cycles add, and so do their cycles; per
    # dispatch means first (two dispatches of the scores kernel)
    rows = [("sc_scores_exp<256, 128>", "SQ_VALU_MFMA_BUSY_CYCLES", 1280.0),
            ("sc_scores_exp<256, 128>", "SQ_VALU_MFMA_BUSY_CYCLES", 1280.0),
            ("sc_scores_exp<256, 128>", "GRBM_GUI_ACTIVE", 20.0),
            ("sc_scores_exp<256, 128>", "GRBM_GUI_ACTIVE", 20.0),
            ("_ZN2at16sc_value_productILi256ELi128EEEvPKDF16b", "SQ_VALU_MFMA_BUSY_CYCLES", 2560.0),
            ("_ZN2at16sc_value_productILi256ELi128EEEvPKDF16b", "GRBM_GUI_ACTIVE", 30.0),
            ("copyBuffer", "GRBM_GUI_ACTIVE", 99.0)]
    _counter_csv(tmp_path / "m.csv", rows)
    busy = bench.mfma_busy(str(tmp_path), "m.csv", bench.smallcache_sweep_key)
    assert set(busy) == {128}
    assert abs(busy[128] - (1280.0 + 2560.0) / (128.0 * (20.0 + 30.0))) < 1e-12
    assert bench.mfma_busy(str(tmp_path), "absent.csv", bench.smallcache_sweep_key) == {}
