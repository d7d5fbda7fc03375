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
    leg = {"kernel_digest": bench.kernel_digest("headline"), "bytes_per_call": 123,
           "read_bytes_per_call": 100, "write_bytes_per_call": 23}
    f.write_text(json.dumps({"legs": {"headline": leg}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for_launch() == 123
    assert bench.leg_traffic("backward") is None  # not profiled
    f.write_text(json.dumps({"legs": {"headline": dict(leg, kernel_digest="0" * 16)}}))
    assert bench.traffic_for_launch() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for_launch() is None


def test_leg_digests_follow_their_sources():
    # each leg is keyed by its own kernel file; the shared headers key all
    assert bench.kernel_digest("backward") != bench.kernel_digest("headline")
    assert (bench.kernel_digest("smallcache_backward_d256") ==
            bench.kernel_digest("smallcache_backward_d128"))


def test_leg_counter_summary_scales_by_the_copy_and_divides_by_calls(tmp_path):
    # the calibration copy of COPY_BYTES reads 1000 FETCH_SIZE units and 500
    # WRITE_SIZE units: one unit = COPY_BYTES / 1000 and COPY_BYTES / 500 bytes
    _counter_csv(tmp_path / "copyfetch_counter_collection.csv",
                 [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1000.0)])
    _counter_csv(tmp_path / "copywrite_counter_collection.csv",
                 [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 500.0)])
    # two calls of the backward: three kernels each, plus a forward call that
    # is not part of the leg
    rows_f = [("bwd_preprocess<128>", "FETCH_SIZE", 1.0), ("bwd_dkdv3<128, 8>", "FETCH_SIZE", 10.0),
              ("bwd_dq3<128, 8, 64>", "FETCH_SIZE", 20.0)] * 2
    rows_f.append(("fwd_fused_bf16_direct_kernel<128, 8, 64, 2>", "FETCH_SIZE", 999.0))
    rows_w = [("bwd_preprocess<128>", "WRITE_SIZE", 2.0), ("bwd_dkdv3<128, 8>", "WRITE_SIZE", 4.0),
              ("bwd_dq3<128, 8, 64>", "WRITE_SIZE", 6.0)] * 2
    _counter_csv(tmp_path / "backward_fetch_counter_collection.csv", rows_f)
    _counter_csv(tmp_path / "backward_write_counter_collection.csv", rows_w)
    (tmp_path / "backward_calls.json").write_text('noise\n{"leg": "backward", "calls": 2}\n')
    out = tmp_path / "t.json"
    bench.summarize_leg_counters(str(tmp_path), str(out))
    t = json.loads(out.read_text())
    leg = t["legs"]["backward"]
    rf, rw = bench.COPY_BYTES / 1000.0, bench.COPY_BYTES / 500.0
    assert leg["read_bytes_per_call"] == round(31.0 * rf)
    assert leg["write_bytes_per_call"] == round(12.0 * rw)
    assert leg["bytes_per_call"] == round(31.0 * rf + 12.0 * rw)
    assert leg["dispatches"] == [6, 6] and leg["kernel_digest"] == bench.kernel_digest("backward")
    assert set(t["legs"]) == {"backward"}


def test_theorem_1_1_takes_the_term_of_its_regime():
    class W:
        bh, n, d = 2, 4096, 128
    w = W()
    n, d = w.n, w.d
    big = bench.theorem_1_1(w, 4 * d * d)  # M >= d^2: (n^2 d^2 + n d^3) / M
    assert big["regime"].startswith("large")
    assert big["elements"] == round(2 * (n * n * d * d + n * d ** 3) / (4 * d * d))
    small = bench.theorem_1_1(w, d * d // 4)  # M < d^2: (n^2 d + n d^2) / sqrt(M)
    assert small["regime"].startswith("small")
    assert small["elements"] == round(2 * (n * n * d + n * d * d) / (d / 2))
    assert small["bytes"] == round(2 * 2 * (n * n * d + n * d * d) / (d / 2))
    # at M = d^2 the two terms coincide
    eq = bench.theorem_1_1(w, d * d)
    assert eq["elements"] == round(2 * (n * n * d + n * d * d) / d)


def _counter_csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, counter, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_sweep_kernel_keys():
    assert bench.fused_sweep_key(
        "at::fwd_fused_bf16_direct_kernel<128, 8, 64, true, 2, false, 2, 0, true>(x)") == (256, 64)
    assert bench.fused_sweep_key("at::fwd_fused_bf16_direct_kernel<256, 4, 32>(x)") is None
    assert bench.fused_sweep_key(
        "_ZN2at28fwd_fused_bf16_direct_kernelILi128ELi4ELi32ELi2EEEvPKDF16b") == (128, 32)
    assert bench.fused_sweep_key("_ZN2at28fwd_fused_bf16_direct_kernelILi256ELi4ELi32E") is None
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


def test_bwd_sweep_keys_and_summary(tmp_path):
    assert bench.bwd_sweep_key("void at::bwd_dkdv3<128, 8>(a)") == ("dkdv", 8)
    assert bench.bwd_sweep_key("_ZN2at9bwd_dkdv3ILi128ELi4EEEvPKDF16b") == ("dkdv", 4)
    assert bench.bwd_sweep_key("void at::bwd_dq3<128, 8, 32>(a)") == ("dq", 8, 32)
    assert bench.bwd_sweep_key("_ZN2at7bwd_dq3ILi128ELi4ELi64EEEvPK") == ("dq", 4, 64)
    assert bench.bwd_sweep_key("void at::bwd_dq3<64, 8, 64>(a)") is None
    assert bench.bwd_sweep_key("bwd_preprocess<128>") is None
    # one shape: its dK/dV and dQ kernels' counters add; copy calibration
    # makes one TCC_READ_SECTORS unit 2 bytes and one FETCH_SIZE unit 4
    c = bench.COPY_BYTES
    _counter_csv(tmp_path / "copyread_counter_collection.csv",
                 [("__amd_rocclr_copyBuffer", "TCC_READ_SECTORS_sum", c / 2)])
    _counter_csv(tmp_path / "copyfetch_counter_collection.csv",
                 [("__amd_rocclr_copyBuffer", "FETCH_SIZE", c / 4)])
    dk, dq = "void at::bwd_dkdv3<128, 8>(a)", "void at::bwd_dq3<128, 8, 64>(a)"
    _counter_csv(tmp_path / "bwdread_counter_collection.csv",
                 [(dk, "TCC_READ_SECTORS_sum", 300.0), (dq, "TCC_READ_SECTORS_sum", 200.0)])
    _counter_csv(tmp_path / "bwdfetch_counter_collection.csv",
                 [(dk, "FETCH_SIZE", 10.0), (dq, "FETCH_SIZE", 5.0)])
    _counter_csv(tmp_path / "bwdmfma_counter_collection.csv",
                 [(dk, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 30), (dk, "GRBM_GUI_ACTIVE", 8 * 60.0),
                  (dq, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 10), (dq, "GRBM_GUI_ACTIVE", 8 * 40.0)])
    timing = tmp_path / "t.jsonl"
    timing.write_text(json.dumps({"tile": "k256q256c64", "keys_per_block": 256,
                                  "queries_per_block": 256, "key_tile": 64, "onchip_elems": 9,
                                  "ms": 1.0, "tflops_at_10N2d": 2.0,
                                  "sched_read_bytes": 1000.0}) + "\n")
    out = tmp_path / "t.md"
    bench.summarize_bwd_sweep(str(tmp_path), str(timing), str(out))
    row = [line for line in out.read_text().splitlines() if line.startswith("| k256")][0]
    cells = [x.strip() for x in row.strip("|").split("|")]
    assert cells[7] == f"{1000 / 1e9:.2f} GB"       # (300 + 200) sectors x 2 bytes
    assert cells[9] == "1.000"                          # against the 1000-byte schedule
    assert cells[10] == f"{60 / 1e9:.3f} GB"           # (10 + 5) x 4 bytes
    assert cells[11] == bench.fmt_busy(40.0 / 100.0)   # (30 + 10) / (60 + 40)
