"""Host logic of bench.py (CPU only): the one-GPU rule, and the guard that
reports stored HBM traffic only while the kernel sources and tile it was
measured on are unchanged."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_is_reported_only_for_the_measured_sources_and_tile(monkeypatch, tmp_path):
    rec = tmp_path / "counters.txt"
    rec.write_text("# comment: ignored\nsource_sha256: abc\ntile: 256x256_w8_k64\nbytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(rec))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda key="gemm_rs_tp4": "abc")
    assert bench.measured_traffic("gemm_rs_tp4", "256x256_w8_k64") == 1234
    assert bench.measured_traffic("gemm_rs_tp4", "128x128") is None           # another tile
    monkeypatch.setattr(bench, "kernel_source_digest", lambda key="gemm_rs_tp4": "def")
    assert bench.measured_traffic("gemm_rs_tp4", "256x256_w8_k64") is None    # sources changed since
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("gemm_rs_tp4", "256x256_w8_k64") is None    # no stored counters


def test_every_counter_record_names_existing_sources():
    for key, (fname, sources) in bench.COUNTERS.items():
        assert fname.endswith(".txt")
        for src in sources:
            assert os.path.exists(os.path.join(bench.CSRC, src)), (key, src)
        assert len(bench.kernel_source_digest(key)) == 64


def test_stats_and_roofline():
    st = bench.stats([3.0, 1.0, 2.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert st["ms_min"] == 1.0 and st["ms_median"] == 6.0 and st["ms_p90"] == 10.0 and st["iters"] == 10
    r = bench.roofline("mfma", 2.0e12, dict(ms_median=1.0), 2500.0, "TFLOP/s")
    assert abs(r["achieved"] - 2000.0) < 1e-9 and abs(r["frac"] - 0.8) < 1e-12
    r = bench.roofline("hbm", 4.0e9, dict(ms_median=1.0), 8000.0, "GB/s")
    assert abs(r["achieved"] - 4000.0) < 1e-9 and abs(r["frac"] - 0.5) < 1e-12
