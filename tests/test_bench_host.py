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
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "abc")
    assert bench.measured_traffic("256x256_w8_k64") == 1234
    assert bench.measured_traffic("128x128") is None           # another tile
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "def")
    assert bench.measured_traffic("256x256_w8_k64") is None    # sources changed since
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("256x256_w8_k64") is None    # no stored counters

