"""bench.py's own contract, without a GPU: one GPU only, and the roofline's traffic is read from a
profile only while the grouped-GEMM sources it was measured on are unchanged."""
import os
import subprocess
import sys

import bench
from sparse_mixture_experts_02_amd.rocprof_summary import gemm_sources_digest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no bench line


def _write_record(root, digest):
    os.makedirs(os.path.join(root, "profiles"))
    with open(os.path.join(root, "profiles", "traffic_wl.txt"), "w") as f:
        f.write("# some header\n")
        f.write(f"# grouped GEMM sources sha256: {digest}\n")
        f.write("# gemm1_silu fetch_bytes: 1000\n")
        f.write("# gemm1_silu write_bytes: 234\n")


def test_recorded_traffic_follows_the_sources_digest(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("wl", "gemm1_silu") is None   # no record
    _write_record(str(tmp_path), gemm_sources_digest())
    assert bench.recorded_traffic("wl", "gemm1_silu") == 1234
    assert bench.recorded_traffic("wl", "gemm2") is None        # no line for that kernel


def test_recorded_traffic_is_dropped_when_the_sources_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_record(str(tmp_path), "0" * 64)
    assert bench.recorded_traffic("wl", "gemm1_silu") is None
