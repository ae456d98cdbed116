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


def _write_counters(d, cname, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        for i, (kernel, kib) in enumerate(rows):
            f.write(f'{i},"{kernel}","{cname}",{kib},0,1000\n')


def test_traffic_calibration_takes_the_copy_not_smaller_dispatches_of_its_kernel(tmp_path):
    """The calibration copy (256 MiB read and written) shares its elementwise kernel with smaller
    scalar multiplies of the program; the scale must come from the copy alone."""
    from sparse_mixture_experts_02_amd.rocprof_summary import _calibrated_means
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float>>"
    gemm = "void moe::gemm_big_kernel<true, false, false>(moe::GemmParams)"
    mib = 1 << 20
    fetch_dir = os.path.join(str(tmp_path), "fetch")
    # the copy counts half its bytes, its two small siblings too; the GEMM 600 MiB
    _write_counters(fetch_dir, "FETCH_SIZE", [(copy, 131072.0), (copy, 16384.0), (copy, 16384.0), (gemm, 614400.0)])
    means, scale = _calibrated_means(fetch_dir, "FETCH_SIZE", "AUnaryFunctor", 256 * mib)
    assert scale == 2.0
    assert means[gemm] == 1200 * mib
