"""Host-side checks of bench.py: the roofline traffic figure is read from the
committed counter summary only while the GEMM source it was measured on is
unchanged, and more than one GPU is refused."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_matches_committed_kernels():
    for src in (bench.DENSE_SOURCE, bench.LOWBIT_SOURCE):
        t = bench.gemm_traffic(src)
        assert t is not None and t > 0, src


def test_traffic_is_null_for_another_source(tmp_path):
    src = tmp_path / os.path.basename(bench.DENSE_SOURCE)
    src.write_text(open(bench.DENSE_SOURCE).read() + "\n// changed\n")
    assert bench.gemm_traffic(str(src)) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
