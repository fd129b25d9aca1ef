"""bench.py pieces that run without a GPU: the one-GPU contract of the
command line, and the HBM-traffic figure taken from the committed counter
summary only while the kernel sources still match it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_figure_follows_the_kernel_sources(monkeypatch, tmp_path):
    got = bench.profiled_traffic()
    assert isinstance(got, int) and got > 18_898_944  # at least the algorithmic bytes
    # any other source text: the summary no longer describes the kernel
    other = tmp_path / "other.hip"
    other.write_text("// a different kernel\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(other),))
    monkeypatch.setattr(bench, "ROOT", "/")
    assert bench.profiled_traffic() is None
