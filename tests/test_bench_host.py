"""Host-side logic of the bench and its profile reader (no GPU): the one-GPU contract, argument
checks, the HBM-traffic reader that drops figures taken on other kernel sources, and the
repetition statistics."""
import os
import subprocess
import sys

import numpy as np

import bench
from gemv_wq_gemm_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_bench_rejects_steps_that_are_not_whole_blocks():
    r = _run_bench("--steps", "3")
    assert r.returncode == 2
    assert "multiple of 5" in r.stderr


def test_read_traffic_requires_the_current_sources(tmp_path):
    digest = rs.source_digest()
    good = tmp_path / "good.md"
    good.write_text(f"# counters\nsource_digest {digest}\ntraffic gemm_fc2 111939870\ntraffic q4_0_n1 33321632\n")
    assert rs.read_traffic(str(good), "gemm_fc2") == 111939870.0
    assert rs.read_traffic(str(good), "q4_0_n1") == 33321632.0
    assert rs.read_traffic(str(good), "absent") is None
    stale = tmp_path / "stale.md"
    stale.write_text("source_digest 0000000000000000\ntraffic gemm_fc2 111939870\n")
    assert rs.read_traffic(str(stale), "gemm_fc2") is None
    undated = tmp_path / "undated.md"
    undated.write_text("traffic gemm_fc2 111939870\n")
    assert rs.read_traffic(str(undated), "gemm_fc2") is None
    assert rs.read_traffic(str(tmp_path / "missing.md"), "gemm_fc2") is None


def test_source_digest_covers_every_kernel_source():
    # Every HIP source and device header of the library (the bench's own read kernel aside), and the
    # build flags, so a change to any of them voids the recorded counters.
    csrc = os.path.join(ROOT, "gemv_wq_gemm_amd", "csrc")
    kernel_files = {f"csrc/{f}" for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")) and f != "bench_read.hip"}
    assert kernel_files <= set(rs.KERNEL_SOURCES)
    assert "build.py" in rs.KERNEL_SOURCES
    d = rs.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert rs.source_digest() == d
    # Another file list gives another digest.
    assert rs.source_digest(rs.KERNEL_SOURCES[:-1]) != d


def test_stats_are_median_min_and_max_in_microseconds():
    st = bench._stats([0.010, 0.030, 0.020, 0.050, 0.040])  # ms per call
    assert st == {"median_us": 30.0, "min_us": 10.0, "max_us": 50.0, "reps": 5}
    assert np.isclose(bench._stats([0.0125])["median_us"], 12.5)
