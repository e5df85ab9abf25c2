"""GPU parity of the bf16 GEMM route that X or W of 4 GiB or more take (gemm_kernel with 64-bit
offsets instead of the pipelined bf16 kernel). The library's WQ_GEMM_WIDE_OFFSETS=1 hook forces it
at small, ragged shapes; the library reads the hook once per process, so the cases run in a child
process (tests/wide_offsets_child.py) against the oracle, with every epilogue flag, alpha, and both
matrix-core paths.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_wide_offset_route_matches_oracle():
    env = dict(os.environ, WQ_GEMM_WIDE_OFFSETS="1")
    r = subprocess.run([sys.executable, "-u", "-m", "tests.wide_offsets_child"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=110)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert r.stdout.strip().splitlines()[-1] == "ok 80", tail
