"""The weight-streaming kernels' tile offsets on the host, at weights above 2 GiB.

The sliced matvec clamps each 16-byte direct-to-LDS load of a tile to
``min(tile_bytes, (m - row0) * rowbytes) - 16``. For a weight whose bytes past
``row0`` exceed 2^31 (a bf16 152064 x 8192 output layer is 2.49 GB) that
product does not fit in 32 bits. This test compiles the kernels' own header
(``wq_tile_math.hpp``) into a host program and checks the clamp against exact
integer arithmetic, on cases where a 32-bit product would wrap.
"""
import os
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "gemv_wq_gemm_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "tile_offsets_test.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _wrap32(v: int) -> int:
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= 1 << 31 else v


def _exact(tile_bytes, m, row0, rowbytes):
    return min(tile_bytes, (m - row0) * rowbytes) - 16


def _int32_formula(tile_bytes, m, row0, rowbytes):
    """The clamp as a 32-bit int product (what the kernel computed before the fix)."""
    return min(tile_bytes, _wrap32((m - row0) * rowbytes)) - 16


CASES = [
    # (tile_bytes, m, row0, rowbytes): bf16 152064 x 8192 (rowbytes 16384) at 2 rows per tile
    (32768, 152064, 0, 16384),          # first tile: 2.49 GB left
    (32768, 152064, 20990, 16384),      # last tile whose bytes left still exceed 2^31
    (32768, 152064, 20992, 16384),      # exactly 2^31 bytes left
    (32768, 152064, 131072, 16384),     # the tile that starts at byte 2^31
    (32768, 152064, 152062, 16384),     # last full tile
    (32768, 152063, 152062, 16384),     # ragged last tile: one row left
    # f32 4096 rows of k = 8192 beyond 2^31 / 32768 rows, and Q4_0 with many rows
    (65536, 100000, 1, 32768),
    (18432, 200000000, 5, 4608),
    # small weights: the clamp is the tile itself or the bytes left
    (4096, 3, 0, 1024),
    (4096, 3, 2, 1024),
]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.access(HIPCC, os.X_OK):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("host") / "tile_offsets")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_cases_reach_past_2_gib():
    # The test is meaningful only if some case wraps in 32 bits.
    wrapped = [c for c in CASES if (c[1] - c[2]) * c[3] >= 1 << 31]
    assert len(wrapped) >= 3
    assert any(_int32_formula(*c) != _exact(*c) for c in CASES)


def test_tile_last_load_matches_exact_arithmetic(driver):
    inp = "".join(" ".join(str(v) for v in c) + "\n" for c in CASES)
    r = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True)
    got = [int(v) for v in r.stdout.split()]
    want = [_exact(*c) for c in CASES]
    assert got == want
    # Every clamp stays inside the tile and inside W.
    for (tb, m, row0, rb), g in zip(CASES, got):
        assert 0 <= g <= tb - 16 and row0 * rb + g + 16 <= m * rb
