"""Child process of tests/test_gpu_gemm_wide_offsets.py: bf16 GEMMs on the route that operands of
4 GiB or more take, forced at small shapes by WQ_GEMM_WIDE_OFFSETS=1 (the library reads it once per
process, so the check runs in a process of its own). Prints one line per case and exits non-zero on
the first failure.
"""
import os
import sys

import numpy as np

if os.environ.get("WQ_GEMM_WIDE_OFFSETS") != "1":
    sys.exit("WQ_GEMM_WIDE_OFFSETS=1 must be set in the environment")

import gemv_wq_gemm_amd as wq  # noqa: E402

if os.environ.get("WQ_TEST_LIB"):
    wq.LIB_PATH = os.environ["WQ_TEST_LIB"]

import synth  # noqa: E402
from tests.parity import (B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol,  # noqa: E402
                          read_guarded)

# (n, m, k): one tile; ragged in n and m past 128-row/column tiles; long k; many tiles with few CUs
# idle (no k split); and few tiles with a long k (the k split of residual layers).
SHAPES = [(1, 32, 32), (130, 259, 96), (257, 129, 1024), (64, 700, 2048), (600, 640, 512)]
FLAGS = [0, wq.BIAS, wq.BIAS | wq.GELU, wq.RESIDUAL, wq.BIAS | wq.RESIDUAL, wq.BIAS | wq.SILU | wq.RESIDUAL,
         wq.RELU, wq.TANH | wq.BIAS]
ACTS = (("gelu", wq.GELU), ("silu", wq.SILU), ("relu", wq.RELU), ("tanh", wq.TANH))


def _case(n, m, k, flags, path, alpha):
    g = synth.rng(97, n, m, k, flags, path)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.bf16_weight(g, m, k, 0.03)
    bias = synth.normal_f32(g, (m,), 0.1) if flags & wq.BIAS else None
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    act = next((name for name, bit in ACTS if flags & bit), None)
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wq.W_BF16, m=m, k=k, bias=None if bias is None else dev(bias), act=act,
            residual=bool(flags & wq.RESIDUAL), out=out, path=path, alpha=alpha)
    got = read_guarded(buf, n, m)
    bound = B_F32 if path == wq.PATH_MFMA_F32 else B_MFMA
    y_ref, tol = oracle_with_tol(x, w, wq.W_BF16, m, k, bias, flags, y_old, bound, alpha=alpha)
    assert_within(got, y_ref, tol, f"wide-offset route {n}x{m}x{k} flags={flags} path={path} alpha={alpha}")


def main():
    count = 0
    for n, m, k in SHAPES:
        for i, flags in enumerate(FLAGS):
            for path in (wq.PATH_MFMA, wq.PATH_MFMA_F32):
                alpha = 0.75 if i % 3 == 0 else 1.0
                print(f"case {n}x{m}x{k} flags={flags} path={path}", flush=True)
                _case(n, m, k, flags, path, alpha)
                count += 1
    print(f"ok {count}", flush=True)


if __name__ == "__main__":
    main()
