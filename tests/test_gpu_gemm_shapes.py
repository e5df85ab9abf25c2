"""GPU parity of the bf16 GEMM on the matrix cores at mid-size and large shapes: the encoder's
n = 1500 layers and ragged neighbours (every tile variant the launcher picks there), a long-k
case with few tiles, and 4096^3 (the 128 x 256 tile), with every epilogue flag, alpha and the
f32-accurate variant; outputs NaN-prefilled with canaries. The bf16 GEMM sums in a fixed order,
so repeated calls must agree bit for bit.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded

pytestmark = pytest.mark.gpu

# (n, m, k)
SHAPES = [
    (1500, 1024, 1024),   # the encoder's output projection
    (1500, 3072, 1024),   # its QKV projection
    (300, 700, 4096),     # few tiles, long k, ragged in both
    (129, 257, 8192),     # one tile row and column past a tile edge, longest k
    (700, 520, 2048),
    (1500, 4096, 1024),   # the MLP up projection: X rounded to bf16 once as it is staged
    (1480, 4200, 512),    # the same route, ragged in n and m
    (1500, 1024, 4096),   # the MLP down projection: 64 x 128 tiles with a 4-slot ring
    (1500, 2048, 1024),   # 64 x 128 tiles two per CU, 2-slot ring
]

FLAGS = [wq.BIAS, wq.BIAS | wq.GELU, wq.BIAS | wq.RESIDUAL, wq.RESIDUAL, wq.BIAS | wq.SILU | wq.RESIDUAL,
         wq.TANH, wq.RELU | wq.BIAS, 0]


def _inputs(n, m, k, flags, seed=0):
    g = synth.rng(90, seed, n, m, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.bf16_weight(g, m, k, 0.03)
    bias = synth.normal_f32(g, (m,), 0.1) if flags & wq.BIAS else None
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    return x, w, bias, y_old


def _act(flags):
    for name, bit in (("gelu", wq.GELU), ("silu", wq.SILU), ("relu", wq.RELU), ("tanh", wq.TANH)):
        if flags & bit:
            return name
    return None


def _run(x, w, m, k, bias, flags, y_old, path, alpha=1.0):
    n = x.shape[0]
    buf, out = guarded_out(n, m, y_old if flags & wq.RESIDUAL else None)
    wq.gemm(dev(x), dev(w), wq.W_BF16, m=m, k=k, bias=None if bias is None else dev(bias), act=_act(flags),
            residual=bool(flags & wq.RESIDUAL), out=out, path=path, alpha=alpha)
    return read_guarded(buf, n, m)


@pytest.mark.parametrize("n,m,k", SHAPES)
@pytest.mark.parametrize("fi", range(len(FLAGS)))
def test_gemm_shape_parity(n, m, k, fi):
    flags = FLAGS[fi]
    x, w, bias, y_old = _inputs(n, m, k, flags)
    alpha = 1.0 if fi % 3 else 0.75
    got = _run(x, w, m, k, bias, flags, y_old, wq.PATH_MFMA, alpha)
    # Columns spread over every tile plus both edges; every row.
    cols = np.unique(np.concatenate([np.arange(min(m, 40)), np.arange(max(0, m - 40), m),
                                     synth.rng(91, n, m).choice(m, min(m, 300), replace=False)]))
    y_ref, tol = oracle_with_tol(x, w, wq.W_BF16, m, k, bias, flags, y_old, B_MFMA, rows=cols, alpha=alpha)
    assert_within(got[:, cols], y_ref, tol, f"bf16 gemm {n}x{m}x{k} flags={flags}")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("n,m,k", [(1500, 1024, 1024), (300, 700, 4096), (129, 257, 8192)])
def test_gemm_shape_f32_accurate(n, m, k):
    flags = wq.BIAS | wq.GELU
    x, w, bias, _ = _inputs(n, m, k, flags, seed=1)
    got = _run(x, w, m, k, bias, flags, None, wq.PATH_MFMA_F32)
    cols = np.unique(np.concatenate([np.arange(min(m, 40)), np.arange(max(0, m - 40), m),
                                     synth.rng(92, n, m).choice(m, min(m, 300), replace=False)]))
    y_ref, tol = oracle_with_tol(x, w, wq.W_BF16, m, k, bias, flags, None, B_F32, rows=cols)
    assert_within(got[:, cols], y_ref, tol, f"f32-accurate {n}x{m}x{k}")


@pytest.mark.parametrize("n,m,k,flags", [(1500, 1024, 4096, wq.BIAS | wq.RESIDUAL), (1500, 4096, 1024, wq.BIAS | wq.GELU)])
def test_bf16_gemm_is_deterministic(n, m, k, flags):
    x, w, bias, y_old = _inputs(n, m, k, flags, seed=2)
    first = _run(x, w, m, k, bias, flags, y_old, wq.PATH_MFMA)
    for _ in range(3):
        again = _run(x, w, m, k, bias, flags, y_old, wq.PATH_MFMA)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_gemm_large_square_sampled():
    """4096^3 (128 x 256 tiles, one per CU): sampled rows and columns against the oracle, every output finite."""
    n = m = k = 4096
    x, w, bias, _ = _inputs(n, m, k, wq.BIAS, seed=3)
    got = _run(x, w, m, k, bias, wq.BIAS, None, wq.PATH_MFMA)
    assert np.isfinite(got).all()
    g = synth.rng(93)
    rows = np.unique(np.concatenate([[0, 127, 128, 4095], g.choice(n, 60, replace=False)]))
    cols = np.unique(np.concatenate([[0, 255, 256, 4095], g.choice(m, 200, replace=False)]))
    y_ref, tol = oracle_with_tol(x[rows], w, wq.W_BF16, m, k, bias, wq.BIAS, None, B_MFMA, rows=cols)
    assert_within(got[np.ix_(rows, cols)], y_ref, tol, "4096^3 sampled")
