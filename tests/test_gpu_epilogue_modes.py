"""GPU parity of the epilogue modes beyond bias / GELU / residual: SiLU, ReLU, tanh and the factor
alpha (wq_linear), wavo's `Epilogue` modes (gpu/mod.rs: Silu, Relu, Tanh, Residual(alpha),
GeluResidual), against the f64 oracle on every kernel route that stores outputs: the three matvec
kernels (general, k-sliced, matrix-core at 9-16 tokens), both GEMM kernels (bf16 tile variants,
quantized, with and without the k split) and the f32-accurate matrix-core path.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded
from tests.test_gpu_parity import _inputs

pytestmark = pytest.mark.gpu

ACTS = {None: 0, "gelu": wq.GELU, "silu": wq.SILU, "relu": wq.RELU, "tanh": wq.TANH}

# (label, wtype, n, m, k, path, bound): one case per kernel route.
ROUTES = [
    ("matvec general", wq.W_Q4_0, 3, 70, 96, wq.PATH_MATVEC, B_F32),
    ("matvec sliced", wq.W_Q8_0, 4, 130, 2048, wq.PATH_MATVEC, B_F32),
    ("matvec sliced bf16", wq.W_BF16, 1, 77, 1024, wq.PATH_MATVEC, B_F32),
    ("matvec matrix cores", wq.W_Q4_0, 12, 75, 2048, wq.PATH_MATVEC, B_F32),
    ("gemm bf16 64x64", wq.W_BF16, 70, 140, 192, wq.PATH_MFMA, B_MFMA),
    ("gemm bf16 64x128 two per CU", wq.W_BF16, 1100, 2000, 64, wq.PATH_MFMA, B_MFMA),
    ("gemm quantized", wq.W_Q8_0, 130, 200, 256, wq.PATH_MFMA, B_MFMA),
    ("gemm f32-accurate", wq.W_Q4_0, 90, 100, 320, wq.PATH_MFMA_F32, B_F32),
    ("gemm f32-accurate bf16", wq.W_BF16, 200, 288, 160, wq.PATH_MFMA_F32, B_F32),
]


def _run(x, w, wtype, m, k, bias, act, residual, alpha, y_old, path):
    n = x.shape[0]
    buf, out = guarded_out(n, m, y_old if residual else None)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=None if bias is None else dev(bias), act=act,
            residual=residual, out=out, path=path, alpha=alpha)
    return read_guarded(buf, n, m)


@pytest.mark.parametrize("route", ROUTES, ids=[r[0] for r in ROUTES])
@pytest.mark.parametrize("act", ["silu", "relu", "tanh", "gelu"])
@pytest.mark.parametrize("residual,alpha", [(False, 1.0), (True, 1.0), (True, 0.5), (False, -2.0)])
def test_activation_and_alpha(route, act, residual, alpha):
    label, wtype, n, m, k, path, bound = route
    flags = wq.BIAS | ACTS[act] | (wq.RESIDUAL if residual else 0)
    x, w, bias, y_old = _inputs(31, wtype, n, m, k, wq.BIAS | wq.RESIDUAL)
    got = _run(x, w, wtype, m, k, bias, act, residual, alpha, y_old, path)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound, alpha=alpha)
    assert_within(got, y_ref, tol, f"{label} act={act} residual={residual} alpha={alpha}")


@pytest.mark.parametrize("route", ROUTES, ids=[r[0] for r in ROUTES])
def test_residual_alpha_without_activation(route):
    """wavo Residual(alpha): c + alpha (a.W^T + b). Linear, so the quantized GEMM may split k."""
    label, wtype, n, m, k, path, bound = route
    flags = wq.BIAS | wq.RESIDUAL
    x, w, bias, y_old = _inputs(32, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, None, True, 0.5, y_old, path)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound, alpha=0.5)
    assert_within(got, y_ref, tol, f"{label} residual alpha=0.5")


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
def test_quantized_k_split_with_alpha(wtype):
    """Few tiles and a long k: the quantized GEMM splits k and adds alpha-scaled partial sums."""
    n, m, k = 300, 700, 512
    flags = wq.BIAS | wq.RESIDUAL
    x, w, bias, y_old = _inputs(33, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, None, True, -0.75, y_old, wq.PATH_MFMA)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_MFMA, alpha=-0.75)
    assert_within(got, y_ref, tol, "k split alpha=-0.75")


def test_activation_alone_on_exact_pre_activations():
    """Identity bf16 weights and bf16-exact inputs make the pre-activation exact on every path, so
    each activation's own evaluation is held to the f32 rounding slack alone."""
    import oracle
    from tests.parity import ULP_SLACK
    n, k = 4, 128
    j = np.arange(-255, 257, dtype=np.float64)
    x = (j / 32.0).astype(np.float32).reshape(n, k)
    w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)
    v = x.astype(np.float64)
    fns = {"silu": oracle.silu, "relu": oracle.relu, "tanh": oracle.tanh, "gelu": oracle.gelu_erf}
    for path in (wq.PATH_MATVEC, wq.PATH_MFMA, wq.PATH_MFMA_F32):
        for act, fn in fns.items():
            got = _run(x, w, wq.W_BF16, k, k, None, act, False, 1.0, None, path)
            y_ref = fn(v)
            assert_within(got, y_ref, ULP_SLACK * (np.abs(v) + np.abs(y_ref)) + 1e-30, f"{act} alone path={path}")
