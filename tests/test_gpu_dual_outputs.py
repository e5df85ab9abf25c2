"""GPU parity of wavo's dual outputs (wq_linear_dual: outputs 0..dual-1 written again after the m
others, each with its own bias) against the f64 oracle, on every kernel route that stores the plain
layer: the matvec path (whose dual calls the general kernel takes, at every k), both GEMM kernels
(bf16 tile variants, quantized with and without the k split, f16 / f32 weights) and the
f32-accurate path, with activations, alpha and residual. The dual = 0 cases run on the sliced and
matrix-core matvec kernels too.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, SLOPES, ULP_SLACK, assert_within, dev, guarded_out, read_guarded

pytestmark = pytest.mark.gpu

# (label, wtype, n, m, k, path, bound)
ROUTES = [
    ("matvec general", wq.W_Q4_0, 3, 70, 96, wq.PATH_MATVEC, B_F32),
    ("matvec k 2048", wq.W_Q8_0, 4, 130, 2048, wq.PATH_MATVEC, B_F32),
    ("matvec 12 tokens k 2048", wq.W_Q8_0, 12, 75, 2048, wq.PATH_MATVEC, B_F32),
    ("gemm bf16 64x64", wq.W_BF16, 70, 140, 192, wq.PATH_MFMA, B_MFMA),
    ("gemm bf16 64x128 two per CU", wq.W_BF16, 1100, 2000, 64, wq.PATH_MFMA, B_MFMA),
    ("gemm bf16 128x256", wq.W_BF16, 2050, 4100, 128, wq.PATH_MFMA, B_MFMA),
    ("gemm quantized", wq.W_Q4_0, 130, 200, 256, wq.PATH_MFMA, B_MFMA),
    ("gemm quantized k split", wq.W_Q8_0, 300, 700, 512, wq.PATH_MFMA, B_MFMA),
    ("gemm f16 weights", wq.W_F16, 90, 100, 320, wq.PATH_MFMA, B_MFMA),
    ("gemm f32-accurate", wq.W_F32, 200, 288, 160, wq.PATH_MFMA_F32, B_F32),
]
ACT_FLAGS = {None: 0, "gelu": wq.GELU, "silu": wq.SILU, "relu": wq.RELU, "tanh": wq.TANH}


def _case(route, dual, act, residual, alpha, seed):
    label, wtype, n, m, k, path, bound = route
    flags = wq.BIAS | ACT_FLAGS[act] | (wq.RESIDUAL if residual else 0)
    g = synth.rng(seed, wtype, n, m, k, dual)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05, dsigma=0.01)
    bias = synth.normal_f32(g, (m + dual,), 0.3)
    y_old = synth.normal_f32(g, (n, m + dual), 1.0)
    buf, out = guarded_out(n, m + dual, y_old if residual else None)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), act=act, residual=residual, out=out, path=path,
            alpha=alpha, dual=dual)
    got = read_guarded(buf, n, m + dual)
    y_ref, S = oracle.linear_dual(x, w, wtype, m, k, dual, bias, flags, y_old if residual else None, alpha=alpha)
    v, _ = oracle.linear_dual(x, w, wtype, m, k, dual, bias, wq.BIAS)
    gs = SLOPES.get(ACT_FLAGS[act], 1.0)
    mag = np.abs(y_ref) + abs(alpha) * (np.abs(v) + np.abs(bias)[None, :]) + (np.abs(y_old) if residual else 0)
    tol = abs(alpha) * gs * bound * S + ULP_SLACK * mag
    assert_within(got, y_ref, tol, f"{label} dual={dual} act={act} residual={residual} alpha={alpha}")


@pytest.mark.parametrize("route", ROUTES, ids=[r[0] for r in ROUTES])
@pytest.mark.parametrize("dual_kind", ["one", "some", "all"])
def test_dual_outputs(route, dual_kind):
    m = route[3]
    dual = {"one": 1, "some": min(m, 33), "all": m}[dual_kind]
    _case(route, dual, "silu", False, 1.0, 91)
    _case(route, dual, None, True, 0.5, 92)


@pytest.mark.parametrize("route", ROUTES, ids=[r[0] for r in ROUTES])
def test_dual_zero_is_the_plain_layer(route):
    label, wtype, n, m, k, path, bound = route
    g = synth.rng(93, wtype)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05)
    bias = synth.normal_f32(g, (m,), 0.3)
    a = wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), act="gelu", path=path)
    b = wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), act="gelu", path=path, dual=0)
    import torch
    torch.cuda.synchronize()
    assert a.shape == b.shape == (n, m)
    assert torch.equal(a, b)
