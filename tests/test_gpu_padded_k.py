"""wavo's padded-k layer on the GPU (its test `gemm_padded_k`): a weight with k = 40 (f32 or f16)
is padded to 64 columns at load by wq_pad_weight, then multiplies 37 activation rows that are 64
wide with zeros after column 40 (as im2col rows are), on both paths. The padding itself must match
the oracle bit for bit, and wq_gemm must still refuse k = 40."""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wtype", [wq.W_F32, wq.W_F16, wq.W_BF16])
@pytest.mark.parametrize("m,k", [(64, 40), (37, 100), (5, 1), (129, 33), (16, 64)])
def test_pad_weight_is_bit_exact(wtype, m, k):
    raw = synth.weight(synth.rng(310, wtype, m, k), wtype, m, k, sigma=0.3)
    kp = wq.padded_k(k)
    buf, out = guarded_out(m, kp)
    wq.pad_weight(dev(raw), wtype, m=m, k=k, out=out)
    got = read_guarded(buf, m, kp)
    want, kp_o = oracle.pad_weight(raw, wtype, m, k)
    assert kp == kp_o
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("wtype", [wq.W_F32, wq.W_F16])
@pytest.mark.parametrize("path", [wq.PATH_AUTO, wq.PATH_MATVEC, wq.PATH_MFMA, wq.PATH_MFMA_F32])
def test_gemm_padded_k(wtype, path):
    n_out, k, rows = 64, 40, 37  # wavo's test: 64 outputs, k = 40 padded to 64, 37 activation rows
    g = synth.rng(311, wtype)
    raw = synth.weight(g, wtype, n_out, k, sigma=0.3)
    x = synth.normal_f32(g, (rows, 64), 1.0)
    x[:, k:] = 0.0
    bias = synth.normal_f32(g, (n_out,), 0.1)
    if path == wq.PATH_MATVEC:
        x = x[:16]
    n = x.shape[0]
    wp = wq.pad_weight(dev(raw), wtype, m=n_out, k=k)
    assert tuple(wp.shape) == (n_out, 64)
    # The unpadded layer is refused by the layer itself.
    with pytest.raises(wq.WqError, match="multiple of 32"):
        wq.gemm(dev(x[:, :k].copy()), dev(raw), wtype, m=n_out, k=k)
    buf, out = guarded_out(n, n_out)
    wq.gemm(dev(x), wp, wq.W_F32, m=n_out, k=64, bias=dev(bias), out=out, path=path)
    got = read_guarded(buf, n, n_out)
    # The oracle: the unpadded product over the first 40 columns (the zero columns add nothing).
    w_ref, _ = oracle.pad_weight(raw, wtype, n_out, k)
    bound = B_MFMA if path == wq.PATH_MFMA or (path == wq.PATH_AUTO and n > 16) else B_F32
    y_ref, tol = oracle_with_tol(x[:, :k], w_ref[:, :k].astype(np.float32), wq.W_F32, n_out, k, bias,
                                 wq.BIAS, None, bound)
    assert_within(got, y_ref, tol, f"padded k, wtype {wtype}, path {path}")
