"""Pins of the oracle's padded-k weights (wavo `Gpu::upload_linear`, the `kp != k` branch used
by `Gpu::conv`): brute force element by element, the product identity with zero-padded inputs,
and the sizes of the page's own `gemm_padded_k` test (k = 40 padded to 64)."""
import math

import numpy as np
import pytest

import oracle
import synth


def _brute_pad(raw, wtype, m, k, kp):
    """Element by element: the decoded weight where a column exists, else 0."""
    # decode one element at a time from its bit pattern (numpy's IEEE types, not oracle.decode)
    if wtype == oracle.W_F32:
        vals = np.asarray(raw, np.float32).reshape(m, k)
        get = lambda r, c: float(vals[r, c])
    elif wtype == oracle.W_F16:
        bits = np.asarray(raw, np.uint16).reshape(m, k)
        get = lambda r, c: float(np.array([bits[r, c]], np.uint16).view(np.float16)[0])
    else:
        bits = np.asarray(raw, np.uint16).reshape(m, k)
        get = lambda r, c: float(np.array([int(bits[r, c]) << 16], np.uint32).view(np.float32)[0])
    out = [[0.0] * kp for _ in range(m)]
    for r in range(m):
        for c in range(kp):
            out[r][c] = get(r, c) if c < k else 0.0
    return np.array(out)


@pytest.mark.parametrize("k,kp", [(1, 32), (31, 32), (32, 32), (33, 64), (40, 64), (100, 128), (240, 256)])
def test_padded_k(k, kp):
    assert oracle.padded_k(k) == kp


@pytest.mark.parametrize("wtype", [oracle.W_F32, oracle.W_F16, oracle.W_BF16])
@pytest.mark.parametrize("m,k", [(1, 1), (3, 40), (5, 33), (2, 64), (4, 100)])
def test_pad_weight_brute_force(wtype, m, k):
    raw = synth.weight(synth.rng(300, wtype, m, k), wtype, m, k, sigma=0.5)
    got, kp = oracle.pad_weight(raw, wtype, m, k)
    assert kp == oracle.padded_k(k) and got.shape == (m, kp)
    assert np.array_equal(got, _brute_pad(raw, wtype, m, k, kp))


def test_pad_weight_product_identity():
    """Zero columns in both operands leave the product unchanged: padded W times im2col-style rows
    (zero past k) equals W times the unpadded rows, summed exactly."""
    m, k, n = 7, 40, 5
    g = synth.rng(301)
    raw = synth.weight(g, oracle.W_F16, m, k, sigma=0.5)
    x = synth.normal_f32(g, (n, k), 1.0)
    wp, kp = oracle.pad_weight(raw, oracle.W_F16, m, k)
    xp = np.zeros((n, kp), np.float32)
    xp[:, :k] = x
    y_pad, s_pad = oracle.linear(xp, wp.astype(np.float32), oracle.W_F32, m, kp)
    w = oracle.decode(raw, oracle.W_F16, m, k)
    for t in range(n):
        for j in range(m):
            ref = math.fsum(float(x[t, c]) * float(w[j, c]) for c in range(k))
            assert y_pad[t, j] == pytest.approx(ref, rel=1e-12, abs=1e-12)
            assert s_pad[t, j] == pytest.approx(math.fsum(abs(float(x[t, c]) * float(w[j, c])) for c in range(k)),
                                                rel=1e-12)


def test_pad_weight_refuses_block_types():
    for wtype in (oracle.W_Q8_0, oracle.W_Q4_0):
        with pytest.raises(ValueError):
            oracle.pad_weight(np.zeros(34, np.uint8), wtype, 1, 32)
