"""GPU parity of the f32-accurate matrix-core path (WQ_PATH_MFMA_F32) against the f64 oracle.

X enters the matrix cores as three bf16 parts that add up to it exactly, against the exact
weights, so the products are exact and the result is held to the f32 bound, 1e-5 * sum_k |x_k w_k| -- the arithmetic of the
f32 encoder on the cortiq-engine page (nemotron_audio.rs module doc: bf16 weights, f32
accumulation). Covered: every weight type, every tile variant of both GEMM kernels with ragged
edges, every epilogue, the closed-form probe, identity weights, and the encoder's full-size
fc1 / fc2 shapes on sampled frames.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded
from tests.test_gpu_parity import GEMM_SHAPES, TILE_VARIANT_SHAPES, WTYPES, _inputs, _probe, _run

pytestmark = pytest.mark.gpu

F32 = wq.PATH_MFMA_F32


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n,m,k", GEMM_SHAPES)
def test_mfma_f32_parity(wtype, n, m, k):
    flags = [0, 3, 5, 7, 2][(n + m + wtype) % 5]
    x, w, bias, y_old = _inputs(21, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, F32)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"mfma f32 wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("n,m,k,flags", TILE_VARIANT_SHAPES)
def test_mfma_f32_bf16_tile_variants(n, m, k, flags):
    x, w, bias, y_old = _inputs(22, wq.W_BF16, n, m, k, flags)
    got = _run(x, w, wq.W_BF16, m, k, bias, flags, y_old, F32)
    y_ref, tol = oracle_with_tol(x, w, wq.W_BF16, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"mfma f32 bf16 n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("n,m,k,flags", [(2050, 8200, 64, 3), (1100, 2000, 128, 5), (300, 700, 512, 4),
                                         (130, 200, 2048, 7)])
def test_mfma_f32_quantized_tile_variants(wtype, n, m, k, flags):
    """128x256 and 64x128 tiles, with and without the k split (residual without GELU)."""
    x, w, bias, y_old = _inputs(23, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, F32)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"mfma f32 wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("flags", range(8))
def test_mfma_f32_every_flag_combination(wtype, flags):
    n, m, k = 70, 140, 192
    x, w, bias, y_old = _inputs(24, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, F32)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"flags={flags}")


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n", [1, 16, 130])
def test_mfma_f32_closed_form_probe_is_exact(wtype, n):
    m, k = 64, 32
    a, w = _probe(wtype, n, m, k)
    got = _run(a, w, wtype, m, k, None, 0, None, F32)
    want, _ = oracle.linear(a, w, wtype, m, k)
    assert np.array_equal(got, want)


def test_mfma_f32_identity_weight_is_exact():
    """With identity weights the three parts add back to x exactly (bf16(x) alone would not)."""
    k, n = 96, 40
    x = synth.normal_f32(synth.rng(25), (n, k), 1.0)
    w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)
    for wtype, wb in ((wq.W_BF16, w), (wq.W_Q8_0, None)):
        if wb is None:  # the same identity as Q8_0 blocks: d = 1.0, q = 1 on the diagonal
            q = np.eye(k, dtype=np.int8).reshape(k, k // 32, 32)
            wb = np.zeros((k, k // 32, 34), np.uint8)
            wb[:, :, 1] = 0x3C
            wb[:, :, 2:] = q.view(np.uint8)
            wb = wb.reshape(k, -1)
        got = _run(x, wb, wtype, k, k, None, 0, None, F32)
        assert np.array_equal(got, x), f"wtype={wtype}"
    bf = _run(x, w, wq.W_BF16, k, k, None, 0, None, wq.PATH_MFMA)
    assert not np.array_equal(bf, x)


SAMPLE_FRAMES = [0, 1, 63, 64, 777, 1499]


@pytest.mark.parametrize("layer,m,k,flags", [("fc1", 4096, 1024, 3), ("fc2", 1024, 4096, 5)])
def test_mfma_f32_encoder_shapes_full_size(layer, m, k, flags):
    """The encoder's MLP layers at n = 1500 frames (bf16 weights ~N(0, 0.02)), sampled frames."""
    n = 1500
    g = synth.rng(26, m, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.bf16_weight(g, m, k, 0.02)
    bias = synth.normal_f32(g, (m,), 0.1)
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wq.W_BF16, m=m, k=k, bias=dev(bias), gelu=bool(flags & wq.GELU),
            residual=bool(flags & wq.RESIDUAL), out=out, path=F32)
    got = read_guarded(buf, n, m)
    t = np.array(SAMPLE_FRAMES)
    y_ref, tol = oracle_with_tol(x[t], w, wq.W_BF16, m, k, bias, flags, None if y_old is None else y_old[t],
                                 B_F32)
    worst = assert_within(got[t], y_ref, tol, f"encoder {layer} f32 path")
    print(f"{layer}: worst err/tol = {worst:.3f}")
