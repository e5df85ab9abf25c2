"""GPU parity of the f32 and f16 weight types (wavo `Linear` GEMM types 0 and 1) against the f64
oracle: exact decode through wq_dequantize, the f32 paths (general and k-sliced matvec kernels,
the MoE over such banks) and the matrix cores, where each weight enters as two (f16) or three
(f32) exact bf16 parts, on both the bf16(X) and the f32-accurate path, with every epilogue and
ragged tiles.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded
from tests.test_gpu_parity import _inputs, _run

pytestmark = pytest.mark.gpu

PLAIN = [wq.W_F32, wq.W_F16]


def _random_bits(g, wtype, m, k):
    """Random finite bit patterns of the type, subnormals and signed zeros included."""
    if wtype == wq.W_F32:
        bits = g.integers(0, 1 << 32, (m, k), dtype=np.uint64).astype(np.uint32)
        exp = (bits >> 23) & 0xFF
        bits = np.where(exp == 0xFF, bits & 0x807FFFFF, bits).astype(np.uint32)
    else:
        bits = g.integers(0, 1 << 16, (m, k), dtype=np.uint16)
        exp = (bits >> 10) & 0x1F
        bits = np.where(exp == 0x1F, bits & 0x83FF, bits).astype(np.uint16)
    bits.flat[0] = 0
    bits.flat[1] = 0x80000000 if wtype == wq.W_F32 else 0x8000
    return bits


@pytest.mark.parametrize("wtype", PLAIN)
@pytest.mark.parametrize("m,k", [(1, 32), (37, 96), (64, 4096), (5, 4128)])
def test_dequantize_is_bit_exact(wtype, m, k):
    raw = _random_bits(synth.rng(41, wtype, m, k), wtype, m, k)
    buf, out = guarded_out(m, k)
    wq.dequantize(dev(raw), wtype, m=m, k=k, out=out)
    got = read_guarded(buf, m, k)
    want = oracle.decode(raw, wtype, m, k).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("wtype", PLAIN)
@pytest.mark.parametrize("n", [1, 2, 4, 7, 16])
@pytest.mark.parametrize("m,k", [(37, 96), (67, 4128), (130, 4096), (33, 8192), (100, 3072)])
def test_matvec_parity(wtype, n, m, k):
    flags = [0, 1, 3, 7, 4, 6][(n + m + wtype) % 6]
    x, w, bias, y_old = _inputs(42, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_MATVEC)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"matvec wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("wtype", PLAIN)
@pytest.mark.parametrize("path,bound", [(wq.PATH_MFMA, B_MFMA), (wq.PATH_MFMA_F32, B_F32)])
@pytest.mark.parametrize("n,m,k", [(17, 1, 32), (64, 37, 96), (130, 128, 256), (200, 288, 160), (257, 130, 1024),
                                   (1100, 2000, 128)])
def test_gemm_parity(wtype, path, bound, n, m, k):
    flags = [0, 3, 5, 7, 2][(n + m + wtype) % 5]
    x, w, bias, y_old = _inputs(43, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, path)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound)
    assert_within(got, y_ref, tol, f"gemm wtype={wtype} path={path} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("wtype", PLAIN)
@pytest.mark.parametrize("flags", range(8))
def test_gemm_every_flag_combination(wtype, flags):
    n, m, k = 70, 140, 192
    x, w, bias, y_old = _inputs(44, wtype, n, m, k, flags)
    for path, bound in ((wq.PATH_MFMA, B_MFMA), (wq.PATH_MFMA_F32, B_F32)):
        got = _run(x, w, wtype, m, k, bias, flags, y_old, path)
        y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound)
        assert_within(got, y_ref, tol, f"wtype={wtype} flags={flags} path={path}")


@pytest.mark.parametrize("wtype", PLAIN)
def test_weights_enter_the_matrix_cores_exactly(wtype):
    """X = identity: every output is one weight times 1, so y == the weight on both matrix-core
    paths (bf16 rounding of the weight would show)."""
    m, k = 40, 96
    g = synth.rng(45, wtype)
    w = synth.weight(g, wtype, m, k, sigma=0.3)
    x = np.eye(k, dtype=np.float32)
    want = oracle.decode(w, wtype, m, k).T.astype(np.float32)
    for path in (wq.PATH_MFMA, wq.PATH_MFMA_F32):
        got = _run(x, w, wtype, m, k, None, 0, None, path)
        assert np.array_equal(got, want), f"path={path}"


@pytest.mark.parametrize("wtype", PLAIN)
@pytest.mark.parametrize("n_tok,n_exp,top_k,m,k", [(16, 4, 2, 75, 1024), (5, 6, 3, 70, 160), (7, 5, 3, 129, 8192)])
@pytest.mark.parametrize("gated", [False, True])
def test_moe_parity(wtype, n_tok, n_exp, top_k, m, k, gated):
    g = synth.rng(46, wtype, n_tok, n_exp, top_k, m, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids.astype(np.int32)), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), "moe")
