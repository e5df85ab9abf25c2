"""GPU parity: the HIP path (through the C ABI) against the f64 oracle.

Small shapes span several tiles and ragged tails; every weight type, both
paths, the epilogue flags, NaN-prefilled outputs (every element must be
written) and a canary region after the output (nothing written past it).
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import (B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol,
                          read_guarded)

pytestmark = pytest.mark.gpu

WTYPES = [wq.W_BF16, wq.W_Q8_0, wq.W_Q4_0]


def _inputs(seed, wtype, n, m, k, flags):
    g = synth.rng(seed, wtype, n, m, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05, dsigma=0.01)
    bias = synth.normal_f32(g, (m,), 0.1) if flags & wq.BIAS else None
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    return x, w, bias, y_old


def _run(x, w, wtype, m, k, bias, flags, y_old, path):
    n = x.shape[0]
    buf, out = guarded_out(n, m, y_old if flags & wq.RESIDUAL else None)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=None if bias is None else dev(bias),
            gelu=bool(flags & wq.GELU), residual=bool(flags & wq.RESIDUAL), out=out, path=path)
    return read_guarded(buf, n, m)


# ---------------------------------------------------------------- dequantize

def _random_weight_bytes(g, wtype, m, k):
    """Random weights over every finite f16 scale (subnormals, zeros, signs included)."""
    if wtype == wq.W_BF16:
        bits = g.integers(0, 1 << 16, (m, k), dtype=np.uint16)
        exp = (bits >> 7) & 0xFF
        return np.where(exp == 0xFF, bits & 0x807F, bits).astype(np.uint16)
    raw = synth.weight(g, wtype, m, k).reshape(m, k // 32, -1).copy()
    raw[:, :, 2:] = g.integers(0, 256, raw[:, :, 2:].shape, dtype=np.uint8)
    d = g.integers(0, 1 << 16, (m, k // 32), dtype=np.uint16)
    d = np.where(((d >> 10) & 0x1F) == 0x1F, d & 0x83FF, d).astype(np.uint16)
    d[0, 0] = 0x0000
    if d.size > 1:
        d.flat[1] = 0x8000
    raw[:, :, 0] = d & 0xFF
    raw[:, :, 1] = d >> 8
    return raw.reshape(m, -1)


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("m,k", [(1, 32), (3, 32), (37, 96), (64, 4096), (5, 4128)])
def test_dequantize_is_bit_exact(wtype, m, k):
    g = synth.rng(7, wtype, m, k)
    raw = _random_weight_bytes(g, wtype, m, k)
    buf, out = guarded_out(m, k)
    wq.dequantize(dev(raw), wtype, m=m, k=k, out=out)
    got = read_guarded(buf, m, k)
    want = oracle.decode(raw, wtype, m, k).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- matvec path (f32)

MV_SHAPES = [(1, 32), (37, 96), (130, 4096), (67, 4128), (21, 8224)]


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 16])
@pytest.mark.parametrize("m,k", MV_SHAPES)
def test_matvec_parity(wtype, n, m, k):
    flags = [0, 1, 3, 7, 4, 6][(n + m) % 6]
    x, w, bias, y_old = _inputs(1, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_MATVEC)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"matvec wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("flags", range(8))
def test_matvec_every_flag_combination(flags):
    wtype, n, m, k = wq.W_Q8_0, 3, 70, 256
    x, w, bias, y_old = _inputs(2, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"flags={flags}")


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("n", [9, 16])
@pytest.mark.parametrize("flags", range(8))
def test_matvec_matrix_core_route_every_flag(wtype, n, flags):
    """Plain calls with 9-16 tokens on Q8_0 / Q4_0 (k 2048-4096) take the matrix-core kernel
    (exact three-part activations), which then applies the epilogue itself."""
    m, k = 75, 2048
    x, w, bias, y_old = _inputs(16, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"matrix-core matvec wtype={wtype} n={n} flags={flags}")


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("n,m", [(5, 8192), (8, 8192), (5, 8176), (4, 8192)])
def test_matvec_route_boundary_on_wide_weights(wtype, n, m):
    """Plain calls of 5-8 tokens on weights with at least two 16-row tiles per CU (8192 rows on
    256 CUs) take the matrix-core kernel; 8176 rows (one tile short) and 4 tokens stay on the f32
    FMA kernel. Both sides of the boundary, every output, against the oracle."""
    k = 2048
    flags = 7 if n == 8 else 1
    print(f"wide-weight route wtype={wtype} n={n} m={m}", flush=True)
    x, w, bias, y_old = _inputs(17, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"wide-weight route wtype={wtype} n={n} m={m}")


# ---------------------------------------------------------------- MFMA path (bf16 x, exact w)

GEMM_SHAPES = [(17, 1, 32), (64, 37, 96), (130, 128, 256), (200, 288, 160), (257, 130, 1024)]


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n,m,k", GEMM_SHAPES)
def test_gemm_parity(wtype, n, m, k):
    flags = [0, 3, 5, 7, 2][(n + m + wtype) % 5]
    x, w, bias, y_old = _inputs(3, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_MFMA)
    assert_within(got, y_ref, tol, f"gemm wtype={wtype} n={n} m={m} k={k} flags={flags}")


# Shapes that take each bf16 tile variant of the GEMM (on a 256-CU MI355X), all with ragged
# edges: 128x256 tiles (one per CU or more), 64x128 tiles two per CU, 64x192 tiles two per CU,
# 64x64 tiles, and 64x128 tiles with a 4-slot ring (few tiles, long k; every epilogue).
TILE_VARIANT_SHAPES = [(2050, 4100, 128, 5), (1100, 2000, 64, 3), (1500, 3000, 64, 3), (1530, 2900, 192, 5),
                       (700, 1000, 192, 1), (1000, 2000, 1088, 7), (1000, 2000, 1088, 5), (900, 2040, 2048, 4)]


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("n,m,k,flags", [(2050, 8200, 64, 3), (1100, 2000, 128, 5), (300, 700, 512, 4)])
def test_gemm_quantized_tile_variants(wtype, n, m, k, flags):
    """Quantized weights on the matrix cores: 128x256 tiles (two per CU or more) and 64x128 tiles
    (with and without the k split), ragged edges."""
    x, w, bias, y_old = _inputs(17, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_MFMA)
    assert_within(got, y_ref, tol, f"gemm wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("n,m,k,flags", TILE_VARIANT_SHAPES)
def test_gemm_bf16_tile_variants(n, m, k, flags):
    x, w, bias, y_old = _inputs(15, wq.W_BF16, n, m, k, flags)
    got = _run(x, w, wq.W_BF16, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wq.W_BF16, m, k, bias, flags, y_old, B_MFMA)
    assert_within(got, y_ref, tol, f"gemm bf16 n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("flags", range(8))
def test_gemm_every_flag_combination(flags):
    wtype, n, m, k = wq.W_Q4_0, 70, 140, 192
    x, w, bias, y_old = _inputs(4, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_AUTO)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_MFMA)
    assert_within(got, y_ref, tol, f"flags={flags}")


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n", [1, 5, 16])
def test_mfma_path_forced_at_small_n(wtype, n):
    m, k = 45, 320
    x, w, bias, y_old = _inputs(5, wtype, n, m, k, 1)
    got = _run(x, w, wtype, m, k, bias, 1, y_old, wq.PATH_MFMA)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, 1, y_old, B_MFMA)
    assert_within(got, y_ref, tol)


# ---------------------------------------------------------------- exact cases

def _probe(wtype, n=130, m=64, k=32):
    r = np.arange(n)[:, None]
    a = (np.arange(k)[None, :] + r % 32).astype(np.float32)
    ones = np.arange(k)[None, :] == (np.arange(m) % 32)[:, None]
    if wtype == wq.W_BF16:
        w = np.where(ones, 0x3F80, 0).astype(np.uint16)
    elif wtype == wq.W_Q8_0:
        w = np.zeros((m, 34), np.uint8)
        w[:, 1] = 0x3C
        w[:, 2:] = ones
    else:
        q = np.where(ones, 9, 8)
        w = np.zeros((m, 18), np.uint8)
        w[:, 1] = 0x3C
        w[:, 2:] = q[:, :16] | (q[:, 16:] << 4)
    return a, w


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("path,n", [(wq.PATH_MFMA, 130), (wq.PATH_MATVEC, 16), (wq.PATH_MATVEC, 1)])
def test_closed_form_probe_is_exact(wtype, path, n):
    m, k = 64, 32
    a, w = _probe(wtype, n, m, k)
    got = _run(a, w, wtype, m, k, None, 0, None, path)
    want, _ = oracle.linear(a, w, wtype, m, k)
    assert np.array_equal(got, want)


def test_identity_weight():
    import torch
    k, n = 96, 40
    x = synth.normal_f32(synth.rng(8), (n, k), 1.0)
    w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)
    got = _run(x, w, wq.W_BF16, k, k, None, 0, None, wq.PATH_MFMA)
    assert np.array_equal(got, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    got = _run(x[:16], w, wq.W_BF16, k, k, None, 0, None, wq.PATH_MATVEC)
    assert np.array_equal(got, x[:16])


@pytest.mark.parametrize("path", [wq.PATH_MATVEC, wq.PATH_MFMA])
def test_gelu_epilogue_alone(path):
    """With identity bf16 weights and bf16-exact activations (j/32, |j| < 256) the pre-activation
    is exact on both paths, so all that is left is the epilogue's erf-GELU. It is held to the f32
    rounding slack alone, against the exact erf."""
    from tests.parity import ULP_SLACK
    n, k = 4, 128
    j = np.arange(-255, 257, dtype=np.float64)  # 512 values in [-7.97, 8.0]
    x = (j / 32.0).astype(np.float32).reshape(n, k)
    w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)
    got = _run(x, w, wq.W_BF16, k, k, None, int(wq.GELU), None, path)
    v = x.astype(np.float64)
    y_ref = oracle.gelu_erf(v)
    assert_within(got, y_ref, ULP_SLACK * (np.abs(v) + np.abs(y_ref)) + 1e-30, f"gelu alone path={path}")


def test_zero_sized_calls_leave_output_alone():
    import torch
    x = torch.zeros(0, 32, device="cuda")
    w = torch.zeros(8, 32, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(0, 8, device="cuda")
    assert wq.gemm(x, w, wq.W_BF16, m=8, k=32, out=out).shape == (0, 8)


# ---------------------------------------------------------------- MoE

def _moe_inputs(seed, wtype, n_tok, n_exp, top_k, m, k):
    g = synth.rng(seed, wtype, n_tok, n_exp, top_k, m, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    return x, bank, ids, gates


def _run_moe(x, bank, wtype, ids, gates, n_exp, m, k):
    n_tok, top_k = ids.shape
    rows = n_tok if gates is not None else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids.astype(np.int32)),
                  None if gates is None else dev(gates), n_experts=n_exp, m=m, k=k, out=out)
    return read_guarded(buf, rows, m)


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n_tok,n_exp,top_k", [(1, 8, 2), (16, 4, 2), (5, 6, 3), (40, 8, 1), (64, 3, 3)])
@pytest.mark.parametrize("gated", [False, True])
def test_moe_parity(wtype, n_tok, n_exp, top_k, gated):
    m, k = 75, 160
    x, bank, ids, gates = _moe_inputs(9, wtype, n_tok, n_exp, top_k, m, k)
    got = _run_moe(x, bank, wtype, ids, gates if gated else None, n_exp, m, k)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), "moe")


def test_moe_out_of_range_ids_give_nan_and_leave_other_slots_right():
    wtype, n_tok, n_exp, top_k, m, k = wq.W_Q4_0, 6, 4, 2, 50, 64
    x, bank, ids, gates = _moe_inputs(10, wtype, n_tok, n_exp, top_k, m, k)
    bad = ids.copy()
    bad[2, 1] = 7
    bad[4, 0] = -1
    got = _run_moe(x, bank, wtype, bad, None, n_exp, m, k)
    assert np.isnan(got[2 * 2 + 1]).all() and np.isnan(got[4 * 2 + 0]).all()
    ok = [s for s in range(n_tok * top_k) if s not in (5, 8)]
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k)
    assert_within(got[ok], y_ref[ok], B_F32 * S[ok] + 1e-12, "moe valid slots")
    gated = _run_moe(x, bank, wtype, bad, gates, n_exp, m, k)
    assert np.isnan(gated[2]).all() and np.isnan(gated[4]).all()
    assert np.isfinite(gated[[0, 1, 3, 5]]).all()


def test_moe_all_tokens_on_one_expert_equals_the_16_row_layer():
    wtype, n_tok, n_exp, m, k = wq.W_Q8_0, 16, 4, 90, 128
    x, bank, _, _ = _moe_inputs(11, wtype, n_tok, n_exp, 1, m, k)
    ids = np.full((n_tok, 1), 3, np.int32)
    got = _run_moe(x, bank, wtype, ids, None, n_exp, m, k)
    y_ref, S = oracle.linear(x, bank[3], wtype, m, k)
    assert_within(got, y_ref, B_F32 * S + 1e-12)


# ---------------------------------------------------------------- sliced matvec kernel (k % 1024 == 0)

SLICED_SHAPES = [(1, 1024), (17, 2048), (100, 3072), (33, 8192), (530, 4096)]


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("m,k", SLICED_SHAPES)
def test_matvec_sliced_parity(wtype, n, m, k):
    flags = [0, 1, 3, 7, 4, 6][(n + m + wtype) % 6]
    x, w, bias, y_old = _inputs(12, wtype, n, m, k, flags)
    got = _run(x, w, wtype, m, k, bias, flags, y_old, wq.PATH_MATVEC)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_F32)
    assert_within(got, y_ref, tol, f"sliced wtype={wtype} n={n} m={m} k={k} flags={flags}")


@pytest.mark.parametrize("wtype", WTYPES)
@pytest.mark.parametrize("n_tok,n_exp,top_k,m,k", [(16, 4, 2, 75, 1024), (1, 8, 2, 300, 4096),
                                                   (40, 3, 1, 64, 2048), (7, 5, 3, 129, 8192)])
@pytest.mark.parametrize("gated", [False, True])
def test_moe_sliced_parity(wtype, n_tok, n_exp, top_k, m, k, gated):
    x, bank, ids, gates = _moe_inputs(13, wtype, n_tok, n_exp, top_k, m, k)
    got = _run_moe(x, bank, wtype, ids, gates if gated else None, n_exp, m, k)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), "moe sliced")


def test_moe_sliced_out_of_range_ids():
    wtype, n_tok, n_exp, top_k, m, k = wq.W_Q8_0, 6, 4, 2, 50, 1024
    x, bank, ids, gates = _moe_inputs(14, wtype, n_tok, n_exp, top_k, m, k)
    bad = ids.copy()
    bad[1, 0] = 4
    got = _run_moe(x, bank, wtype, bad, None, n_exp, m, k)
    assert np.isnan(got[2]).all()
    ok = [s for s in range(n_tok * top_k) if s != 2]
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k)
    assert_within(got[ok], y_ref[ok], B_F32 * S[ok] + 1e-12, "moe sliced valid slots")


# ---------------------------------------------------------------- MoE on matrix cores (Q8_0 / Q4_0, k in 2048..4096)

@pytest.mark.gpu
@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("n_tok,n_exp,top_k,m,k", [
    (16, 8, 2, 75, 4096),   # the C4 routing shape at a ragged m
    (64, 2, 1, 33, 2048),   # ~32 slots per expert: several passes of 16
    (20, 3, 2, 129, 3072),  # six waves: uneven rows per wave
    (5, 6, 3, 1, 4096),     # one row
    (3, 4, 1, 16, 2560),    # five waves, one full tile
])
@pytest.mark.parametrize("gated", [False, True])
def test_moe_mfma_parity(wtype, n_tok, n_exp, top_k, m, k, gated):
    print(f"moe mfma wtype={wtype} n_tok={n_tok} n_exp={n_exp} top_k={top_k} m={m} k={k} gated={gated}", flush=True)
    x, bank, ids, gates = _moe_inputs(15, wtype, n_tok, n_exp, top_k, m, k)
    got = _run_moe(x, bank, wtype, ids, gates if gated else None, n_exp, m, k)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), "moe mfma")


@pytest.mark.gpu
def test_moe_mfma_out_of_range_ids():
    wtype, n_tok, n_exp, top_k, m, k = wq.W_Q4_0, 6, 4, 2, 70, 4096
    x, bank, ids, gates = _moe_inputs(16, wtype, n_tok, n_exp, top_k, m, k)
    bad = ids.copy()
    bad[0, 1] = 9
    bad[3, 0] = -2
    got = _run_moe(x, bank, wtype, bad, None, n_exp, m, k)
    assert np.isnan(got[1]).all() and np.isnan(got[6]).all()
    ok = [s for s in range(n_tok * top_k) if s not in (1, 6)]
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k)
    assert_within(got[ok], y_ref[ok], B_F32 * S[ok] + 1e-12, "moe mfma valid slots")
