"""GPU parity on the method's edge cases, through the C ABI, on every kernel route:

* an output that starts at an arbitrary element of a larger buffer (wavo's
  `gemv_and_embed` test writes the gemv result from offset 3 of its output),
  with canaries on both sides;
* quantized blocks with negative, zero and subnormal f16 scales and the Q8_0
  quant -128 (a scale's sign and -128 are both legal in the block formats;
  the workload generators never draw them);
* activations that are exact bf16 ties (low half 0x8000): the MFMA path must
  round them to nearest even, which ties-away or truncation would not match.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import (B_F32, B_MFMA, ULP_SLACK, assert_within, dev, guarded_at_offset, guarded_out,
                          literal_ratio, oracle_with_tol, read_at_offset, read_guarded)

pytestmark = pytest.mark.gpu

# Routes of the plain layer, as (label, n, m, k, path): the sliced matvec (k % 1024 == 0), the
# general matvec (other k), the matrix-core matvec (Q8_0 / Q4_0, 9..16 tokens, k 2048..4096), the
# bf16-rounded GEMM, the f32-accurate GEMM.
ROUTES = [
    ("sliced", 1, 100, 4096, wq.PATH_AUTO),
    ("sliced-n4", 4, 77, 1024, wq.PATH_AUTO),
    ("general", 2, 70, 96, wq.PATH_AUTO),
    ("mfma-matvec", 12, 50, 2048, wq.PATH_AUTO),
    ("gemm", 70, 130, 256, wq.PATH_MFMA),
    ("gemm-f32", 33, 65, 128, wq.PATH_MFMA_F32),
]


def _bound(path, n):
    if path == wq.PATH_MFMA or (path == wq.PATH_AUTO and n > wq.MATVEC_MAX_N):
        return B_MFMA
    return B_F32


# ---------------------------------------------------------------- y at an offset

@pytest.mark.parametrize("wtype", [wq.W_BF16, wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("label,n,m,k,path", ROUTES)
@pytest.mark.parametrize("residual", [False, True])
def test_output_at_offset_3(wtype, label, n, m, k, path, residual):
    g = synth.rng(61, wtype, n, m, k)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05)
    bias = synth.normal_f32(g, (m,), 0.1)
    y_old = synth.normal_f32(g, (n, m), 1.0) if residual else None
    flags = wq.BIAS | (wq.RESIDUAL if residual else 0)
    buf, out = guarded_at_offset(n, m, 3, y_old)
    assert out.data_ptr() % 16 == 12
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), residual=residual, out=out, path=path)
    got = read_at_offset(buf, n, m, 3)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, _bound(path, n))
    assert_within(got, y_ref, tol, f"{label} y at offset 3")


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("k", [96, 1024, 2048])
def test_moe_output_at_offset_3(gated, k):
    n_tok, n_exp, top_k, m = 5, 3, 2, 40
    g = synth.rng(62, n_tok, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.q8_0_weight(g, m, k) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_at_offset(rows, m, 3)
    wq.moe_matvec(dev(x), dev(bank), wq.W_Q8_0, dev(ids), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_at_offset(buf, rows, m, 3)
    y_ref, S = oracle.moe(x, bank, wq.W_Q8_0, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), f"moe y at offset 3, k={k}")


# ---------------------------------------------------------------- unusual block contents

def _odd_blocks(g, wtype, m, k):
    """Quantized weights whose scales take both signs, zero (both signs) and f16 subnormals, and,
    for Q8_0, quants over the whole int8 range including -128."""
    nb = k // 32
    raw = synth.weight(g, wtype, m, k).reshape(m, nb, -1).copy()
    d = np.abs(synth.normal_f32(g, (m, nb), 0.01)).astype(np.float16).view(np.uint16)
    sign = g.integers(0, 2, (m, nb), dtype=np.uint16) << 15
    d = d | sign
    pick = g.random((m, nb))
    d = np.where(pick < 0.05, sign, d)                                         # +0 / -0
    d = np.where((pick >= 0.05) & (pick < 0.10), sign | g.integers(1, 0x400, (m, nb), dtype=np.uint16), d)
    raw[:, :, 0] = (d & 0xFF).astype(np.uint8)
    raw[:, :, 1] = (d >> 8).astype(np.uint8)
    if wtype == wq.W_Q8_0:
        q = g.integers(-128, 128, (m, nb, 32), dtype=np.int16).astype(np.int8)
        q[:, :, 0] = -128  # every block holds the most negative quant at least once
        raw[:, :, 2:] = q.view(np.uint8)
    return raw.reshape(m, -1)


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
@pytest.mark.parametrize("label,n,m,k,path", ROUTES)
def test_negative_zero_and_subnormal_scales(wtype, label, n, m, k, path):
    g = synth.rng(63, wtype, n, m, k)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _odd_blocks(g, wtype, m, k)
    bias = synth.normal_f32(g, (m,), 0.1)
    flags = wq.BIAS | wq.GELU
    buf, out = guarded_out(n, m)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), gelu=True, out=out, path=path)
    got = read_guarded(buf, n, m)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, None, _bound(path, n))
    assert_within(got, y_ref, tol, f"{label} odd blocks")


@pytest.mark.parametrize("wtype", [wq.W_Q8_0, wq.W_Q4_0])
def test_split_k_route_with_odd_blocks(wtype):
    """Residual without activation on few tiles: the quantized GEMM splits k across workgroups."""
    n, m, k = 40, 64, 2048
    g = synth.rng(64, wtype)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _odd_blocks(g, wtype, m, k)
    bias = synth.normal_f32(g, (m,), 0.1)
    y_old = synth.normal_f32(g, (n, m), 1.0)
    flags = wq.BIAS | wq.RESIDUAL
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), residual=True, out=out)
    got = read_guarded(buf, n, m)
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, B_MFMA)
    assert_within(got, y_ref, tol, "split-k odd blocks")


@pytest.mark.parametrize("k", [96, 1024, 2048])
def test_moe_odd_blocks(k):
    n_tok, n_exp, top_k, m = 6, 4, 2, 48
    for wtype in (wq.W_Q8_0, wq.W_Q4_0):
        g = synth.rng(65, wtype, k)
        x = synth.normal_f32(g, (n_tok, k), 1.0)
        bank = np.stack([_odd_blocks(g, wtype, m, k) for _ in range(n_exp)])
        ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
        buf, out = guarded_out(n_tok, m)
        wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids), dev(gates), n_experts=n_exp, m=m, k=k, out=out)
        got = read_guarded(buf, n_tok, m)
        y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates)
        assert_within(got, y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), f"moe odd blocks wtype={wtype} k={k}")


# ---------------------------------------------------------------- bf16 ties

def _tie_activations(g, n, k):
    """f32 values whose low 16 bits are exactly 0x8000 (half-way between two bf16 values), with
    upper halves of both parities, plus a few just below and above a tie."""
    upper = g.integers(0x3E00, 0x4100, (n, k), dtype=np.uint32)  # |x| in about [0.125, 8)
    upper |= g.integers(0, 2, (n, k), dtype=np.uint32) << 15      # both signs
    low = np.full((n, k), 0x8000, np.uint32)
    near = g.random((n, k))
    low = np.where(near < 0.1, 0x7FFF, np.where(near < 0.2, 0x8001, low))
    return ((upper << 16) | low).view(np.float32)


def _ties_away(x):
    u = x.view(np.uint32).astype(np.uint64)
    return (((u + 0x8000) >> 16) << 16).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("wtype", [wq.W_BF16, wq.W_Q8_0, wq.W_Q4_0])
def test_mfma_rounds_ties_to_even(wtype):
    n, k = 70, 128
    x = _tie_activations(synth.rng(66), n, k)
    rne = (synth.bf16_bits(x).astype(np.uint32) << 16).view(np.float32)
    # The case tells the two rules apart on many elements.
    assert (rne != _ties_away(x)).sum() > n * k // 4
    if wtype == wq.W_BF16:
        w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)  # identity
    else:
        # d = 1.0 (f16 0x3C00); Q8_0 quant 1 on the diagonal, Q4_0 nibble 9 (9 - 8 = 1), else 0 / 8.
        nb = k // 32
        per = 34 if wtype == wq.W_Q8_0 else 18
        w = np.zeros((k, nb, per), np.uint8)
        w[:, :, 0], w[:, :, 1] = 0x00, 0x3C
        for j in range(k):
            b, e = divmod(j, 32)
            if wtype == wq.W_Q8_0:
                w[j, b, 2 + e] = 1
            else:
                w[j, :, 2:] = 0x88
                w[j, b, 2 + (e % 16)] = (0x89 if e < 16 else 0x98)
        w = w.reshape(k, -1)
        assert np.array_equal(oracle.decode(w, wtype, k, k), np.eye(k))
    buf, out = guarded_out(n, k)
    wq.gemm(dev(x), dev(w), wtype, m=k, k=k, out=out, path=wq.PATH_MFMA)
    got = read_guarded(buf, n, k)
    assert np.array_equal(got.view(np.uint32), rne.view(np.uint32))
    # The f32-accurate path returns the activations themselves.
    buf, out = guarded_out(n, k)
    wq.gemm(dev(x), dev(w), wtype, m=k, k=k, out=out, path=wq.PATH_MFMA_F32)
    assert np.array_equal(read_guarded(buf, n, k).view(np.uint32), x.view(np.uint32))
