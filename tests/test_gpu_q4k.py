"""GPU parity of Q4_K weights (hanzo-ml ``matvec_q4k_gpu`` / ``moe_matvec_gpu``) through the C ABI.

The layer and the MoE on Q4_K super-blocks against the f64 oracle: every k class (the sliced kernel
for k a multiple of 1024 up to 8192, the general kernel for every other multiple of 256 and for
dual outputs), 1 to 16 tokens, ragged rows, every epilogue flag, NaN-prefilled outputs with
canaries after them, the MoE with and without gates and with ids outside the bank, and the two
workload-sized cases checked in full.

Bound. A Q4_K weight is the difference of two exact products, ``P = d sc_j q`` and
``N = dmin m_j``; the kernels sum ``x q`` and ``x`` per sub-block and finish with
``d sc_j * sum(x q) - dmin m_j * sum(x)``, so their roundings scale with
``S2 = sum |x| (|P| + |N|)`` rather than ``S = sum |x w|`` (the two differ by the cancellation inside
a sub-block whose weights straddle zero). The f32 path's bound is taken as ``1e-5 * S2``, stretched
by the activation's slope as for the other types; every test also reports the error against
``1e-5 * S`` alone.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import (B_F32, assert_within, dev, guarded_out, literal_ratio, read_guarded,
                          tolerance)

pytestmark = pytest.mark.gpu


def _weight(seed, m, k):
    return synth.q4_k_weight(synth.rng(seed, 5, m, k), m, k)


def _ref_tol(x, w, m, k, bias=None, flags=0, y_old=None, rows=None, alpha=1.0):
    y_ref, S = oracle.linear(x, w, wq.W_Q4_K, m, k, bias, flags, y_old, rows=rows, alpha=alpha)
    S2 = oracle.q4_k_part_scale(x, w, m, k, rows=rows)
    v = None
    if flags & (wq.GELU | 8 | 16 | 32):
        v, _ = oracle.linear(x, w, wq.W_Q4_K, m, k, bias, flags & wq.BIAS, rows=rows)
    b = None if bias is None else (np.asarray(bias)[rows] if rows is not None else bias)
    yo = None
    if y_old is not None:
        yo = np.asarray(y_old, np.float64).reshape(-1, m)
        yo = yo[:, rows] if rows is not None else yo
    return y_ref, S, tolerance(S2, y_ref, B_F32, flags, v, b, yo, alpha)


# ---------------------------------------------------------------- dequantize

@pytest.mark.parametrize("m,k", [(1, 256), (3, 512), (37, 1024), (64, 4096), (5, 2816)])
def test_q4k_dequantize_is_bit_exact(m, k):
    g = synth.rng(70, m, k)
    raw = g.integers(0, 256, (m, k // 256, 144), dtype=np.uint8)
    # d and dmin over every finite f16 (signs, zeros and subnormals included)
    for off in (0, 2):
        f = g.integers(0, 1 << 16, (m, k // 256), dtype=np.uint16)
        f = np.where(((f >> 10) & 0x1F) == 0x1F, f & 0x83FF, f).astype(np.uint16)
        f.flat[0] = 0x8000 if off else 0x0000
        raw[:, :, off] = f & 0xFF
        raw[:, :, off + 1] = f >> 8
    raw = raw.reshape(m, -1)
    got = wq.dequantize(dev(raw), wq.W_Q4_K, m=m, k=k).cpu().numpy()
    # every value d sc q - dmin m is a multiple of 2^-24 below 2^26, so exact in f64; one rounding to f32
    want = oracle.decode_q4_k(raw, m, k).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- the layer

# k classes: 256 .. 768 and 2560, 9216 on the general kernel; 1024 .. 8192 (multiples of 1024) on the sliced one.
@pytest.mark.parametrize("k", [256, 768, 1024, 2560, 4096, 8192, 9216])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 9, 16])
def test_q4k_layer_parity(n, k):
    m = 301
    g = synth.rng(71, n, k)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _weight(72 + n, m, k)
    buf, out = guarded_out(n, m)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, out=out)
    got = read_guarded(buf, n, m)
    y_ref, S, tol = _ref_tol(x, w, m, k)
    r = assert_within(got, y_ref, tol, f"Q4_K n={n} k={k}")
    print(f"Q4_K n={n} k={k}: err/tol {r:.3f}, err/(1e-5 S) {literal_ratio(got, y_ref, S, B_F32):.3f}")


@pytest.mark.parametrize("n,m", [(5, 12288), (8, 12288), (5, 12272), (4, 12288)])
def test_q4k_route_boundary_on_wide_weights(n, m):
    """Plain calls of 5-8 tokens on Q4_K weights with at least three 16-row tiles per CU (12288
    rows on 256 CUs) take the matrix-core kernel; 12272 rows (one tile short) and 4 tokens stay on
    the sliced kernel. Both sides, every output, against the oracle."""
    k = 2048
    print(f"Q4_K wide-weight route n={n} m={m}", flush=True)
    g = synth.rng(79, n, m)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _weight(80, m, k)
    bias = synth.normal_f32(g, (m,), 0.1)
    buf, out = guarded_out(n, m)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, bias=dev(bias), out=out)
    got = read_guarded(buf, n, m)
    y_ref, _, tol = _ref_tol(x, w, m, k, bias, wq.BIAS)
    assert_within(got, y_ref, tol, f"Q4_K wide-weight route n={n} m={m}")


@pytest.mark.parametrize("k", [2560, 4096])
@pytest.mark.parametrize("flags", [wq.BIAS, wq.BIAS | wq.GELU, wq.RESIDUAL, wq.BIAS | wq.GELU | wq.RESIDUAL])
@pytest.mark.parametrize("n", [1, 4, 13])
def test_q4k_epilogue(n, k, flags):
    m = 200
    g = synth.rng(73, n, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _weight(74, m, k)
    bias = synth.normal_f32(g, (m,), 0.1) if flags & wq.BIAS else None
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, bias=None if bias is None else dev(bias),
            gelu=bool(flags & wq.GELU), residual=bool(flags & wq.RESIDUAL), out=out)
    got = read_guarded(buf, n, m)
    y_ref, _, tol = _ref_tol(x, w, m, k, bias, flags, y_old)
    assert_within(got, y_ref, tol, f"Q4_K flags={flags} n={n} k={k}")


@pytest.mark.parametrize("act", ["silu", "relu", "tanh"])
def test_q4k_activations_and_alpha(act):
    n, m, k = 3, 150, 1024
    flag = {"silu": 8, "relu": 16, "tanh": 32}[act]
    g = synth.rng(75, flag)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _weight(76, m, k)
    bias = synth.normal_f32(g, (m,), 0.1)
    y_old = synth.normal_f32(g, (n, m), 1.0)
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, bias=dev(bias), act=act, residual=True, out=out, alpha=0.75)
    got = read_guarded(buf, n, m)
    flags = wq.BIAS | flag | wq.RESIDUAL
    y_ref, _, tol = _ref_tol(x, w, m, k, bias, flags, y_old, alpha=0.75)
    assert_within(got, y_ref, tol, f"Q4_K {act}")


@pytest.mark.parametrize("k", [1024, 2816])
def test_q4k_dual_outputs(k):
    n, m, dual = 2, 120, 50
    g = synth.rng(77, k)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = _weight(78, m, k)
    bias = synth.normal_f32(g, (m + dual,), 0.1)
    buf, out = guarded_out(n, m + dual)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, bias=dev(bias), gelu=True, out=out, dual=dual)
    got = read_guarded(buf, n, m + dual)
    y_ref, S = oracle.linear_dual(x, w, wq.W_Q4_K, m, k, dual, bias, wq.BIAS | wq.GELU)
    S2 = oracle.q4_k_part_scale(x, w, m, k)
    S2 = np.concatenate([S2, S2[:, :dual]], axis=1)
    v, _ = oracle.linear_dual(x, w, wq.W_Q4_K, m, k, dual, bias, wq.BIAS)
    tol = tolerance(S2, y_ref, B_F32, wq.BIAS | wq.GELU, v, bias)
    assert_within(got, y_ref, tol, f"Q4_K dual k={k}")


def test_q4k_rows_beyond_one_launch_and_repeatable():
    # 70,001 rows at k = 1024 (sliced) and 1280 (general): runs of tiles per workgroup, the last one
    # ragged; sampled rows from the first, middle and last tiles, and bit-identical repeats.
    for k in (1024, 1280):
        n, m = 2, 70001
        g = synth.rng(79, k)
        x = synth.normal_f32(g, (n, k), 1.0)
        w = _weight(80, m, k)
        buf, out = guarded_out(n, m)
        xd, wd = dev(x), dev(w)
        wq.gemm(xd, wd, wq.W_Q4_K, m=m, k=k, out=out)
        got = read_guarded(buf, n, m)
        assert np.isfinite(got).all()
        rows = np.r_[0:40, 35000:35040, m - 40:m]
        y_ref, _, tol = _ref_tol(x, w, m, k, rows=rows)
        assert_within(got[:, rows], y_ref, tol, f"Q4_K 70001 rows k={k}")
        again = wq.gemm(xd, wd, wq.W_Q4_K, m=m, k=k).cpu().numpy()
        assert np.array_equal(again.view(np.uint32), got.view(np.uint32))


# ---------------------------------------------------------------- MoE

def _moe_part_scale(x, bank, ids, m, k, rows=None):
    """S2 of every routed slot, ``[n_tok][top_k][rows]``: each expert's parts decoded once."""
    n_tok, top_k = ids.shape
    width = m if rows is None else len(rows)
    s2 = np.zeros((n_tok, top_k, width))
    for e in np.unique(ids):
        if not 0 <= e < bank.shape[0]:
            continue
        per_tok = oracle.q4_k_part_scale(x, bank[e], m, k, rows=rows)
        t_idx, j_idx = np.nonzero(ids == e)
        s2[t_idx, j_idx] = per_tok[t_idx]
    return s2


@pytest.mark.parametrize("k", [4096, 2560])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("n_tok,n_exp,top_k", [(1, 8, 2), (16, 8, 2), (5, 3, 3), (64, 64, 2)])
def test_q4k_moe(n_tok, n_exp, top_k, k, gated):
    m = 260
    g = synth.rng(81, n_tok, n_exp, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([_weight(82 + e, m, k) for e in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    rows_out = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows_out, m)
    wq.moe_matvec(dev(x), dev(bank), wq.W_Q4_K, dev(ids), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, rows_out, m)
    y_ref, S = oracle.moe(x, bank, wq.W_Q4_K, ids, n_exp, m, k, gates if gated else None)
    s2 = _moe_part_scale(x, bank, ids, m, k)
    S2 = (np.abs(gates)[:, :, None] * s2).sum(axis=1) if gated else s2.reshape(n_tok * top_k, m)
    tol = B_F32 * S2 + 8 * 2.0 ** -24 * np.abs(y_ref)
    assert_within(got, y_ref, tol, f"Q4_K MoE {n_tok}x top-{top_k} of {n_exp} k={k} gated={gated}")


@pytest.mark.parametrize("k", [4096, 2560])
def test_q4k_moe_out_of_range_ids_give_nan(k):
    n_tok, top_k, n_exp, m = 4, 2, 4, 130
    g = synth.rng(83, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([_weight(84 + e, m, k) for e in range(n_exp)])
    ids, _ = synth.moe_routing(g, n_tok, n_exp, top_k)
    ids[1, 0] = -1
    ids[2, 1] = n_exp
    buf, out = guarded_out(n_tok * top_k, m)
    wq.moe_matvec(dev(x), dev(bank), wq.W_Q4_K, dev(ids), None, n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, n_tok * top_k, m)
    bad = {2, 5}  # slots (1, 0) and (2, 1)
    assert np.isnan(got[sorted(bad)]).all()
    good = [s for s in range(n_tok * top_k) if s not in bad]
    ids_ok = ids.copy()
    ids_ok[1, 0] = 0
    ids_ok[2, 1] = 0
    y_ref, _ = oracle.moe(x, bank, wq.W_Q4_K, ids_ok, n_exp, m, k)
    tol = B_F32 * _moe_part_scale(x, bank, ids_ok, m, k).reshape(n_tok * top_k, m) + 8 * 2.0 ** -24 * np.abs(y_ref)
    assert_within(got[good], y_ref[good], tol[good], "Q4_K MoE in-range slots")


# ---------------------------------------------------------------- workload-sized, checked in full

def test_q4k_matvec_14336x4096_full():
    """Q4_K 14336 x 4096 at one token (the Q4_0 matvec workload's shape on Q4_K): every output."""
    m, k = 14336, 4096
    g = synth.rng(85)
    x = synth.normal_f32(g, (1, k), 1.0)
    w = _weight(86, m, k)
    buf, out = guarded_out(1, m)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, out=out)
    got = read_guarded(buf, 1, m)
    worst, lit = 0.0, 0.0
    for r0 in range(0, m, 2048):
        rows = np.arange(r0, min(m, r0 + 2048))
        y_ref, S, tol = _ref_tol(x, w, m, k, rows=rows)
        worst = max(worst, assert_within(got[:, rows], y_ref, tol, f"rows {r0}.."))
        lit = max(lit, literal_ratio(got[:, rows], y_ref, S, B_F32))
    print(f"Q4_K 14336x4096 n=1: err/tol {worst:.3f}, err/(1e-5 S) {lit:.3f}")


def test_q4k_moe_16_tokens_top2_of_8_full():
    """16 tokens, top-2 of 8 Q4_K experts of 14336 x 4096, gated: every output."""
    n_tok, top_k, n_exp, m, k = 16, 2, 8, 14336, 4096
    g = synth.rng(87)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([_weight(88 + e, m, k) for e in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    buf, out = guarded_out(n_tok, m)
    wq.moe_matvec(dev(x), dev(bank), wq.W_Q4_K, dev(ids), dev(gates), n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, n_tok, m)
    worst = 0.0
    for r0 in range(0, m, 2048):
        rows = np.arange(r0, min(m, r0 + 2048))
        y_ref, _ = oracle.moe(x, bank, wq.W_Q4_K, ids, n_exp, m, k, gates, rows=rows)
        s2 = (np.abs(gates)[:, :, None] * _moe_part_scale(x, bank, ids, m, k, rows=rows)).sum(axis=1)
        tol = B_F32 * s2 + 8 * 2.0 ** -24 * np.abs(y_ref)
        worst = max(worst, assert_within(got[:, rows], y_ref, tol, f"rows {r0}.."))
    print(f"Q4_K MoE 16 tok top-2 of 8: err/tol {worst:.3f}")


# ---------------------------------------------------------------- seeded random sweep

Q4K_K = [256, 512, 768, 1024, 1280, 2048, 2304, 2560, 3072, 4096, 5120, 8192, 9216]
ACTS = [None, "gelu", "silu", "relu", "tanh"]
ACT_FLAG = {None: 0, "gelu": 2, "silu": 8, "relu": 16, "tanh": 32}


@pytest.mark.parametrize("i", range(40))
def test_q4k_random_layer(i):
    g = np.random.default_rng(5000 + i)
    k = int(g.choice(Q4K_K))
    n = int(g.integers(1, 17))
    m = int(g.integers(1, 300))
    act = ACTS[int(g.integers(0, 5))]
    bias_on, res_on = bool(g.integers(0, 2)), bool(g.integers(0, 2))
    alpha = float(g.choice([1.0, 0.5, -1.25]))
    dual = int(g.integers(0, m + 1)) if g.integers(0, 4) == 0 else 0
    gs = synth.rng(5100, i)
    x = synth.normal_f32(gs, (n, k), 1.0)
    w = _weight(5200 + i, m, k)
    bias = synth.normal_f32(gs, (m + dual,), 0.1) if bias_on else None
    y_old = synth.normal_f32(gs, (n, m + dual), 1.0) if res_on else None
    buf, out = guarded_out(n, m + dual, y_old)
    wq.gemm(dev(x), dev(w), wq.W_Q4_K, m=m, k=k, bias=None if bias is None else dev(bias), act=act,
            residual=res_on, out=out, alpha=alpha, dual=dual)
    got = read_guarded(buf, n, m + dual)
    flags = (wq.BIAS if bias_on else 0) | ACT_FLAG[act] | (wq.RESIDUAL if res_on else 0)
    y_ref, _ = oracle.linear_dual(x, w, wq.W_Q4_K, m, k, dual, bias, flags, y_old, alpha=alpha)
    v = None
    if ACT_FLAG[act]:
        v, _ = oracle.linear_dual(x, w, wq.W_Q4_K, m, k, dual, bias, flags & wq.BIAS)
    S2 = oracle.q4_k_part_scale(x, w, m, k)
    S2 = np.concatenate([S2, S2[:, :dual]], axis=1)
    tol = tolerance(S2, y_ref, B_F32, flags, v, bias, y_old, alpha)
    assert_within(got, y_ref, tol, f"case {i}: n={n} m={m} k={k} act={act} bias={bias_on} res={res_on} "
                                   f"alpha={alpha} dual={dual}")


@pytest.mark.parametrize("i", range(16))
def test_q4k_random_moe(i):
    g = np.random.default_rng(6000 + i)
    k = int(g.choice([256, 1024, 2048, 2304, 3072, 4096, 5120]))
    n_exp = int(g.integers(1, 9))
    top_k = int(g.integers(1, min(n_exp, 4) + 1))
    n_tok = int(g.integers(1, 40))
    m = int(g.integers(1, 200))
    gated = bool(g.integers(0, 2))
    gs = synth.rng(6100, i)
    x = synth.normal_f32(gs, (n_tok, k), 1.0)
    bank = np.stack([_weight(6200 + 16 * i + e, m, k) for e in range(n_exp)])
    ids, gates = synth.moe_routing(gs, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wq.W_Q4_K, dev(ids), dev(gates) if gated else None, n_experts=n_exp, m=m, k=k,
                  out=out)
    got = read_guarded(buf, rows, m)
    y_ref, _ = oracle.moe(x, bank, wq.W_Q4_K, ids, n_exp, m, k, gates if gated else None)
    s2 = _moe_part_scale(x, bank, ids, m, k)
    S2 = (np.abs(gates)[:, :, None] * s2).sum(axis=1) if gated else s2.reshape(n_tok * top_k, m)
    assert_within(got, y_ref, B_F32 * S2 + 8 * 2.0 ** -24 * np.abs(y_ref),
                  f"moe case {i}: n_tok={n_tok} n_exp={n_exp} top_k={top_k} m={m} k={k} gated={gated}")
