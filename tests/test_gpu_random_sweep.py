"""Seeded random sweep of the layer and the MoE matvec through the C ABI, against the oracle.

Each case draws a weight type, sizes (ragged against every tile and slice size the kernels
use), epilogue flags and a path from a fixed seed, so a failure names a reproducible case. The
shapes stay small enough for the f64 oracle to finish in well under a second each.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded

pytestmark = pytest.mark.gpu

WTYPES = [wq.W_BF16, wq.W_Q8_0, wq.W_Q4_0]
# k values: multiples of 32 that hit the general kernel, the sliced kernel (multiples of 1024), the
# matrix-core kernel (multiples of 512 in 2048..4096) and both GEMM k steps (32 and 64).
K_CHOICES = [32, 96, 160, 512, 1024, 1056, 2048, 2560, 3072, 4096, 5120]


def _layer_case(i):
    g = np.random.default_rng(1000 + i)
    wtype = WTYPES[i % 3]
    k = int(g.choice(K_CHOICES))
    path = [wq.PATH_AUTO, wq.PATH_MATVEC, wq.PATH_MFMA][int(g.integers(0, 3))]
    n = int(g.integers(1, 17)) if path == wq.PATH_MATVEC else int(g.integers(1, 200))
    m = int(g.integers(1, 300))
    flags = int(g.integers(0, 8))
    return wtype, n, m, k, flags, path


@pytest.mark.parametrize("i", range(48))
def test_random_layer(i):
    wtype, n, m, k, flags, path = _layer_case(i)
    g = synth.rng(77, i)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05, dsigma=0.01)
    bias = synth.normal_f32(g, (m,), 0.1) if flags & wq.BIAS else None
    y_old = synth.normal_f32(g, (n, m), 1.0) if flags & wq.RESIDUAL else None
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=None if bias is None else dev(bias),
            gelu=bool(flags & wq.GELU), residual=bool(flags & wq.RESIDUAL), out=out, path=path)
    got = read_guarded(buf, n, m)
    taken = path if path != wq.PATH_AUTO else wq.gemm_path(n, m, k, wtype)
    bound = B_F32 if taken == wq.PATH_MATVEC else B_MFMA
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound)
    assert_within(got, y_ref, tol, f"case {i}: wtype={wtype} n={n} m={m} k={k} flags={flags} path={path}")


@pytest.mark.parametrize("i", range(16))
def test_random_moe(i):
    g = np.random.default_rng(2000 + i)
    wtype = WTYPES[i % 3]
    k = int(g.choice([32, 512, 1024, 2048, 3072, 4096]))
    n_exp = int(g.integers(1, 9))
    top_k = int(g.integers(1, min(n_exp, 4) + 1))
    n_tok = int(g.integers(1, 40))
    m = int(g.integers(1, 200))
    gated = bool(g.integers(0, 2))
    gs = synth.rng(78, i)
    x = synth.normal_f32(gs, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(gs, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(gs, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids.astype(np.int32)), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref),
                  f"moe case {i}: wtype={wtype} n_tok={n_tok} n_exp={n_exp} top_k={top_k} m={m} k={k} gated={gated}")


# The same sweep over everything the layer takes: all five weight types, each activation, a factor
# alpha, and every path including the f32-accurate matrix-core path.
ALL_WTYPES = [wq.W_BF16, wq.W_Q8_0, wq.W_Q4_0, wq.W_F32, wq.W_F16]
ACTS = [None, "gelu", "silu", "relu", "tanh"]
PATHS = [wq.PATH_AUTO, wq.PATH_MATVEC, wq.PATH_MFMA, wq.PATH_MFMA_F32]


@pytest.mark.parametrize("i", range(64))
def test_random_layer_every_type_activation_and_path(i):
    g = np.random.default_rng(3000 + i)
    wtype = ALL_WTYPES[i % 5]
    k = int(g.choice(K_CHOICES))
    path = PATHS[int(g.integers(0, 4))]
    n = int(g.integers(1, 17)) if path == wq.PATH_MATVEC else int(g.integers(1, 200))
    m = int(g.integers(1, 300))
    act = ACTS[int(g.integers(0, 5))]
    residual = bool(g.integers(0, 2))
    has_bias = bool(g.integers(0, 2))
    alpha = float(g.choice([1.0, 1.0, 0.5, -1.25, 3.0]))
    flags = ((wq.BIAS if has_bias else 0) | (wq.RESIDUAL if residual else 0) |
             {None: 0, "gelu": wq.GELU, "silu": wq.SILU, "relu": wq.RELU, "tanh": wq.TANH}[act])
    gs = synth.rng(79, i)
    x = synth.normal_f32(gs, (n, k), 1.0)
    w = synth.weight(gs, wtype, m, k, sigma=0.05, dsigma=0.01)
    bias = synth.normal_f32(gs, (m,), 0.1) if has_bias else None
    y_old = synth.normal_f32(gs, (n, m), 1.0) if residual else None
    buf, out = guarded_out(n, m, y_old)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=None if bias is None else dev(bias), act=act,
            residual=residual, out=out, path=path, alpha=alpha)
    got = read_guarded(buf, n, m)
    taken = path if path != wq.PATH_AUTO else wq.gemm_path(n, m, k, wtype)
    bound = B_MFMA if taken == wq.PATH_MFMA else B_F32
    y_ref, tol = oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound, alpha=alpha)
    assert_within(got, y_ref, tol, f"case {i}: wtype={wtype} n={n} m={m} k={k} act={act} residual={residual} "
                                   f"bias={has_bias} alpha={alpha} path={path}")


@pytest.mark.parametrize("i", range(12))
def test_random_moe_every_type(i):
    g = np.random.default_rng(4000 + i)
    wtype = ALL_WTYPES[i % 5]
    k = int(g.choice([32, 512, 1024, 2048, 3072, 4096]))
    n_exp = int(g.integers(1, 9))
    top_k = int(g.integers(1, min(n_exp, 4) + 1))
    n_tok = int(g.integers(1, 40))
    m = int(g.integers(1, 200))
    gated = bool(g.integers(0, 2))
    gs = synth.rng(80, i)
    x = synth.normal_f32(gs, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(gs, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(gs, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids.astype(np.int32)), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref),
                  f"moe case {i}: wtype={wtype} n_tok={n_tok} n_exp={n_exp} top_k={top_k} m={m} k={k} gated={gated}")
