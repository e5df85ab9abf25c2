"""GPU parity at the documented limits: the MoE at its maximum of 4096 routed slots on every MoE
kernel route (general, k-sliced, matrix cores for Q4_0 and Q8_0; 64 ballot windows of slots), and
the GEMM with 70,000 rows of X (more 64-row tiles than one grid dimension of 65,535 would hold)
on both GEMM kernels and the f32-accurate path, checked on sampled rows against the f64 oracle.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, guarded_out, oracle_with_tol, read_guarded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wtype,k", [(wq.W_Q4_0, 160), (wq.W_Q8_0, 1024), (wq.W_Q4_0, 2048), (wq.W_Q8_0, 2048),
                                     (wq.W_BF16, 1024)])
@pytest.mark.parametrize("gated", [False, True])
def test_moe_at_the_slot_limit(wtype, k, gated):
    n_tok, top_k, n_exp, m = 2048, 2, 8, 40
    assert n_tok * top_k == 4096
    g = synth.rng(81, wtype, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    rows = n_tok if gated else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids.astype(np.int32)), dev(gates) if gated else None,
                  n_experts=n_exp, m=m, k=k, out=out)
    got = read_guarded(buf, rows, m)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates if gated else None)
    assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), f"moe 4096 slots wtype={wtype} k={k}")


def test_moe_above_the_slot_limit_is_refused():
    import torch
    x = torch.zeros((4097, 32), device="cuda")
    bank = torch.zeros((2, 8, 18), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((4097, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(wq.WqError):
        wq.moe_matvec(x, bank, wq.W_Q4_0, ids, n_experts=2, m=8, k=32)


FRAMES = [0, 1, 63, 64, 65535 * 64 // 64, 69998, 69999]


@pytest.mark.parametrize("wtype,path,bound", [(wq.W_BF16, wq.PATH_MFMA, B_MFMA), (wq.W_Q8_0, wq.PATH_MFMA, B_MFMA),
                                              (wq.W_BF16, wq.PATH_MFMA_F32, B_F32)])
def test_gemm_with_70000_rows(wtype, path, bound):
    n, m, k, flags = 70000, 96, 64, wq.BIAS | wq.GELU
    g = synth.rng(82, wtype, path)
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.weight(g, wtype, m, k, sigma=0.05)
    bias = synth.normal_f32(g, (m,), 0.1)
    buf, out = guarded_out(n, m)
    wq.gemm(dev(x), dev(w), wtype, m=m, k=k, bias=dev(bias), gelu=True, out=out, path=path)
    got = read_guarded(buf, n, m)
    assert np.isfinite(got).all()
    t = np.array(FRAMES)
    y_ref, tol = oracle_with_tol(x[t], w, wtype, m, k, bias, flags, None, bound)
    assert_within(got[t], y_ref, tol, f"gemm 70000 rows wtype={wtype} path={path}")
