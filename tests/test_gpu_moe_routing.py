"""MoE routings that exercise the device-side scheduling over touched experts: sparse routing
(1 token to 2 of 8 experts, 16 tokens to 2 of 64), every slot on one expert, every id out of range
(no expert touched: every output NaN), a mix of valid and invalid ids, and more experts than the
touched-expert bitmap holds (the grid is then split over all experts). Both MoE kernels (the
matrix-core one for Q8_0/Q4_0 at k 2048..4096, the sliced one otherwise), gated and per slot."""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, ULP_SLACK, assert_within, dev, guarded_out, read_guarded

pytestmark = pytest.mark.gpu


def _run(x, bank, wtype, ids, gates, n_exp, m, k):
    n_tok, top_k = ids.shape
    rows = n_tok if gates is not None else n_tok * top_k
    buf, out = guarded_out(rows, m)
    wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids), None if gates is None else dev(gates),
                  n_experts=n_exp, m=m, k=k, out=out)
    return read_guarded(buf, rows, m)


def _check(x, bank, wtype, ids, gates, n_exp, m, k, what):
    got = _run(x, bank, wtype, ids, gates, n_exp, m, k)
    y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates)
    assert_within(got, y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), what)


CASES = [  # (n_tok, n_exp, top_k, m, k, wtype)
    (1, 8, 2, 700, 4096, wq.W_Q4_0),     # matrix-core kernel, 2 of 8 experts touched
    (1, 8, 2, 700, 1024, wq.W_Q8_0),     # sliced kernel
    (16, 64, 2, 300, 2048, wq.W_Q8_0),
    (16, 64, 2, 300, 1024, wq.W_BF16),
    (3, 256, 2, 90, 2048, wq.W_Q4_0),    # the bitmap's largest bank
]


@pytest.mark.parametrize("n_tok,n_exp,top_k,m,k,wtype", CASES)
@pytest.mark.parametrize("gated", [False, True])
def test_sparse_routing(n_tok, n_exp, top_k, m, k, wtype, gated):
    g = synth.rng(400, n_tok, n_exp, m, k, wtype)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    _check(x, bank, wtype, ids, gates if gated else None, n_exp, m, k, f"sparse {n_tok}x top{top_k}/{n_exp}")


@pytest.mark.parametrize("k,wtype", [(4096, wq.W_Q4_0), (1024, wq.W_Q8_0)])
def test_every_slot_on_one_expert(k, wtype):
    n_tok, n_exp, m = 40, 8, 257
    g = synth.rng(401, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids = np.full((n_tok, 1), 5, np.int32)
    _check(x, bank, wtype, ids, None, n_exp, m, k, "one expert")


@pytest.mark.parametrize("k,wtype", [(4096, wq.W_Q4_0), (1024, wq.W_Q8_0)])
def test_no_expert_touched_gives_nan(k, wtype):
    n_tok, n_exp, m = 4, 8, 100
    g = synth.rng(402, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k) for _ in range(n_exp)])
    ids = np.array([[-1, 8], [9, -5], [100, 8], [-2, 12]], np.int32)
    got = _run(x, bank, wtype, ids, None, n_exp, m, k)
    assert np.isnan(got).all()


@pytest.mark.parametrize("k,wtype", [(4096, wq.W_Q8_0), (1024, wq.W_Q4_0)])
def test_mixed_valid_and_invalid_ids(k, wtype):
    n_tok, n_exp, m = 6, 8, 130
    g = synth.rng(403, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, _ = synth.moe_routing(g, n_tok, n_exp, 2)
    ids[1, 0] = 8
    ids[4, 1] = -1
    got = _run(x, bank, wtype, ids, None, n_exp, m, k)
    bad = np.zeros(n_tok * 2, bool)
    bad[[2, 9]] = True
    assert np.isnan(got[bad]).all()
    ok_ids = np.where(ids < 0, 0, np.where(ids >= n_exp, 0, ids))
    y_ref, S = oracle.moe(x, bank, wtype, ok_ids, n_exp, m, k)
    assert_within(got[~bad], y_ref[~bad], B_F32 * S[~bad] + ULP_SLACK * np.abs(y_ref[~bad]), "mixed ids")


@pytest.mark.parametrize("k,wtype", [(2048, wq.W_Q4_0), (1024, wq.W_Q8_0)])
def test_more_experts_than_the_bitmap(k, wtype):
    n_tok, n_exp, top_k, m = 5, 300, 3, 48
    g = synth.rng(404, k)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    _check(x, bank, wtype, ids, gates, n_exp, m, k, "300 experts")
