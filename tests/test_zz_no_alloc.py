"""wq_moe_matvec_noalloc, the MoE entry point that allocates nothing, against wq_moe_matvec.

Two gated calls in a row through the C ABI, the second one smaller (the scratch array then holds
the first call's values beyond what the second one writes): each must equal wq_moe_matvec's
result bit for bit (the same kernels) and meet the oracle's bound. An ungated call, which uses
no scratch, is checked the same way.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, ULP_SLACK, assert_within, dev, guarded_out, read_guarded

pytestmark = pytest.mark.gpu


def _case(seed, n_tok, n_exp, top_k, m, k, wtype):
    g = synth.rng(80, seed)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k, sigma=0.05) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    return x, bank, ids, gates


def _both(x, bank, ids, gates, wtype, n_exp, m, k):
    rows = ids.shape[0] if gates is not None else ids.size
    outs = []
    for noalloc in (False, True):
        buf, out = guarded_out(rows, m)
        wq.moe_matvec(dev(x), dev(bank), wtype, dev(ids), None if gates is None else dev(gates),
                      n_experts=n_exp, m=m, k=k, out=out, noalloc=noalloc)
        outs.append(read_guarded(buf, rows, m))
    return outs


@pytest.mark.parametrize("wtype", [wq.W_Q4_0, wq.W_Q8_0])
def test_noalloc_matches_allocating_entry_point(wtype):
    # The first call is the MoE workload's shape (16 tokens, top-2 of 8, 14336 x 4096), the second
    # a smaller one on other kernels (5 tokens, top-3 of 4, 300 x 1024).
    for seed, (n_tok, n_exp, top_k, m, k) in enumerate([(16, 8, 2, 14336, 4096), (5, 4, 3, 300, 1024)]):
        x, bank, ids, gates = _case(seed, n_tok, n_exp, top_k, m, k, wtype)
        ref_alloc, got = _both(x, bank, ids, gates, wtype, n_exp, m, k)
        assert np.array_equal(got.view(np.uint32), ref_alloc.view(np.uint32)), f"call {seed}"
        cols = np.unique(np.concatenate([np.arange(min(m, 256)), np.arange(max(0, m - 256), m),
                                         synth.rng(81, seed).choice(m, min(m, 512), replace=False)]))
        y_ref, S = oracle.moe(x, bank, wtype, ids, n_exp, m, k, gates, rows=cols)
        assert_within(got[:, cols], y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), f"noalloc call {seed}")


def test_noalloc_ungated_and_limit():
    x, bank, ids, _ = _case(3, 6, 3, 2, 200, 2048, wq.W_Q8_0)
    ref_alloc, got = _both(x, bank, ids, None, wq.W_Q8_0, 3, 200, 2048)
    assert np.array_equal(got.view(np.uint32), ref_alloc.view(np.uint32))
    # A gated call beyond the scratch is refused before anything is enqueued.
    import torch
    n_tok, top_k, m, k = 4096, 1, 4096, 32
    xs = torch.zeros((n_tok, k), device="cuda")
    bank = torch.zeros((1, m * 34), dtype=torch.uint8, device="cuda")
    ids_t = torch.zeros((n_tok, top_k), dtype=torch.int32, device="cuda")
    gates_t = torch.ones((n_tok, top_k), device="cuda")
    with pytest.raises(wq.WqError, match="scratch"):
        wq.moe_matvec(xs, bank, wq.W_Q8_0, ids_t, gates_t, n_experts=1, m=m, k=k, noalloc=True)
