"""The entry points inside a captured HIP graph.

A serving loop captures its calls once and replays the graph. Nothing the library enqueues may
need the host while captured (no synchronization, no allocation, no memset node). Here one graph
holds a bf16 layer on the matrix cores (bias + GELU), a Q8_0 matvec with a residual, a gated MoE
through the entry point that never allocates, and one encoder block (with its bf16 hand-offs).
It is replayed several times with new inputs copied into its input buffers, the program's own
eager work and synchronizations between replays, and every replay is compared bit for bit with
the same calls made eagerly on the same inputs.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import synth
from tests.parity import dev

pytestmark = pytest.mark.gpu


def _layer_dev(L):
    return {k: None if v is None else dev(v) for k, v in L.items()}


def test_graph_replays_match_eager_calls():
    import torch
    g = synth.rng(900)
    # bf16 layer, n = 96: 96 x 512 x 256 + bias + GELU
    n1, m1, k1 = 96, 512, 256
    x1 = dev(synth.normal_f32(g, (n1, k1), 1.0))
    w1 = dev(synth.bf16_weight(g, m1, k1, 0.05))
    b1 = dev(synth.normal_f32(g, (m1,), 0.1))
    y1 = torch.empty((n1, m1), device="cuda")
    # Q8_0 matvec, n = 3, residual
    n2, m2, k2 = 3, 1000, 1024
    x2 = dev(synth.normal_f32(g, (n2, k2), 1.0))
    w2 = dev(synth.q8_0_weight(g, m2, k2))
    y2 = torch.empty((n2, m2), device="cuda")
    # gated MoE, Q4_0: 8 tokens top-2 of 4 experts of 300 x 2048 (the matrix-core kernel)
    nt, ne, tk, m3, k3 = 8, 4, 2, 300, 2048
    x3 = dev(synth.normal_f32(g, (nt, k3), 1.0))
    bank = dev(np.stack([synth.q4_0_weight(g, m3, k3) for _ in range(ne)]))
    ids, gates = synth.moe_routing(g, nt, ne, tk)
    ids_d, gates_d = dev(ids), dev(gates)
    y3 = torch.empty((nt, m3), device="cuda")
    # one encoder block on the bf16 matrix cores: 70 frames, d = 128, 2 heads, MLP 256
    n4, d4, heads, inter, rot = 70, 128, 2, 256, 64
    L = _layer_dev(synth.encoder_block_weights(0, seed=3, d=d4, heads=heads, inter=inter, sigma=0.05))
    valid = dev(synth.key_mask(n4, 60))
    cs = wq.rope_table(n4, rot).cuda()
    ws = torch.empty(wq.encoder_workspace_bytes(n4, d4, heads, inter), dtype=torch.uint8, device="cuda")
    h = torch.empty((n4, d4), device="cuda")
    desc = wq.encoder_layer_desc(L)

    def calls():
        wq.gemm(x1, w1, wq.W_BF16, m=m1, k=k1, bias=b1, gelu=True, out=y1)
        wq.gemm(x2, w2, wq.W_Q8_0, m=m2, k=k2, residual=True, out=y2)
        wq.moe_matvec(x3, bank, wq.W_Q4_0, ids_d, gates_d, n_experts=ne, m=m3, k=k3, out=y3, noalloc=True)
        wq.encoder_layer(h, desc, wq.W_BF16, valid, cs, n=n4, d=d4, heads=heads, rot=rot, inter=inter,
                         path=wq.PATH_MFMA, workspace=ws)

    def fill(seed):
        r = synth.rng(901, seed)
        x1.copy_(dev(synth.normal_f32(r, (n1, k1), 1.0)))
        x2.copy_(dev(synth.normal_f32(r, (n2, k2), 1.0)))
        y2.copy_(dev(synth.normal_f32(r, (n2, m2), 1.0)))
        x3.copy_(dev(synth.normal_f32(r, (nt, k3), 1.0)))
        h.copy_(dev(synth.normal_f32(r, (n4, d4), 1.0)))
        torch.cuda.synchronize()

    def outputs():
        torch.cuda.synchronize()
        return [t.cpu().numpy().copy() for t in (y1, y2, y3, h)]

    # Warm-up outside capture (first calls fill the library's per-device caches).
    fill(0)
    calls()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fill(0)
        with torch.cuda.graph(graph, stream=s):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(1, 5):
        fill(rep)
        graph.replay()
        got = outputs()
        # eager work between replays: the same calls on the same inputs
        fill(rep)
        calls()
        want = outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.isfinite(a).all(), f"replay {rep}, output {i}: non-finite values"
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {rep}, output {i} differs"
