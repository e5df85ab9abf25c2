"""Calls from several host threads at once, on shared and on separate streams.

Every entry point may be called concurrently (include/wq.h). The gated MoE call is the one with
shared host state: a per-(device, stream) combine workspace that a call may have to grow while
another thread's work on the same stream still reads the old one. Each thread here repeats a
sequence of calls whose MoE sizes force that growth; the results must equal, bit for bit, those
of the same calls made one at a time, and the one-at-a-time MoE results are checked against the
oracle. Every call made here sums in a fixed order, so a race shows as a difference. (The one route
that does not, the k split of residual layers without activation on quantized, f16 and f32 weights
at few tiles, is not among them: the Q8_0 call has 4 rows and takes the matvec, and the bf16 GEMM
has GELU.)
"""
import threading

import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, B_MFMA, assert_within, dev, oracle_with_tol

pytestmark = pytest.mark.gpu

N_EXP, M, K, TOP_K = 8, 1024, 2048, 2
# n_slots * M * 4 bytes: 64 KiB, 320 KiB, then 1.25 MiB, past the workspace's first 1 MiB.
TOKENS = (8, 40, 160)
N_THREADS = 4
REPEATS = 3


def _case(tid: int):
    """Inputs of one thread: a gated MoE call per size in TOKENS, a Q8_0 matvec and a bf16 GEMM."""
    g = synth.rng(95, tid)
    bank = np.stack([synth.weight(g, wq.W_Q4_0, M, K, sigma=0.05) for _ in range(N_EXP)])
    moe = []
    for n_tok in TOKENS:
        x = synth.normal_f32(g, (n_tok, K), 1.0)
        ids, gates = synth.moe_routing(g, n_tok, N_EXP, TOP_K)
        moe.append((x, ids, gates))
    xq = synth.normal_f32(g, (4, 1024), 1.0)
    wq8 = synth.weight(g, wq.W_Q8_0, 512, 1024, sigma=0.05)
    xb = synth.normal_f32(g, (100, 1024), 1.0)
    wb = synth.weight(g, wq.W_BF16, 300, 1024, sigma=0.05)
    bias = synth.normal_f32(g, (300,), 0.1)
    return bank, moe, (xq, wq8), (xb, wb, bias)


class _Thread:
    """Device copies and outputs of one thread's calls."""

    def __init__(self, tid: int):
        import torch
        self.host = _case(tid)
        bank, moe, (xq, wq8), (xb, wb, bias) = self.host
        self.bank = dev(bank)
        self.moe = [(dev(x), dev(ids.astype(np.int32)), dev(gates)) for x, ids, gates in moe]
        self.moe_out = [torch.empty((len(x), M), device="cuda") for x, _, _ in moe]
        self.xq, self.wq8 = dev(xq), dev(wq8)
        self.q_out = torch.empty((4, 512), device="cuda")
        self.xb, self.wb, self.bias = dev(xb), dev(wb), dev(bias)
        self.b_out = torch.empty((100, 300), device="cuda")

    def run(self):
        for (x, ids, gates), out in zip(self.moe, self.moe_out):
            wq.moe_matvec(x, self.bank, wq.W_Q4_0, ids, gates, n_experts=N_EXP, m=M, k=K, out=out)
        wq.gemm(self.xq, self.wq8, wq.W_Q8_0, m=512, k=1024, out=self.q_out)
        wq.gemm(self.xb, self.wb, wq.W_BF16, m=300, k=1024, bias=self.bias, act="gelu", out=self.b_out)

    def results(self):
        return [o.cpu().numpy() for o in self.moe_out] + [self.q_out.cpu().numpy(), self.b_out.cpu().numpy()]


def test_concurrent_calls_match_serial_calls_bit_for_bit():
    import torch
    threads = [_Thread(t) for t in range(N_THREADS)]
    for th in threads:
        th.run()
    torch.cuda.synchronize()
    serial = [th.results() for th in threads]

    # Anchor the serial results: thread 0's MoE calls and the two layers against the oracle.
    bank, moe, (xq, wq8), (xb, wb, bias) = threads[0].host
    for (x, ids, gates), got in zip(moe, serial[0][:len(TOKENS)]):
        y_ref, S = oracle.moe(x, bank, wq.W_Q4_0, ids, N_EXP, M, K, gates)
        assert_within(got, y_ref, B_F32 * S + 8 * 2.0 ** -24 * np.abs(y_ref), f"moe n_tok={len(x)}")
    y_ref, tol = oracle_with_tol(xq, wq8, wq.W_Q8_0, 512, 1024, None, 0, None, B_F32)
    assert_within(serial[0][-2], y_ref, tol, "Q8_0 matvec")
    y_ref, tol = oracle_with_tol(xb, wb, wq.W_BF16, 300, 1024, bias, wq.BIAS | wq.GELU, None, B_MFMA)
    assert_within(serial[0][-1], y_ref, tol, "bf16 GEMM")

    # Threads 0 and 1 share one stream; threads 2 and 3 each have a stream of their own. These are
    # not the stream of the serial calls, so their workspaces can start small and grow meanwhile.
    for th in threads:
        for o in th.moe_out + [th.q_out, th.b_out]:
            o.fill_(float("nan"))
    torch.cuda.synchronize()
    shared = torch.cuda.Stream()
    streams = [shared, shared, torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []
    start = threading.Barrier(N_THREADS)

    def work(t):
        try:
            start.wait()
            with torch.cuda.stream(streams[t]):
                for _ in range(REPEATS):
                    threads[t].run()
        except Exception as exc:  # reported in the main thread
            errors.append(f"thread {t}: {exc!r}")

    workers = [threading.Thread(target=work, args=(t,)) for t in range(N_THREADS)]
    for w in workers:
        w.start()
    for w in workers:
        w.join(timeout=60)
    assert not any(w.is_alive() for w in workers), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for t, th in enumerate(threads):
        for i, (got, want) in enumerate(zip(th.results(), serial[t])):
            assert np.array_equal(got, want), f"thread {t}, call {i}: concurrent result differs from the serial one"
