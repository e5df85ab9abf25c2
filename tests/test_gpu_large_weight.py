"""A weight above 2 GiB on the matvec path: bf16 152064 x 8192 (2.49 GB, an output layer's size)
at n = 1 and n = 4.

The sliced matvec kernel clamps each tile's 16-byte loads to the bytes left in W. Those bytes
pass 2^31 for the first 20,992 rows of this weight, where a 32-bit product would wrap (the clamp
itself is checked on the host in test_host_offsets.py). The weight is built on the device by
repeating a seeded block of 997 rows: 997 does not divide the 2^31-byte (131072-row) or 2^32-byte
stride, so a read from the wrong 2 GiB half gives a different row. Outputs are checked against the
oracle on the first tiles, on the tiles where the bytes left cross 2^31, on the tiles around byte
offset 2^31, on the last tiles and on random rows; the rest must be finite.
"""
import numpy as np
import pytest

import gemv_wq_gemm_amd as wq
import oracle
import synth
from tests.parity import B_F32, ULP_SLACK, assert_within, dev, guarded_out, literal_ratio, read_guarded

pytestmark = pytest.mark.gpu

M, K, BLOCK_ROWS = 152064, 8192, 997


@pytest.fixture(scope="module")
def big_weight():
    import torch
    blk = synth.bf16_weight(synth.rng(70), BLOCK_ROWS, K, 0.02)
    reps = -(-M // BLOCK_ROWS)
    w = dev(blk.view(np.int16)).repeat(reps, 1)[:M]
    assert w.is_contiguous() and w.numel() * 2 == wq.weight_bytes(wq.W_BF16, M, K) > 2 ** 31
    yield blk, w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 4])
def test_bf16_weight_over_2_gib(big_weight, n):
    blk, w = big_weight
    x = synth.normal_f32(synth.rng(71, n), (n, K), 1.0)
    assert wq.gemm_path(n, M, K, wq.W_BF16) == wq.PATH_MATVEC
    buf, out = guarded_out(n, M)
    wq.gemm(dev(x), w, wq.W_BF16, m=M, k=K, out=out)
    got = read_guarded(buf, n, M)
    assert np.isfinite(got).all()
    rows = np.unique(np.concatenate([
        np.arange(0, 256),                 # first tiles: 2.49 GB left
        np.arange(20928, 21056),           # bytes left cross 2^31 at row 20992
        np.arange(131008, 131136),         # byte offset 2^31 at row 131072
        np.arange(M - 256, M),             # last tiles
        synth.rng(72).choice(M, 512, replace=False),
    ]))
    ref_blk, s_blk = oracle.linear(x, blk, wq.W_BF16, BLOCK_ROWS, K)
    y_ref, S = ref_blk[:, rows % BLOCK_ROWS], s_blk[:, rows % BLOCK_ROWS]
    assert_within(got[:, rows], y_ref, B_F32 * S + ULP_SLACK * np.abs(y_ref), f"bf16 {M}x{K} n={n}")
    print(f"bf16 {M}x{K} n={n}: err/(1e-5 S) = {literal_ratio(got[:, rows], y_ref, S, B_F32):.4f}")
