"""Pins of the oracle's contraction, epilogue and MoE combine.

* brute force: per-element Python decoding (``struct`` half/single formats)
  and ``math.fsum`` dot products on tiny shapes, every weight type and flag set;
* the closed-form GEMM probe of wavo ``gpu/mod.rs`` (``Gpu::probe_tensor``);
* identity weights; epilogue order on hand examples; tabulated GELU values and
  the Abramowitz-Stegun erf that cortiq-engine's ``ae_erf`` uses, within that
  formula's published error bound;
* MoE reductions: top-1 with gate 1 is the plain layer, slot order does not
  matter, all tokens on one expert is a 16-row product.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import golden_path

FLAGS = [0, 1, 2, 3, 4, 5, 6, 7]


def _half(b0, b1):
    return struct.unpack("<e", bytes([b0, b1]))[0]


def _brute_weight(raw, wtype, m, k):
    """Python-scalar decode of one weight, element by element."""
    w = [[0.0] * k for _ in range(m)]
    if wtype == oracle.W_BF16:
        bits = np.asarray(raw).view(np.uint16).reshape(m, k)
        for j in range(m):
            for x in range(k):
                v = int(bits[j, x])
                w[j][x] = struct.unpack("<f", bytes([0, 0, v & 0xFF, v >> 8]))[0]
        return w
    if wtype in (oracle.W_F32, oracle.W_F16):
        by = np.asarray(raw).view(np.uint8).reshape(m, -1)
        size, fmt = (4, "<f") if wtype == oracle.W_F32 else (2, "<e")
        for j in range(m):
            for x in range(k):
                w[j][x] = struct.unpack(fmt, bytes(int(b) for b in by[j, size * x:size * x + size]))[0]
        return w
    bpb = 34 if wtype == oracle.W_Q8_0 else 18
    raw = np.asarray(raw).view(np.uint8).reshape(m, -1)
    for j in range(m):
        for b in range(k // 32):
            blk = [int(v) for v in raw[j, b * bpb:(b + 1) * bpb]]
            d = _half(blk[0], blk[1])
            for i in range(32):
                if wtype == oracle.W_Q8_0:
                    q = blk[2 + i] - 256 if blk[2 + i] > 127 else blk[2 + i]
                else:
                    byte = blk[2 + (i % 16)]
                    q = (byte & 0xF if i < 16 else byte >> 4) - 8
                w[j][b * 32 + i] = d * q
    return w


def _brute(x, raw, wtype, m, k, bias, flags, y_old):
    n = x.shape[0]
    w = _brute_weight(raw, wtype, m, k)
    y = np.zeros((n, m))
    s = np.zeros((n, m))
    for t in range(n):
        for j in range(m):
            v = math.fsum(float(x[t, i]) * w[j][i] for i in range(k))
            s[t, j] = math.fsum(abs(float(x[t, i]) * w[j][i]) for i in range(k))
            if flags & 1:
                v += float(bias[j])
            if flags & 2:
                v = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
            if flags & 4:
                v += float(y_old[t, j])
            y[t, j] = v
    return y, s


@pytest.mark.parametrize("wtype", [oracle.W_BF16, oracle.W_Q8_0, oracle.W_Q4_0, oracle.W_F32, oracle.W_F16])
@pytest.mark.parametrize("shape", [(1, 1, 32), (2, 3, 64), (3, 2, 32)])
@pytest.mark.parametrize("flags", FLAGS)
def test_linear_matches_brute_force(wtype, shape, flags):
    n, m, k = shape
    g = synth.rng(99, wtype, n, m, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    raw = synth.weight(g, wtype, m, k, sigma=0.5, dsigma=0.1)
    bias = synth.normal_f32(g, (m,), 0.3)
    y_old = synth.normal_f32(g, (n, m), 1.0)
    got, s = oracle.linear(x, raw, wtype, m, k, bias, flags, y_old)
    want, ws = _brute(x, raw, wtype, m, k, bias, flags, y_old)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, ws, rtol=1e-12, atol=1e-14)


def _probe_inputs(wtype, n=130, m=64, k=32):
    r = np.arange(n)[:, None]
    xx = np.arange(k)[None, :]
    a = (xx + r % 32).astype(np.float32)
    ones = (np.arange(k)[None, :] == (np.arange(m) % 32)[:, None])
    if wtype == oracle.W_BF16:
        w = np.where(ones, 0x3F80, 0).astype(np.uint16)
    elif wtype == oracle.W_Q8_0:
        w = np.zeros((m, 34), np.uint8)
        w[:, 0], w[:, 1] = 0x00, 0x3C
        w[:, 2:] = ones.astype(np.uint8)
    else:
        q = np.where(ones, 9, 8)
        w = np.zeros((m, 18), np.uint8)
        w[:, 0], w[:, 1] = 0x00, 0x3C
        w[:, 2:] = (q[:, :16] | (q[:, 16:] << 4)).astype(np.uint8)
    return a, w


@pytest.mark.parametrize("wtype", [oracle.W_BF16, oracle.W_Q8_0, oracle.W_Q4_0])
def test_closed_form_probe(wtype):
    n, m, k = 130, 64, 32
    a, w = _probe_inputs(wtype)
    got, _ = oracle.linear(a, w, wtype, m, k)
    want = (np.arange(m)[None, :] % 32) + (np.arange(n)[:, None] % 32)
    assert np.array_equal(got, want)
    for line in open(golden_path("probe_closed_form.txt")):
        if line.startswith("#") or not line.strip():
            continue
        r, j, c = (int(v) for v in line.split())
        assert got[r, j] == c


def test_identity_weight_returns_x():
    k = 64
    g = synth.rng(5)
    x = synth.normal_f32(g, (3, k), 1.0)
    w = np.where(np.eye(k, dtype=bool), 0x3F80, 0).astype(np.uint16)
    got, s = oracle.linear(x, w, oracle.W_BF16, k, k)
    assert np.array_equal(got, x.astype(np.float64))
    assert np.array_equal(s, np.abs(x).astype(np.float64))


def _golden_gelu():
    pts = []
    for line in open(golden_path("gelu_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        x, v = line.split()
        pts.append((float(x), float(v)))
    return pts


def test_gelu_tabulated_values():
    for x, v in _golden_gelu():
        assert oracle.gelu_erf(x) == pytest.approx(v, rel=1e-14, abs=1e-16)


def test_gelu_odd_part_identity_and_limits():
    x = np.linspace(-8, 8, 4001)
    np.testing.assert_allclose(oracle.gelu_erf(x) - oracle.gelu_erf(-x), x, rtol=0, atol=1e-14)
    assert oracle.gelu_erf(40.0) == 40.0 and oracle.gelu_erf(-40.0) == 0.0


def _erf_as7126(x):
    # Abramowitz & Stegun 7.1.26, the rational-exponential erf behind ae_erf,
    # made odd by the sign of x; published maximum absolute error 1.5e-7.
    p, a1, a2, a3, a4, a5 = 0.3275911, 0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429
    ax = np.abs(x)
    t = 1.0 / (1.0 + p * ax)
    y = 1.0 - (((((a5 * t + a4) * t) + a3) * t + a2) * t + a1) * t * np.exp(-ax * ax)
    return np.where(x < 0, -y, y)


def test_oracle_erf_within_the_pages_approximation_bound():
    x = np.linspace(-6, 6, 200001)
    from scipy.special import erf
    assert np.abs(erf(x) - _erf_as7126(x)).max() <= 1.5e-7
    # and the GELU built on it inherits |x|/2 * 1.5e-7
    z = np.linspace(-6, 6, 2001)
    approx = 0.5 * z * (1.0 + _erf_as7126(z / np.sqrt(2.0)))
    assert (np.abs(oracle.gelu_erf(z) - approx) <= 0.5 * np.abs(z) * 1.5e-7 + 1e-16).all()


def test_epilogue_order_bias_then_gelu_then_residual():
    # one output, v = 0: bias 1 -> GELU(1) -> + 2
    x = np.zeros((1, 32), np.float32)
    w = np.zeros((1, 32), np.uint16)
    bias = np.array([1.0], np.float32)
    y_old = np.array([[2.0]], np.float32)
    got, _ = oracle.linear(x, w, oracle.W_BF16, 1, 32, bias, 7, y_old)
    gelu1 = dict(_golden_gelu())[1.0]
    assert got[0, 0] == pytest.approx(2.0 + gelu1, rel=1e-15)
    # residual with a zero old output is the plain call
    g = synth.rng(6)
    x = synth.normal_f32(g, (4, 64), 1.0)
    w = synth.bf16_weight(g, 5, 64, 0.1)
    b = synth.normal_f32(g, (5,), 0.1)
    plain, _ = oracle.linear(x, w, oracle.W_BF16, 5, 64, b, 3)
    res, _ = oracle.linear(x, w, oracle.W_BF16, 5, 64, b, 7, np.zeros((4, 5)))
    assert np.array_equal(plain, res)


def _moe_case(wtype=oracle.W_Q4_0, n_tok=16, n_exp=4, top_k=2, m=40, k=64, seed=3):
    g = synth.rng(seed)
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.weight(g, wtype, m, k) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    return x, bank, ids, gates


def test_moe_top1_gate1_is_plain_linear():
    x, bank, ids, _ = _moe_case(top_k=1)
    got, s = oracle.moe(x, bank, oracle.W_Q4_0, ids, 4, 40, 64, gates=np.ones((16, 1)))
    for t in range(16):
        want, ws = oracle.linear(x[t:t + 1], bank[ids[t, 0]], oracle.W_Q4_0, 40, 64)
        assert np.array_equal(got[t], want[0]) and np.array_equal(s[t], ws[0])


def test_moe_slot_order_does_not_matter():
    x, bank, ids, gates = _moe_case()
    a, _ = oracle.moe(x, bank, oracle.W_Q4_0, ids, 4, 40, 64, gates)
    b, _ = oracle.moe(x, bank, oracle.W_Q4_0, ids[:, ::-1], 4, 40, 64, gates[:, ::-1])
    np.testing.assert_allclose(a, b, rtol=1e-15, atol=1e-15)


def test_moe_all_tokens_on_one_expert_is_a_16_row_product():
    x, bank, _, _ = _moe_case(top_k=1)
    ids = np.full((16, 1), 2, np.int32)
    got, _ = oracle.moe(x, bank, oracle.W_Q4_0, ids, 4, 40, 64)
    want, _ = oracle.linear(x, bank[2], oracle.W_Q4_0, 40, 64)
    assert np.array_equal(got, want)


def test_moe_per_slot_matches_brute_force():
    x, bank, ids, gates = _moe_case(n_tok=3, n_exp=3, m=3, k=32, seed=8)
    slots, _ = oracle.moe(x, bank, oracle.W_Q4_0, ids, 3, 3, 32)
    combined, _ = oracle.moe(x, bank, oracle.W_Q4_0, ids, 3, 3, 32, gates)
    for t in range(3):
        acc = np.zeros(3)
        for j in range(2):
            w = _brute_weight(bank[ids[t, j]], oracle.W_Q4_0, 3, 32)
            dots = [math.fsum(float(x[t, i]) * w[r][i] for i in range(32)) for r in range(3)]
            np.testing.assert_allclose(slots[t * 2 + j], dots, rtol=1e-12, atol=1e-14)
            acc += float(gates[t, j]) * np.array(dots)
        np.testing.assert_allclose(combined[t], acc, rtol=1e-12, atol=1e-14)


def test_moe_rejects_out_of_range_ids():
    x, bank, ids, _ = _moe_case()
    ids = ids.copy()
    ids[0, 0] = 9
    with pytest.raises(ValueError):
        oracle.moe(x, bank, oracle.W_Q4_0, ids, 4, 40, 64)
