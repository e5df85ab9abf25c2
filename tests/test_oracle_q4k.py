"""Pins of the oracle's Q4_K decode and of the layer and MoE on Q4_K weights.

The pages name Q4_K (hanzo-ml ``wgpu_backend.rs``, ``matvec_q4k_gpu``: 144-byte super-blocks of 256
weights) but do not print its bytes; the layout is GGML's published k-quant super-block. What
pins the oracle here, apart from itself:

* hand-built super-blocks whose values were worked out by hand from that layout (tests/golden);
* a packer written in this file from the layout (field -> bit position, byte by byte), so that a
  wrong index, shift or nibble order in the oracle's unpacking breaks the round trip;
* a scalar decode, element by element, inside a brute-force ``math.fsum`` layer and MoE.

The packer and the hand-built blocks pin the oracle to one reading of the layout; they cannot pin
that reading to the pages, which do not give it.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import golden_path


def _golden():
    cases, blk = [], None
    for line in open(golden_path("q4_k_blocks.txt")):
        line = line.strip()
        if line.startswith("block "):
            blk = np.frombuffer(bytes.fromhex(line.split()[1]), np.uint8)
        elif line.startswith("values "):
            vals = []
            for tok in line.split()[1:]:
                cnt, _, v = tok.partition("x") if "x" in tok else ("1", "", tok)
                vals += [float(Fraction(v))] * int(cnt)
            cases.append((blk, {i: v for i, v in enumerate(vals)}))
        elif line.startswith("at "):
            pairs = (tok.split(":") for tok in line.split()[1:])
            cases.append((blk, {int(i): float(Fraction(v)) for i, v in pairs}))
    return cases


@pytest.mark.parametrize("case", range(3))
def test_q4_k_golden_blocks(case):
    blk, want = _golden()[case]
    assert blk.size == 144
    got = oracle.decode_q4_k(blk, 1, 256)[0]
    if len(want) == 256:
        assert np.array_equal(got, np.array([want[i] for i in range(256)]))
    for i, v in want.items():
        assert got[i] == v, (i, got[i], v)


def _pack(d_bits, dmin_bits, sc, mn, q):
    """One 144-byte super-block from its fields, written from the layout bit by bit."""
    out = bytearray(144)
    out[0:2] = int(d_bits).to_bytes(2, "little")
    out[2:4] = int(dmin_bits).to_bytes(2, "little")
    scales = [0] * 12
    for j in range(8):
        s, m = int(sc[j]), int(mn[j])
        assert 0 <= s < 64 and 0 <= m < 64
        if j < 4:
            scales[j] |= s            # bits 0-5 of scale byte j
            scales[j + 4] |= m        # bits 0-5 of scale byte j + 4
        else:
            scales[j + 4] |= s & 0xF          # low nibble of byte j + 4: scale bits 0-3
            scales[j + 4] |= (m & 0xF) << 4   # high nibble: min bits 0-3
            scales[j - 4] |= (s >> 4) << 6    # bits 6-7 of byte j - 4: scale bits 4-5
            scales[j] |= (m >> 4) << 6        # bits 6-7 of byte j: min bits 4-5
    out[4:16] = bytes(scales)
    for e in range(256):
        j, l = divmod(e, 32)          # sub-block j, element l
        byte = 16 + 32 * (j // 2) + l
        out[byte] |= int(q[e]) << (4 * (j % 2))
    return np.frombuffer(bytes(out), np.uint8)


def _f16(bits):
    return struct.unpack("<e", int(bits).to_bytes(2, "little"))[0]


def test_q4_k_round_trip_through_an_independent_packer():
    g = np.random.default_rng(21)
    for _ in range(40):
        d_bits, dmin_bits = (int(b) for b in g.integers(0, 0x7C00, 2))  # finite, non-negative f16
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        got = oracle.decode_q4_k(_pack(d_bits, dmin_bits, sc, mn, q), 1, 256)[0]
        d, dmin = _f16(d_bits), _f16(dmin_bits)
        want = [d * int(sc[e // 32]) * int(q[e]) - dmin * int(mn[e // 32]) for e in range(256)]
        assert np.array_equal(got, np.array(want))


def test_q4_k_scale_fields_reach_every_value():
    # Every (sc, m) pair value 0..63 in every sub-block position round-trips.
    for v in range(64):
        for j in range(8):
            sc = np.zeros(8, int)
            mn = np.zeros(8, int)
            sc[j] = v
            mn[(j + 3) % 8] = 63 - v
            blk = _pack(0x3C00, 0x3C00, sc, mn, np.zeros(256, int))
            got_sc, got_mn = oracle.q4_k_scale_min(blk[4:16])
            assert list(got_sc) == list(sc) and list(got_mn) == list(mn)


def test_q4_k_negative_and_subnormal_factors():
    # Sign bits and f16 subnormals in d and dmin decode exactly.
    for d_bits, dmin_bits in ((0x8001, 0x03FF), (0xBC00, 0x8400), (0x0001, 0xFBFF)):
        sc = np.arange(8) * 9 % 64
        mn = (np.arange(8) * 13 + 5) % 64
        q = np.arange(256) % 16
        got = oracle.decode_q4_k(_pack(d_bits, dmin_bits, sc, mn, q), 1, 256)[0]
        d, dmin = _f16(d_bits), _f16(dmin_bits)
        want = [d * int(sc[e // 32]) * int(q[e]) - dmin * int(mn[e // 32]) for e in range(256)]
        assert np.array_equal(got, np.array(want))


def _scalar_row(raw_row, k):
    """Python-scalar decode of one Q4_K row, element by element from the layout."""
    b = [int(v) for v in raw_row]
    out = []
    for s in range(k // 256):
        o = 144 * s
        d, dmin = _f16(b[o] | b[o + 1] << 8), _f16(b[o + 2] | b[o + 3] << 8)
        sb = b[o + 4:o + 16]
        for e in range(256):
            j, l = divmod(e, 32)
            if j < 4:
                sc, mn = sb[j] & 63, sb[j + 4] & 63
            else:
                sc = (sb[j + 4] & 15) | ((sb[j - 4] >> 6) << 4)
                mn = (sb[j + 4] >> 4) | ((sb[j] >> 6) << 4)
            qb = b[o + 16 + 32 * (j // 2) + l]
            q = (qb >> 4) if j % 2 else (qb & 15)
            out.append(d * sc * q - dmin * mn)
    return out


@pytest.mark.parametrize("shape", [(1, 1, 256), (2, 3, 512), (3, 2, 256)])
@pytest.mark.parametrize("flags", [0, 1, 3, 5, 7])
def test_q4_k_linear_matches_brute_force(shape, flags):
    n, m, k = shape
    g = synth.rng(98, n, m, k, flags)
    x = synth.normal_f32(g, (n, k), 1.0)
    raw = synth.q4_k_weight(g, m, k, dsigma=0.1)
    bias = synth.normal_f32(g, (m,), 0.3)
    y_old = synth.normal_f32(g, (n, m), 1.0)
    got, s = oracle.linear(x, raw, oracle.W_Q4_K, m, k, bias, flags, y_old)
    w = [_scalar_row(raw[j], k) for j in range(m)]
    for t in range(n):
        for j in range(m):
            v = math.fsum(float(x[t, i]) * w[j][i] for i in range(k))
            sv = math.fsum(abs(float(x[t, i]) * w[j][i]) for i in range(k))
            if flags & 1:
                v += float(bias[j])
            if flags & 2:
                v = 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))
            if flags & 4:
                v += float(y_old[t, j])
            assert got[t, j] == pytest.approx(v, rel=1e-12, abs=1e-12)
            assert s[t, j] == pytest.approx(sv, rel=1e-12, abs=1e-14)


def test_q4_k_moe_slots_match_brute_force():
    g = synth.rng(97)
    n_tok, top_k, n_exp, m, k = 3, 2, 3, 2, 256
    x = synth.normal_f32(g, (n_tok, k), 1.0)
    bank = np.stack([synth.q4_k_weight(g, m, k) for _ in range(n_exp)])
    ids, gates = synth.moe_routing(g, n_tok, n_exp, top_k)
    slots, _ = oracle.moe(x, bank, oracle.W_Q4_K, ids, n_exp, m, k)
    combined, _ = oracle.moe(x, bank, oracle.W_Q4_K, ids, n_exp, m, k, gates)
    for t in range(n_tok):
        for r in range(m):
            tot = 0.0
            for j in range(top_k):
                w = _scalar_row(bank[ids[t, j]][r], k)
                v = math.fsum(float(x[t, i]) * w[i] for i in range(k))
                assert slots[t * top_k + j, r] == pytest.approx(v, rel=1e-12, abs=1e-15)
                tot += float(gates[t, j]) * v
            assert combined[t, r] == pytest.approx(tot, rel=1e-12, abs=1e-15)


def test_q4_k_rows_subset_and_sizes():
    g = synth.rng(96)
    raw = synth.q4_k_weight(g, 5, 512)
    assert raw.shape == (5, 2 * 144) and oracle.weight_nbytes(oracle.W_Q4_K, 5, 512) == 5 * 288
    full = oracle.decode(raw, oracle.W_Q4_K, 5, 512)
    assert np.array_equal(oracle.decode(raw, oracle.W_Q4_K, 5, 512, rows=[4, 1]), full[[4, 1]])
    with pytest.raises(ValueError):
        oracle.decode_q4_k(raw, 5, 480)


def test_q4_k_parts_are_the_two_products():
    g = np.random.default_rng(23)
    for _ in range(10):
        d_bits, dmin_bits = (int(b) for b in g.integers(0, 0x7C00, 2))
        sc, mn, q = g.integers(0, 64, 8), g.integers(0, 64, 8), g.integers(0, 16, 256)
        blk = _pack(d_bits, dmin_bits, sc, mn, q)
        pos, neg = oracle.decode_q4_k_parts(blk, 1, 256)
        d, dmin = _f16(d_bits), _f16(dmin_bits)
        assert np.array_equal(pos[0], [d * int(sc[e // 32]) * int(q[e]) for e in range(256)])
        assert np.array_equal(neg[0], [dmin * int(mn[e // 32]) for e in range(256)])
        assert np.array_equal(oracle.decode_q4_k(blk, 1, 256), pos - neg)


def test_q4_k_part_scale_brute_force():
    g = synth.rng(95)
    x = synth.normal_f32(g, (2, 512), 1.0)
    raw = synth.q4_k_weight(g, 3, 512)
    got = oracle.q4_k_part_scale(x, raw, 3, 512)
    for j in range(3):
        b = [int(v) for v in raw[j]]
        for t in range(2):
            tot = []
            for s in range(2):
                o = 144 * s
                d, dmin = _f16(b[o] | b[o + 1] << 8), _f16(b[o + 2] | b[o + 3] << 8)
                sc, mn = oracle.q4_k_scale_min(np.array(b[o + 4:o + 16]))
                for e in range(256):
                    jj, l = divmod(e, 32)
                    qb = b[o + 16 + 32 * (jj // 2) + l]
                    q = (qb >> 4) if jj % 2 else (qb & 15)
                    tot.append(abs(float(x[t, 256 * s + e])) * (abs(d * int(sc[jj]) * q) + abs(dmin * int(mn[jj]))))
            assert got[t, j] == pytest.approx(math.fsum(tot), rel=1e-12)
    assert (got >= oracle.linear(x, raw, oracle.W_Q4_K, 3, 512)[1] - 1e-12).all()
