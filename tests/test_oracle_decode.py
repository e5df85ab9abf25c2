"""Pins of the oracle's scalar formats and weight decoders.

Each check compares the oracle with something other than itself: numpy's own
IEEE float16 / float32 conversions, hand-built blocks whose values are fixed
by the format (tests/golden), exact algebraic identities, and the Q8_0 test
encoder of wavo ``gpu/mod.rs`` (helper ``weights``).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.conftest import golden_path


def _read_blocks(name):
    cases, blk = [], None
    for line in open(golden_path(name)):
        line = line.strip()
        if line.startswith("block "):
            blk = np.frombuffer(bytes.fromhex(line.split()[1]), np.uint8)
        elif line.startswith("values "):
            vals = [float(Fraction(v)) for v in line.split()[1:]]
            cases.append((blk, np.array(vals)))
    return cases


def test_f16_decode_all_bit_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.f16_bits_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    # signs of zeros survive too
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_decode_all_bit_patterns_match_f32_upper_half():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns widen to quiet NaNs
        want = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_f32_decode_matches_numpy_on_edge_and_random_patterns():
    g = np.random.default_rng(15)
    edge = np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x3F800000, 0xBF800000, 0x7F7FFFFF,
                     0x7F800000, 0xFF800000, 0x7FC00000, 0x34000000], np.uint32)
    bits = np.concatenate([edge, g.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)])
    got = oracle.f32_bits_to_f64(bits)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns widen to quiet NaNs
        want = bits.view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert np.signbit(got[1]) and not np.signbit(got[0])
    assert got[2] == 2.0 ** -149 and got[5] == 1.0


def test_plain_f32_and_f16_weights_decode_to_their_values():
    g = np.random.default_rng(16)
    w32 = g.standard_normal((5, 64)).astype(np.float32)
    assert np.array_equal(oracle.decode(w32, oracle.W_F32, 5, 64), w32.astype(np.float64))
    w16 = g.standard_normal((5, 64)).astype(np.float16)
    assert np.array_equal(oracle.decode(w16.view(np.uint16), oracle.W_F16, 5, 64), w16.astype(np.float64))
    assert np.array_equal(oracle.decode(w32, oracle.W_F32, 5, 64, rows=[4, 1]), w32[[4, 1]].astype(np.float64))
    assert oracle.weight_nbytes(oracle.W_F32, 5, 64) == 4 * 5 * 64
    assert oracle.weight_nbytes(oracle.W_F16, 5, 64) == 2 * 5 * 64


def test_f16_subnormals_are_exact():
    # every subnormal f16 is f * 2^-24 for f in 1..1023
    f = np.arange(1, 1024)
    assert np.array_equal(oracle.f16_bits_to_f64(f), f * 2.0 ** -24)


@pytest.mark.parametrize("case", range(4))
def test_q8_0_golden_blocks(case):
    blk, want = _read_blocks("q8_0_blocks.txt")[case]
    got = oracle.decode_q8_0(blk, 1, 32)[0]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", range(3))
def test_q4_0_golden_blocks(case):
    blk, want = _read_blocks("q4_0_blocks.txt")[case]
    got = oracle.decode_q4_0(blk, 1, 32)[0]
    assert np.array_equal(got, want)


def test_q8_0_identity_d_times_q_on_random_rows():
    g = np.random.default_rng(11)
    m, k = 7, 96
    d = g.standard_normal((m, k // 32)).astype(np.float16)
    q = g.integers(-128, 128, (m, k // 32, 32), dtype=np.int8)
    raw = np.concatenate([d.view(np.uint8).reshape(m, k // 32, 2), q.view(np.uint8)], axis=2)
    got = oracle.decode_q8_0(raw.reshape(m, -1), m, k)
    want = (d.astype(np.float64)[:, :, None] * q.astype(np.float64)).reshape(m, k)
    assert np.array_equal(got, want)


def test_q4_0_identity_d_times_q_minus_8_with_nibble_order():
    g = np.random.default_rng(12)
    m, k = 5, 64
    d = g.standard_normal((m, k // 32)).astype(np.float16)
    q = g.integers(0, 16, (m, k // 32, 32))
    packed = (q[:, :, :16] | (q[:, :, 16:] << 4)).astype(np.uint8)
    raw = np.concatenate([d.view(np.uint8).reshape(m, k // 32, 2), packed], axis=2)
    got = oracle.decode_q4_0(raw.reshape(m, -1), m, k)
    want = (d.astype(np.float64)[:, :, None] * (q - 8)).reshape(m, k)
    assert np.array_equal(got, want)


def test_decode_rows_subset_matches_full():
    g = np.random.default_rng(13)
    for wt, nbpb in ((oracle.W_Q8_0, 34), (oracle.W_Q4_0, 18)):
        raw = g.integers(0, 256, (9, 3 * nbpb), dtype=np.uint8)
        full = oracle.decode(raw, wt, 9, 96)
        sub = oracle.decode(raw, wt, 9, 96, rows=[8, 0, 3])
        assert np.array_equal(sub, full[[8, 0, 3]], equal_nan=True)


def test_q8_0_round_trip_through_the_wavo_test_encoder():
    g = np.random.default_rng(14)
    w = g.uniform(-1, 1, (6, 128)).astype(np.float32)
    w[2, :32] = 0.0  # an all-zero block encodes to d = 0, q = 0
    raw = oracle.encode_q8_0(w)
    dec = oracle.decode_q8_0(raw, 6, 128)
    blocks = w.reshape(6, 4, 32).astype(np.float64)
    d = np.abs(blocks).max(axis=2) / 127.0
    dh = d.astype(np.float16).astype(np.float64)
    # |x - dh*q| <= |x - d*q| + |d - dh|*|q| <= d/2 + 127*|d - dh| (plus f32 slack)
    bound = d / 2 + 127 * np.abs(d - dh) + 1e-6 * np.abs(blocks).max(axis=2)
    err = np.abs(dec.reshape(6, 4, 32) - blocks).max(axis=2)
    assert (err <= bound).all()
    assert np.array_equal(dec[2, :32], np.zeros(32))
    # the largest element of each nonzero block encodes to +-127
    q = raw.reshape(6, 4, 34)[:, :, 2:].view(np.int8)
    nz = np.abs(blocks).max(axis=2) > 0
    assert (np.abs(q).max(axis=2)[nz] == 127).all()
