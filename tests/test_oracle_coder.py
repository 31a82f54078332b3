"""Pins of the oracle's range coder (CPU only).

Source: LMCache CacheGen page (0539edu.com), section 4 (CDF-driven arithmetic
coding, at most 256 tokens per stream) and section 5 (decoding with the CDF
and the prefix sums of the lengths). The page does not define the coder; the
reading is a byte-wise 32-bit range coder, stated in oracle/cachegen_oracle.c.

Pins: a hand-derived worked example, an independent unbounded-integer
formulation (tests/bignum_coder.py) that must agree byte for byte, brute force
round trips on every short sequence, closed forms of constant streams, and the
information-content bounds on the stream length.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import bignum_coder
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))

LOSS_PER_SYMBOL = -math.log2(1 - 2.0**-8)  # worst truncation loss of r = range >> 16


def _random_cdf(rng, A, T=None, alpha=0.3):
    T = T or int(rng.integers(1, 5000))
    cnt = rng.multinomial(T, rng.dirichlet(np.full(A, alpha))).astype(np.uint32).reshape(1, 1, 1, A)
    cnt = np.concatenate([cnt, cnt])
    return oracle.cdf_from_counts(cnt, T)[0, 0, 0]


def _sample(rng, cdf, n):
    p = np.diff(cdf.astype(np.float64))
    p /= p.sum()
    return rng.choice(len(p), n, p=p).astype(np.uint8)


def test_worked_example():
    g = GOLD["coder"]
    cdf = np.array(g["cdf"], np.int32)
    out = oracle.encode_stream(g["symbols"], cdf)
    assert out.hex() == g["bytes_hex"]
    assert oracle.decode_stream(out, len(g["symbols"]), cdf).tolist() == g["symbols"]


@pytest.mark.parametrize("A", [4, 16, 32, 128])
def test_matches_bignum_formulation(A):
    rng = np.random.default_rng(A)
    for trial in range(60):
        cdf = _random_cdf(rng, A, alpha=[0.05, 0.3, 3.0][trial % 3])
        n = int(rng.integers(0, 257))
        if trial % 4 == 0:
            s = rng.integers(0, A, n).astype(np.uint8)  # symbols regardless of probability
        else:
            s = _sample(rng, cdf, n)
        got = oracle.encode_stream(s, cdf)
        want, intervals, shifts, v, k = bignum_coder.encode(s.tolist(), cdf.tolist())
        assert got == want, (A, trial)
        assert bignum_coder.value_in_all_intervals(v, k, intervals)
        assert max(shifts, default=0) <= 2
        assert oracle.decode_stream(got, n, cdf).tolist() == s.tolist()


def test_carry_paths_agree_with_bignum():
    """Streams that end in long runs of 0xFF force carries through several bytes."""
    rng = np.random.default_rng(99)
    A = 4
    seen_carry_runs = 0
    for trial in range(3000):
        cdf = _random_cdf(rng, A, T=int(rng.integers(2, 50)), alpha=1.0)
        s = rng.integers(0, A, int(rng.integers(1, 40))).astype(np.uint8)
        got = oracle.encode_stream(s, cdf)
        want, _, _, _, _ = bignum_coder.encode(s.tolist(), cdf.tolist())
        assert got == want
        if b"\x00\x00" in got:
            seen_carry_runs += 1
    assert seen_carry_runs > 0


@pytest.mark.parametrize("A", [2, 3, 4])
def test_brute_force_all_short_sequences(A):
    rng = np.random.default_rng(A + 100)
    tables = [_random_cdf(rng, A, T=T) for T in (1, 3, 8, 1000)]
    tables.append(np.array([0] + [k * (65536 // A) for k in range(1, A)] + [65536], np.int32))
    for cdf in tables:
        for n in range(0, 7):
            for seq in itertools.product(range(A), repeat=n):
                out = oracle.encode_stream(seq, cdf)
                assert oracle.decode_stream(out, n, cdf).tolist() == list(seq)
                if n <= 4:
                    assert out == bignum_coder.encode(list(seq), cdf.tolist())[0]


def test_constant_stream_closed_forms():
    A, T = 32, 32768
    # A channel that is symbol 0 at every token: one table entry holds 2^16 - A + 1.
    cnt = np.zeros((2, 1, 1, A), np.uint32)
    cnt[..., 0] = T
    cdf0 = oracle.cdf_from_counts(cnt, T)[0, 0, 0]
    assert oracle.encode_stream(np.zeros(256, np.uint8), cdf0) == b""
    # Symbol 15 at every token: cdf[15] = 15; low stays far below 2^24 * 255,
    # the range never drops below 2^24, so exactly one byte is written.
    cnt = np.zeros((2, 1, 1, A), np.uint32)
    cnt[..., 15] = T
    cdf15 = oracle.cdf_from_counts(cnt, T)[0, 0, 0]
    assert cdf15[15] == 15
    out = oracle.encode_stream(np.full(256, 15, np.uint8), cdf15)
    assert len(out) == 1
    assert oracle.decode_stream(out, 256, cdf15).tolist() == [15] * 256


def test_length_bounds():
    """8*len >= I_q - 8 and len <= floor((I_q + n*loss)/8) + 1 for every stream."""
    rng = np.random.default_rng(5)
    worst = 0
    for trial in range(400):
        A = int(rng.choice([4, 16, 32, 128]))
        cdf = _random_cdf(rng, A, alpha=float(rng.choice([0.02, 0.3, 2.0])))
        n = int(rng.integers(1, 257))
        s = _sample(rng, cdf, n) if trial % 2 else rng.integers(0, A, n).astype(np.uint8)
        out = oracle.encode_stream(s, cdf)
        iq = bignum_coder.information_bits(s.tolist(), cdf.tolist())
        assert 8 * len(out) >= iq - 8 - 1e-9
        assert len(out) <= math.floor((iq + n * LOSS_PER_SYMBOL) / 8 + 1e-9) + 1
        worst = max(worst, len(out))
    # Absolute worst case: 256 symbols of frequency 1 -> 16 bits each.
    cdf = np.array([0] + list(range(65536 - 3, 65536)), np.int32)  # freq 65533, 1, 1, 1
    s = np.full(256, 2, np.uint8)
    out = oracle.encode_stream(s, cdf)
    assert len(out) <= 513
    assert oracle.decode_stream(out, 256, cdf).tolist() == s.tolist()


def test_decoder_zero_padding():
    """Bytes past the stored length read as zero: trailing zero bytes are implied."""
    rng = np.random.default_rng(8)
    cdf = _random_cdf(rng, 32)
    s = _sample(rng, cdf, 200)
    out = oracle.encode_stream(s, cdf)
    assert oracle.decode_stream(out + b"\0\0\0\0", 200, cdf).tolist() == s.tolist()
