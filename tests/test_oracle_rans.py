"""Pins for the oracle's interleaved rANS coder.

Hand-computed states and words (tests/golden/rans_cases.json), a closed form
for the word count under the uniform table, information bounds derived from
the coder's arithmetic, and round trips.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rans_cases.json")


def _table(pairs):
    f = np.zeros(256, dtype=np.uint16)
    for s, v in pairs:
        f[s] = v
    return f


def _sym(case):
    if "sym" in case:
        return np.array(case["sym"], dtype=np.uint8)
    s = np.zeros(case["n"], dtype=np.uint8)
    for lo, hi, v in case["sym_ranges"]:
        s[lo:hi + 1] = v
    return s


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_computed_encodings(case):
    f = _table(case["f"])
    sym = _sym(case)
    states, words = oracle.rans_encode(sym, f)
    expect = [case["states"].get(str(l), case["states"]["default"]) for l in range(64)]
    assert states.tolist() == expect, case["derivation"]
    assert words.tolist() == case["words"]
    rc, back = oracle.rans_decode(words, states, f, sym.size)
    assert rc == 0 and np.array_equal(back, sym)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4097, 65536])
def test_uniform_table_word_count_closed_form(n):
    """With every f = 16 a lane's state alternates between [2^16, 2^24) and
    [2^24, 2^25), so a lane coding k symbols emits exactly floor(k/2) words."""
    rng = np.random.default_rng(n)
    sym = rng.integers(0, 256, n).astype(np.uint8)
    f = np.full(256, 16, dtype=np.uint16)
    states, words = oracle.rans_encode(sym, f)
    k = [len(range(l, n, 64)) for l in range(64)]
    assert words.size == sum(kl // 2 for kl in k)
    rc, back = oracle.rans_decode(words, states, f, n)
    assert rc == 0 and np.array_equal(back, sym)


def _bits(sym, f):
    return float(sum(math.log2(4096 / f[s]) for s in sym.tolist()))


@pytest.mark.parametrize("alpha", [0.05, 0.3, 1.0, 5.0])
def test_word_count_information_bounds(alpha):
    """16W >= sum log2(M/f) - 2*log2(16/15)*n - 1024 (each coding step and each
    renormalisation loses at most log2(16/15) bits because x >= 16 f and
    x >= 2^20 where they act; the 64 final states hold at most 16 bits more
    than the initial ones) and 16W <= sum log2(M/f) + log2(17/16)*n (a step
    gains at most log2(1 + f/x) <= log2(1 + 1/16) over the ideal)."""
    rng = np.random.default_rng(int(alpha * 100))
    p = rng.dirichlet(np.full(40, alpha))
    sym = rng.choice(40, size=50000, p=p).astype(np.uint8) + 90
    f = oracle.normalize(oracle.histogram(sym))
    states, words = oracle.rans_encode(sym, f)
    bits = _bits(sym, f)
    lo = bits - 2 * math.log2(16 / 15) * sym.size - 1024
    hi = bits + math.log2(17 / 16) * sym.size
    assert lo <= 16 * words.size <= hi
    rc, back = oracle.rans_decode(words, states, f, sym.size)
    assert rc == 0 and np.array_equal(back, sym)


def test_entropy_margin_skewed_stream():
    """Coded size stays within 1% + 1024 bits of n*H (order-0 Shannon entropy)."""
    rng = np.random.default_rng(9)
    p = np.exp(-0.5 * ((np.arange(30) - 12) / 3.0) ** 2)
    p /= p.sum()
    sym = rng.choice(30, size=65536, p=p).astype(np.uint8) + 100
    h = oracle.histogram(sym).astype(np.float64)
    q = h[h > 0] / h.sum()
    H = float(-(q * np.log2(q)).sum())
    f = oracle.normalize(oracle.histogram(sym))
    _, words = oracle.rans_encode(sym, f)
    assert 16 * words.size <= 1.01 * sym.size * H + 1024
    assert 16 * words.size >= sym.size * H - 0.1862 * sym.size - 1024


@pytest.mark.parametrize("n", [2, 3, 64, 65, 200, 4096, 70000])
def test_round_trip_various(n):
    rng = np.random.default_rng(n + 1)
    for k in (2, 3, 17, 256):
        sym = rng.integers(0, k, n).astype(np.uint8)
        sym[0], sym[-1] = 0, k - 1  # at least two symbols
        f = oracle.normalize(oracle.histogram(sym))
        states, words = oracle.rans_encode(sym, f)
        assert np.all(states >= 65536)
        rc, back = oracle.rans_decode(words, states, f, n)
        assert rc == 0 and np.array_equal(back, sym)


def test_decoder_detects_tampering():
    rng = np.random.default_rng(4)
    sym = rng.integers(0, 8, 3000).astype(np.uint8)
    f = oracle.normalize(oracle.histogram(sym))
    states, words = oracle.rans_encode(sym, f)
    assert oracle.rans_decode(words[:-1], states, f, sym.size)[0] == oracle.ERR_CORRUPT
    bad = states.copy()
    bad[5] ^= 1 << 20
    rc, out = oracle.rans_decode(words, bad, f, sym.size)
    assert rc == oracle.ERR_CORRUPT or not np.array_equal(out, sym)


def test_p_max_strict_threshold():
    # largest integer strictly below theta*n, evaluated in binary64
    assert oracle.p_max(2, 0.95) == 1
    assert oracle.p_max(100, 0.95) == 94      # 0.95*100 rounds to exactly 95.0
    assert oracle.p_max(20, 0.95) == 18       # 0.95*20 rounds to exactly 19.0
    assert oracle.p_max(65536, 0.95) == 62259  # 62259.2
    assert oracle.p_max(32768, 0.95) == 31129  # 31129.6
    assert oracle.p_max(1000, 1.0) == 999
    assert oracle.p_max(1, 0.5) == 0
