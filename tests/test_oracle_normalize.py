"""Pins for the oracle's normalisation of histograms to a 4096 total."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "normalize_cases.json")


def _expand(ranges):
    out = np.zeros(256, dtype=np.uint64)
    for lo, hi, v in ranges:
        out[lo:hi + 1] = v
    return out


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    f = oracle.normalize(_expand(case["hist"]))
    assert np.array_equal(f.astype(np.uint64), _expand(case["f"])), case["derivation"]


def _check_invariants(h, f):
    f = f.astype(np.int64)
    assert f.sum() == 4096
    assert np.array_equal(f > 0, h > 0)
    assert f.max() <= 4095


def test_invariants_random_histograms():
    rng = np.random.default_rng(7)
    for trial in range(400):
        k = int(rng.integers(2, 257))
        support = rng.choice(256, size=k, replace=False)
        h = np.zeros(256, dtype=np.uint64)
        scale = 10 ** rng.uniform(0, 6)
        h[support] = (rng.pareto(1.0, size=k) * scale).astype(np.uint64) + 1
        _check_invariants(h, oracle.normalize(h))


def test_invariants_small_brute_force():
    """All histograms with n <= 10 over 2..4 symbols at spread positions."""
    positions = [0, 17, 128, 255]
    count = 0
    for k in range(2, 5):
        def rec(prefix, remaining):
            nonlocal count
            if len(prefix) == k:
                h = np.zeros(256, dtype=np.uint64)
                for p, c in zip(positions[:k], prefix):
                    h[p] = c
                _check_invariants(h, oracle.normalize(h))
                count += 1
                return
            for c in range(1, remaining - (k - len(prefix) - 1) + 1):
                rec(prefix + [c], remaining - c)
        for n in range(k, 11):
            rec([], n)
    assert count > 100


def test_order0_proportionality():
    """Away from the clamps the result is the floor of the proportional share
    plus at most one unit of correction per symbol (here: exactly floor)."""
    h = np.zeros(256, dtype=np.uint64)
    h[:64] = 4096  # 64 * 4096 = n, each share exactly 64
    f = oracle.normalize(h).astype(np.int64)
    assert np.all(f[:64] == 64) and np.all(f[64:] == 0)


def test_rejects_degenerate():
    h = np.zeros(256, dtype=np.uint64)
    h[3] = 10
    with pytest.raises(ValueError):
        oracle.normalize(h)
