"""Pins of the router-quality oracle (oracle/quality.py): coverage is 1 for the
full causal set, equals a plain-loop softmax mass on tiny inputs, equals
1 - delta of the missed-mass bound, and adds up over disjoint block sets;
recall on hand-made sets."""
import math

import numpy as np

from oracle import attention, quality


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_full_causal_set_has_coverage_one():
    n, d, b = 40, 8, 8
    q, k = _rand((n, d), 1), _rand((n, d), 2)
    pos = np.arange(n)
    c = quality.coverage(q, pos, k, n, b, list(range(5)))
    assert np.max(np.abs(c - 1.0)) < 1e-12


def test_coverage_equals_plain_loops_tiny():
    n, d, b = 9, 3, 4
    q, k = _rand((n, d), 3), _rand((n, d), 4)
    blocks = [0, 2]
    pos = np.arange(n)
    c = quality.coverage(q, pos, k, n, b, blocks)
    for i in range(n):
        w = [math.exp(sum(q[i, e] * k[p, e] for e in range(d)) / math.sqrt(d)) for p in range(i + 1)]
        inside = sum(w[p] for p in range(i + 1) if p // b in blocks)
        assert abs(c[i] - inside / sum(w)) < 1e-12


def test_coverage_is_one_minus_missed_mass_and_additive():
    n, d, b = 48, 6, 8
    q, k = _rand((n, d), 5), _rand((n, d), 6)
    pos = np.arange(n)
    a, rest = [0, 3], [1, 2, 4, 5]
    ca = quality.coverage(q, pos, k, n, b, a)
    cr = quality.coverage(q, pos, k, n, b, rest)
    assert np.max(np.abs(ca + cr - 1.0)) < 1e-12            # disjoint sets add up
    dense = attention.masked_attention(q, pos, k, k, n, b, list(range(6)), causal=True)
    inside = attention.allowed_mask(pos, n, b, a, causal=True)
    delta = 1.0 - np.sum(np.where(inside, dense["p"], 0.0), axis=1)
    assert np.max(np.abs(ca - (1.0 - delta))) < 1e-12
    # a padded key never counts: keys past the length do not change coverage
    k2 = np.vstack([k, np.full((5, d), 50.0)])
    assert np.array_equal(quality.coverage(q, pos, k2, n, b, a), ca)


def test_recall():
    assert quality.recall([3, 5, 7], [5, 7]) == 1.0
    assert quality.recall([3, 5], [5, 7, 9, 11]) == 0.25
    assert quality.recall([1], []) == 1.0
