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


def _plain_probs(q, k, i, d):
    """Dense causal softmax of query i over keys 0 .. i, in plain loops."""
    w = [math.exp(sum(q[i, e] * k[p, e] for e in range(d)) / math.sqrt(d)) for p in range(i + 1)]
    z = sum(w)
    return [x / z for x in w]


def test_row_quality_against_plain_loops_tiny():
    n, d, b = 11, 3, 4
    q, k, v = _rand((n, d), 7), _rand((n, d), 8), _rand((n, d), 9)
    blocks = [0, 2]
    pos = np.arange(n)
    res = quality.row_quality(q, pos, k, v, n, b, blocks, ts=(1, 3, 20))
    for i in range(n):
        p = _plain_probs(q, k, i, d)
        inside = [pp // b in blocks for pp in range(i + 1)]
        c = sum(p[pp] for pp in range(i + 1) if inside[pp])
        assert abs(res["coverage"][i] - c) < 1e-12
        o_s = [sum(p[pp] / c * v[pp, e] for pp in range(i + 1) if inside[pp]) for e in range(d)]
        o_d = [sum(p[pp] * v[pp, e] for pp in range(i + 1)) for e in range(d)]
        assert np.max(np.abs(res["o_sparse"][i] - o_s)) < 1e-12
        assert np.max(np.abs(res["o_dense"][i] - o_d)) < 1e-12
        nd = math.sqrt(sum(x * x for x in o_d))
        ns = math.sqrt(sum(x * x for x in o_s))
        err = math.sqrt(sum((a - b_) ** 2 for a, b_ in zip(o_d, o_s)))
        assert abs(res["rel_err"][i] - err / nd) < 1e-12
        assert abs(res["cosine"][i] - sum(a * b_ for a, b_ in zip(o_d, o_s)) / (nd * ns)) < 1e-12
        ranked = sorted(range(i + 1), key=lambda pp: (-p[pp], pp))
        assert bool(res["top1_routed"][i]) == inside[ranked[0]]
        for t in (1, 3, 20):
            g = ranked[:min(t, i + 1)]
            hit = [pp for pp in g if inside[pp]]
            assert abs(res[f"recall@{t}"][i] - len(hit) / len(g)) < 1e-15
            assert abs(res[f"lost@{t}"][i] - sum(p[pp] for pp in g if not inside[pp])) < 1e-12
            assert abs(res[f"moved@{t}"][i] - sum(abs(p[pp] / c - p[pp]) for pp in hit)) < 1e-12


def test_row_quality_full_set_and_bounds():
    n, d, b = 64, 8, 8
    q, k, v = _rand((n, d), 10), _rand((n, d), 11), _rand((n, d), 12)
    pos = np.arange(n)
    full = quality.row_quality(q, pos, k, v, n, b, list(range(8)))
    assert np.max(np.abs(full["coverage"] - 1.0)) < 1e-12
    for t in (8, 64):
        assert np.all(full[f"recall@{t}"] == 1.0)
        assert np.max(full[f"lost@{t}"]) == 0.0 and np.max(full[f"moved@{t}"]) < 1e-14
    assert np.max(full["rel_err"]) < 1e-12 and np.max(np.abs(full["cosine"] - 1.0)) < 1e-12
    assert full["top1_routed"].all()
    # a sparse set: the output is masked attention over the set, and the error obeys
    # |o_dense - o_sparse|_inf <= 2 max|v| delta ([P2] §3.1, delta = 1 - C)
    blocks = [0, 3, 7]
    res = quality.row_quality(q, pos, k, v, n, b, blocks)
    ref = attention.masked_attention(q, pos, k, v, n, b, blocks, causal=True)
    attended = attention.allowed_mask(pos, n, b, blocks, causal=True).any(axis=1)
    assert np.max(np.abs(res["o_sparse"][attended] - ref["o"][attended])) < 1e-12
    assert np.max(np.abs(res["coverage"] - quality.coverage(q, pos, k, n, b, blocks))) < 1e-12
    delta = 1.0 - res["coverage"][attended]
    gap = np.max(np.abs(res["o_dense"][attended] - res["o_sparse"][attended]), axis=1)
    assert np.all(gap <= 2 * np.max(np.abs(v)) * delta + 1e-12)
    # lost mass is part of the missed mass; moved weight is the kept teacher mass times 1/C - 1
    for t in (8, 64):
        assert np.all(res[f"lost@{t}"][attended] <= delta + 1e-12)
        assert np.all(res[f"recall@{t}"] <= 1.0)


def test_row_quality_decode_query_and_ties():
    # decode: one query at position L - 1 is the prefill row of the last token
    n, d, b = 50, 4, 8
    q, k, v = _rand((n, d), 13), _rand((n, d), 14), _rand((n, d), 15)
    blocks = [0, 6]
    last = quality.row_quality(q[-1:], np.array([n - 1]), k, v, n, b, blocks)
    allq = quality.row_quality(q, np.arange(n), k, v, n, b, blocks)
    for key in ("coverage", "recall@8", "lost@8", "moved@8", "rel_err", "cosine"):
        assert abs(last[key][0] - allq[key][-1]) < 1e-12, key
    # equal keys tie: the teacher takes the lower positions
    kt = np.zeros((16, d))
    qt = np.ones((1, d))
    res = quality.row_quality(qt, np.array([15]), kt, v[:16], 16, 4, [2, 3], ts=(4, 8))
    assert res["recall@4"][0] == 0.0 and res["recall@8"][0] == 0.0   # teacher = keys 0..7
    assert not res["top1_routed"][0]
    assert abs(res["lost@4"][0] - 4 / 16) < 1e-15


def test_teacher_is_the_sorted_prefix():
    rng = np.random.default_rng(3)
    for n, t in ((10, 3), (40, 40), (5, 9), (64, 8)):
        p = np.round(rng.random(n), 1)        # many exact ties
        ranked = sorted(range(n), key=lambda i: (-p[i], i))[:min(t, n)]
        assert sorted(quality.teacher(p, t).tolist()) == sorted(ranked)
