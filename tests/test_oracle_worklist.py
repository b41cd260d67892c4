"""Pins for oracle.worklist and oracle.counting against the printed budget of
[P2] §2.2 (Eq 8, Eq 9, the deduplicated total) and brute-force properties."""
import os

import numpy as np
import pytest

from oracle import attention as att
from oracle import counting, worklist as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "budget_counts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


def test_eq8_dense_causal_pairs_from_mask():
    g = _golden()
    n, b = g["n"], g["block"]
    assert counting.dense_causal_pairs(n) == g["dense_causal_pairs"]
    # count the oracle's own mask row by row (every block selected)
    total = 0
    nb = n // b
    for r in range(nb):
        toks = np.arange(r * b, (r + 1) * b)
        total += int(att.allowed_mask(toks, n, b, range(r + 1), True).sum())
    assert total == g["dense_causal_pairs"]


def test_eq9_and_dedup_counts_through_worklist():
    g = _golden()
    nb, b = g["n_blocks"], g["block"]
    rng = np.random.default_rng(0)
    k_b = g["blocks_per_row"]
    rows, rows_dup, meta = [], [], []
    for r in range(nb):
        picks = rng.choice(nb, size=k_b, replace=False)
        rows.append(picks)
        dup = picks.copy()
        dup[-g["overlapping_per_row"]:] = picks[:g["overlapping_per_row"]]   # two overlaps
        rows_dup.append(dup)
        meta.append((nb, r, "count", []))   # the page's count: no causal trimming
    a = wl.build(np.array(rows), meta, k_b)
    d = wl.build(np.array(rows_dup), meta, k_b)
    assert counting.physical_pairs(a["lengths"], b, b) == g["physical_pairs_8_per_row"]
    assert counting.physical_pairs(d["lengths"], b, b) == g["physical_pairs_deduped"]
    # the intra-block waste example: 5 dynamic blocks, 8 useful tokens each
    assert nb * b * g["dynamic_blocks"] * g["useful_tokens_per_block"] == g["dynamic_logical_pairs"]
    assert counting.physical_pairs([g["dynamic_blocks"]] * nb, b, b) == g["dynamic_physical_pairs"]


def test_rows_sorted_unique_forced_and_errors():
    J = np.array([
        [3, 1, 3, -1, 1],        # duplicates, padding
        [-1, -1, -1, -1, -1],    # empty dynamic branch -> forced only
        [9, -5, 2, 7, 0],        # out of range (9 >= 8, -5 < -1), acausal 7 > 2
        [0, 1, 2, 3, 4],
    ])
    meta = [(8, 4, "prefill", [4]), (8, 0, "prefill", [0]), (8, 2, "prefill", [0, 2]),
            (8, 7, "prefill", [0, 7])]
    out = wl.build(J, meta, 7)
    rows = [out["col_idx"][out["row_ptr"][i]:out["row_ptr"][i + 1]].tolist() for i in range(4)]
    assert rows == [[1, 3, 4], [0], [0, 2], [0, 1, 2, 3, 4, 7]]
    assert out["err"] == wl.ERR_RANGE | wl.ERR_ACAUSAL
    # buckets: 3->4, 1->4, 2->4, 6->8 ; NB for width 7 is 2 (4, 8)
    assert out["bucket_ptr"].tolist() == [0, 3, 4]
    assert out["row_perm"].tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("seed", range(4))
def test_bucket_permutation_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, k_b, n_k = 57, 40, 64
    J = rng.integers(-1, n_k, size=(R, k_b))
    J[rng.random((R, k_b)) < 0.6] = -1
    meta = [(n_k, n_k - 1, "prefill", [n_k - 1]) for _ in range(R)]
    out = wl.build(J, meta, k_b + 1)
    lens = out["lengths"]
    sizes = [max(4, 1 << int(np.ceil(np.log2(max(x, 1))))) for x in lens]
    expect = sorted(range(R), key=lambda i: (sizes[i], i))
    assert out["row_perm"].tolist() == expect
    nb = wl.bucket_count(k_b + 1)
    assert nb == 5      # widest possible row 41 -> buckets 4, 8, 16, 32, 64
    counts = [sum(1 for x in sizes if x == 4 << i) for i in range(nb)]
    assert out["bucket_ptr"].tolist() == np.concatenate([[0], np.cumsum(counts)]).tolist()
