"""Oracle: router-quality measures.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P2] §4 measures how much of the dense attention a block selection keeps:
coverage (Eq 10) is the dense causal softmax mass of query i that falls on
the keys the sparse row attends, and delta_i = 1 - C_i is the mass it misses,
which bounds the output error (||o_dense - o_sparse|| <= 2 V delta_i, pinned
in the attention tests).  [P2] §4 also asks whether the router finds the
blocks that matter; with planted inputs the relevant blocks are known, and
recall is the fraction of them a row keeps.

  coverage  C_i = sum over keys p in A_i of softmax_p(q_i . k_p / sqrt(d)),
            the softmax taken over every causal key of the sequence  ([P2] Eq 10)
  recall    |W_r intersect R_r| / |R_r| for the relevant blocks R_r a row could
            select (planted blocks j < r); 1 when R_r is empty

  row_quality  the per-query report of [P2] §3.1's second validation layer
            for one row: coverage, token recall@t against the dense top-t
            teacher, the teacher's misses split into "block not routed" and
            "weight moved inside a selected block", and the dense-vs-sparse
            output error (relative error and cosine)

Readings: the dense reference is causal attention over the whole sequence (a
decode query attends every cached key); a padded key never counts.  The
teacher G_i holds the t causal keys of largest dense probability, ties to
the lower position, t clipped to the number of causal keys.  The sparse
attention is exact over the selected blocks, so a teacher key outside them
loses its whole dense weight, and one inside has its weight divided by C_i.

Pinned (tests/test_oracle_quality.py): coverage and row_quality against plain
loops on tiny inputs, the full causal set (coverage 1, nothing lost or moved,
zero error), disjoint sets adding up, the 2 V delta output bound, the sparse
output against masked_attention, ties to the lower position, the teacher
against a full sort with many exact ties, and recall on hand-made sets.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask, masked_attention


def coverage(q_rows, q_pos, k, length: int, b: int, blocks) -> np.ndarray:
    """C_i of [P2] Eq 10 for each query row: dense causal probability mass on
    the keys of `blocks` (the row's worklist set) that query i may attend."""
    n_blk = -(-length // b)
    dense = masked_attention(q_rows, q_pos, k, k, length, b, list(range(n_blk)), causal=True)
    inside = allowed_mask(q_pos, length, b, blocks, causal=True)
    return np.sum(np.where(inside, dense["p"], 0.0), axis=1)


def recall(selected, relevant) -> float:
    """Fraction of the relevant blocks that the row selected (1 when none are relevant)."""
    rel = set(int(x) for x in relevant)
    if not rel:
        return 1.0
    return len(rel & set(int(x) for x in selected)) / len(rel)


def teacher(p_row, t: int) -> np.ndarray:
    """Positions of the t largest entries of p_row, equal values taken from the
    lower position up (all of them when t >= len(p_row))."""
    n = len(p_row)
    if t >= n:
        return np.arange(n)
    tau = np.partition(p_row, n - t)[n - t]     # the t-th largest value
    above = np.nonzero(p_row > tau)[0]
    tied = np.nonzero(p_row == tau)[0][:t - len(above)]
    return np.concatenate([above, tied])


def row_quality(q_rows, q_pos, k, v, length: int, b: int, blocks, ts=(8, 64)) -> dict:
    """Per-query quality of one row's selected blocks against dense causal attention.

    q_rows [m, d] (one query head), q_pos their positions (decode: length - 1),
    k, v [>= length, d] of the row's KV head, `blocks` the row's worklist set.
    Returns per-query arrays: coverage (Eq 10); for each t in ts, recall@t =
    |G_i & N(i)| / |G_i|, lost@t = dense mass of the teacher keys outside the
    selected blocks (block not routed), moved@t = sum over the teacher keys
    inside of |p_sparse - p_dense| (weight moved inside a selected block);
    top1_routed (the dense arg-max key is attended); rel_err = |o_dense -
    o_sparse| / |o_dense| and cosine(o_dense, o_sparse) (Euclidean norms);
    o_dense and o_sparse [m, d].
    """
    q_pos = np.asarray(q_pos)
    hi = min(int(q_pos.max()) + 1, length)   # keys past the last query are causally masked
    n_blk = -(-hi // b)
    dense = masked_attention(q_rows, q_pos, k, v, hi, b, list(range(n_blk)), causal=True)
    p = dense["p"]
    inside = allowed_mask(q_pos, hi, b, blocks, causal=True)
    cov = np.sum(np.where(inside, p, 0.0), axis=1)
    p_sparse = np.where(inside, p / cov[:, None], 0.0)
    vv = np.asarray(v[:hi], np.float64)
    o_dense = dense["o"]
    o_sparse = p_sparse @ vv
    n_causal = np.minimum(q_pos + 1, hi)
    out = dict(coverage=cov, o_dense=o_dense, o_sparse=o_sparse)
    rows = np.arange(p.shape[0])
    for t in ts:
        rec, lost, moved = np.zeros(len(rows)), np.zeros(len(rows)), np.zeros(len(rows))
        for i in rows:
            g = teacher(p[i, :n_causal[i]], t)
            hit = inside[i, g]
            rec[i] = hit.sum() / len(g)
            lost[i] = p[i, g[~hit]].sum()
            moved[i] = np.abs(p_sparse[i, g[hit]] - p[i, g[hit]]).sum()
        out[f"recall@{t}"], out[f"lost@{t}"], out[f"moved@{t}"] = rec, lost, moved
    out["top1_routed"] = inside[rows, np.argmax(p, axis=1)]   # argmax: the first (lowest) of equal maxima
    diff = np.linalg.norm(o_dense - o_sparse, axis=1)
    nd, ns = np.linalg.norm(o_dense, axis=1), np.linalg.norm(o_sparse, axis=1)
    out["rel_err"] = diff / nd
    out["cosine"] = np.sum(o_dense * o_sparse, axis=1) / (nd * ns)
    return out
