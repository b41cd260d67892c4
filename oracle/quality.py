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

Readings (parity unpinned): the dense reference is causal attention over the
whole sequence; a padded key never counts.
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
