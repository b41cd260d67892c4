"""Oracle: work counts in the units of [P2] §2.2 "a recomputable block budget".

TEST INFRASTRUCTURE ONLY (see the package docstring).

  dense causal token pairs      n (n + 1) / 2                       ([P2] Eq 8)
  physical pairs of a worklist  sum over rows of |W_row| * b_q * b_k ([P2] Eq 9,
                                counted the page's way: full rectangles, no causal
                                triangle, unique tiles only)
  effective pairs               pairs a query actually attends (diagonal tile
                                counts its lower triangle only)

Pinned in tests: dense_causal_pairs and physical_pairs against the values the
page prints (Eq 8, Eq 9 and the deduplicated total); effective_pairs_prefill
against Eq 8 with every causal block listed and the closed form N b (b + 1) / 2
with the diagonal alone.
"""
from __future__ import annotations

import numpy as np


def dense_causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def physical_pairs(row_lengths, b_q: int, b_k: int) -> int:
    return int(np.sum(np.asarray(row_lengths, dtype=np.int64))) * b_q * b_k


def effective_pairs_prefill(rows, length: int, b: int) -> int:
    """Attended (query, key) pairs for prefill rows given as (r, W) tuples."""
    total = 0
    for r, w in rows:
        for j in w:
            for i in range(r * b, min((r + 1) * b, length)):
                lo, hi = j * b, min((j + 1) * b, length)
                total += max(0, min(hi, i + 1) - lo)
    return total
