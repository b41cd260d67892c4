"""Oracle: J -> worklist (sort, dedup, force, CSR, length buckets).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows [P2] §1.2 (indices sorted by address; a block entering twice would be
counted twice in the softmax denominator, so duplicates must go before the
kernel), [P2] §3.1 "index-to-kernel acceptance table" (fixed-width J and
CSR row_ptr/col_idx as kernel index forms; 32-bit ids), [P2] §2.1 Eq 7's
capacity buckets and [P3] "from index output to worklist" (sort, dedup,
row pointers and column indices; rows grouped by candidate length).

Per row (rows in (sequence, routing head, query block) row-major order):
  W = ascending unique({j in J_row : j != -1} U F_r)
  invalid entries are dropped and flagged in `err`:
    bit 0  j < -1 or j >= N_k(sequence)
    bit 1  prefill and j > r (a block after the query block: acausal)
  row_ptr   exclusive scan of |W|           ([P2] §3.1 CSR form)
  col_idx   concatenation of the rows' W
  bucket    smallest power of two >= max(|W|, 4), i.e. 4, 8, 16, ...
  bucket_ptr  exclusive scan of rows per bucket, buckets ascending
  row_perm  rows sorted by (bucket ascending, row ascending)

The bucket list has NB entries 4 * 2^i, i < NB, with NB the smallest count
whose last bucket holds the widest possible row (k_b + forced).  The bucket
layout itself is a convention (parity unpinned); dedup and counts are pinned
by the Eq 9 / deduplicated-budget values of [P2] §2.2.
"""
from __future__ import annotations

import numpy as np

ERR_RANGE = 1
ERR_ACAUSAL = 2


def bucket_count(width_max: int) -> int:
    nb = 1
    while 4 * (1 << (nb - 1)) < width_max:
        nb += 1
    return nb


def bucket_index(length: int) -> int:
    size, idx = 4, 0
    while size < max(length, 4):
        size *= 2
        idx += 1
    return idx


def row_set(j_row, n_k: int, r: int, mode: str, forced: list[int]):
    """W for one row and its error bits (see module docstring)."""
    err = 0
    w = set()
    for j in j_row:
        j = int(j)
        if j == -1:
            continue
        if j < -1 or j >= n_k:
            err |= ERR_RANGE
            continue
        if mode == "prefill" and j > r:
            err |= ERR_ACAUSAL
            continue
        w.add(j)
    w.update(forced)
    return sorted(w), err


def build(J_rows, row_meta, width_max: int):
    """Worklist for rows of J.

    J_rows: [R, k_b] ints; row_meta: list of (n_k, r, mode, forced) per row.
    Returns dict(row_ptr, col_idx, row_perm, bucket_ptr, err, lengths).
    """
    R = len(row_meta)
    lengths = np.zeros(R, dtype=np.int64)
    cols = []
    err = 0
    for i in range(R):
        n_k, r, mode, forced = row_meta[i]
        w, e = row_set(J_rows[i], n_k, r, mode, forced)
        err |= e
        lengths[i] = len(w)
        cols.extend(w)
    row_ptr = np.zeros(R + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(lengths)
    nb = bucket_count(width_max)
    bidx = np.array([bucket_index(int(x)) for x in lengths], dtype=np.int64)
    if R and bidx.max() >= nb:
        raise ValueError("row longer than the widest bucket")
    counts = np.bincount(bidx, minlength=nb) if R else np.zeros(nb, np.int64)
    bucket_ptr = np.zeros(nb + 1, dtype=np.int64)
    bucket_ptr[1:] = np.cumsum(counts)
    row_perm = np.array(sorted(range(R), key=lambda i: (bidx[i], i)), dtype=np.int64)
    return dict(row_ptr=row_ptr, col_idx=np.array(cols, dtype=np.int64),
                row_perm=row_perm, bucket_ptr=bucket_ptr, err=err, lengths=lengths)
