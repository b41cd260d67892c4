"""Oracle: decode-cache maintenance (append K/V rows, keep block summaries).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P2] §3.1 treats block summaries as cache state: in decode they are kept with
the KV cache and updated as keys arrive rather than recomputed by a scan over
the history ([P2] §3.1 Eq 11: a running sum s_j <- s_j + k_t over the r_j valid
keys of block j, and c_j = s_j / r_j).  This module states what appending new
tokens to a cache must produce:

  cache     rows [L0, L0 + n) of every (sequence, KV head) receive the new K/V
            rows, in order; nothing else in the cache changes
  summary   every block j touched by the append holds the mean of all its
            valid keys afterwards: the same value as block_summaries() over
            the grown cache ([P2] Eq 6 mean, Eq 11 count r_j)

`append_update` is Eq 11 applied to a chunk of keys at once: the block's
running sum r_j * c_j (the summary times its count) plus the chunk's sum,
divided by the new count.  It is pinned against the batch mean of the grown
block and against a key-by-key Eq 11 stream (`routing.incremental_summary`).

Readings where the pages are silent (parity unpinned; both sides follow them):
  * A decode cache stores every sequence at one common length (the same
    uniform length the decode attention takes); an append adds the same
    number of tokens to every sequence.
  * The stored state is the mean c_j, not the sum s_j: the update multiplies
    back by the old count r_j (a block with r_j = 0 starts from the new keys).
"""
from __future__ import annotations

import numpy as np

from .routing import block_summaries, num_blocks


def append_update(c_old: np.ndarray, r_old: int, new_keys: np.ndarray, kpool: str = "mean") -> np.ndarray:
    """Summary of a block after `new_keys` join its r_old valid keys.

    [P2] §3.1 Eq 11 over a chunk: s = r_old * c_old + sum(new_keys),
    c_new = s / (r_old + len(new_keys)).  With r_old = 0 the old summary is
    ignored (the block had no valid key).  Max-pooled summaries (kpool
    "max") keep the per-dimension maximum: c_new = max(c_old, max(new_keys)),
    again ignoring c_old when r_old = 0.
    """
    n = new_keys.shape[0]
    if n == 0:
        return np.asarray(c_old, dtype=np.float64).copy()
    if kpool == "max":
        m = new_keys.astype(np.float64).max(axis=0)
        return np.maximum(m, np.asarray(c_old, dtype=np.float64)) if r_old > 0 else m
    s = new_keys.astype(np.float64).sum(axis=0)
    if r_old > 0:
        s = s + r_old * np.asarray(c_old, dtype=np.float64)
    return s / (r_old + n)


def touched_blocks(len0: int, n_new: int, b: int) -> range:
    """Blocks that receive at least one of the tokens [len0, len0 + n_new)."""
    if n_new <= 0:
        return range(0)
    return range(len0 // b, (len0 + n_new - 1) // b + 1)


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, summaries: np.ndarray, len0: int,
              k_new: np.ndarray, v_new: np.ndarray, b: int,
              kpool: str = "mean"):
    """Append n new rows to one (sequence, KV head) of a decode cache.

    k_cache, v_cache: [capacity, d]; summaries: [ceil(capacity / b), d] whose
    blocks below ceil(len0 / b) hold the means of the cached keys;
    k_new, v_new: [n, d].  Returns new (k_cache, v_cache, summaries) arrays;
    the inputs are not modified.  Each touched block is updated by
    `append_update` with the new keys that fall into it.
    """
    n = k_new.shape[0]
    assert len0 + n <= k_cache.shape[0], "append past the cache capacity"
    k2, v2, c2 = k_cache.copy(), v_cache.copy(), summaries.astype(np.float64).copy()
    k2[len0:len0 + n] = k_new
    v2[len0:len0 + n] = v_new
    for j in touched_blocks(len0, n, b):
        lo, hi = j * b, (j + 1) * b
        r_old = max(0, min(hi, len0) - lo)                 # valid keys before the append
        t0, t1 = max(lo, len0), min(hi, len0 + n)          # new tokens inside block j
        c2[j] = append_update(c2[j], r_old, k_new[t0 - len0:t1 - len0], kpool)
    return k2, v2, c2


def summaries_after(k_cache: np.ndarray, length: int, b: int, kpool: str = "mean") -> np.ndarray:
    """What the summaries of a cache of `length` valid rows must equal: the
    batch block summaries of [P2] Eq 6 (`routing.block_summaries`, mean or
    per-dimension max)."""
    return block_summaries(k_cache, length, b, kpool)


def blocks_after(length: int, b: int) -> int:
    """Summary slots in use after the cache holds `length` rows."""
    return num_blocks(length, b)
