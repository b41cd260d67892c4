"""Oracle: routing (block summaries, pooled scores, candidates, selection).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What routing computes, following [P2] §2.1 Eq (6) and Eq (7), the causal
boundary paragraph of [P2] §2.1, and [P2] §4.1:

  summary   c_j = mean of the valid keys of key block j          ([P2] Eq 6)
  score     g_rj = pool over the queries of block r of q . c_j    ([P2] Eq 6)
            (no 1/sqrt(d) factor: Eq 6 pools the raw dot product)
  GQA       routing per KV head averages the per-query-head pooled
            score over the head group                             ([P2] §4)
  causal    only complete history blocks j < r are candidates; the current
            block is always added as a fixed local branch and is
            never scored                                          ([P2] §2.1, §4.1)
  select    fixed top-k_b (k_b counts the forced blocks), or Eq 7's
            clipped threshold count; ties by lower block id       ([P2] Eq 7; [P1])

Readings where the pages are silent (parity unpinned; both sides follow them):
  * k_b is the total per-row budget including forced blocks.
  * A local window of W blocks forces the current block and the W - 1 before
    it; they are excluded from scoring like the current block ([P2] §3.2:
    the local branch is fixed, the dynamic branch picks among the rest).
  * "query pool = max" is the max over per-query *scores*, not an elementwise
    max of query vectors ([P2] §3.2 warns the latter builds a vector that
    does not exist).
  * Eq 7: tau_r = max over the non-forced candidates minus tau_rel; forced
    blocks count as selected; ">=" is inclusive.
  * decode: the current block is the last cached block N_k - 1; candidates
    are 0 .. N_k - 2.
"""
from __future__ import annotations

import numpy as np


def num_blocks(length: int, b: int) -> int:
    """N = ceil(length / b)  ([P2] opening paragraph: N_q = ceil(n / b))."""
    return -(-length // b)


def block_summaries(k: np.ndarray, length: int, b: int, kpool: str = "mean") -> np.ndarray:
    """Key summaries c_j for one (sequence, KV head).

    k: [n_tokens >= length, d].  Block j covers tokens [j*b, min((j+1)*b, length));
    padding past `length` never enters a summary ([P2] §4.1).
    kpool "mean": the block mean of [P2] Eq 6; a partial block divides by its
    own count (the r_j of [P2] §3.1 Eq 11).
    kpool "max": the per-dimension maximum over the block's valid keys, the
    max-pooled summary that [P2] §2.1 and §4 set against the mean (it keeps
    each dimension's extreme, possibly taken from different keys).
    Pinned: the incremental Eq 11 form, a hand-computed mean, and for max a
    brute-force loop, a two-key fixture and an upper-bound property in tests.
    """
    if kpool not in ("mean", "max"):
        raise ValueError(kpool)
    n_blk = num_blocks(length, b)
    c = np.zeros((n_blk, k.shape[1]), dtype=np.float64)
    for j in range(n_blk):
        lo = j * b
        hi = min((j + 1) * b, length)
        blk = k[lo:hi].astype(np.float64)
        c[j] = blk.sum(axis=0) / (hi - lo) if kpool == "mean" else blk.max(axis=0)
    return c


def incremental_summary(keys: np.ndarray) -> np.ndarray:
    """Eq 11 of [P2] §3.1: s <- s + k_t, c = s / r after each appended key.

    Returns the summary after every prefix (row t = summary of keys[0..t]).
    Used to pin `block_summaries` (a batch mean must equal the streamed one).
    """
    s = np.zeros(keys.shape[1], dtype=np.float64)
    out = np.zeros_like(keys, dtype=np.float64)
    for t in range(keys.shape[0]):
        s = s + keys[t]
        out[t] = s / (t + 1)
    return out


def forced_blocks(r: int, n_blocks: int, mode: str, forced_first: bool, window: int = 1) -> list[int]:
    """Forced set F_r: the local window ending at the current block, plus block 0 when asked.

    Prefill: the current block of query block r is r ([P2] §2.1 causal boundary).
    Decode: the current block is the last cached block n_blocks - 1.
    [P2] §3.2 builds a row as the union of a local branch (the most recent
    blocks), a global branch (the first block, a sink) and the dynamic top-k
    branch; the local and global branches are fixed, never scored.  `window`
    is the local branch's length in blocks, the current one included (1 = the
    current block only).
    """
    cur = r if mode == "prefill" else n_blocks - 1
    f = set(range(max(cur - max(window, 1) + 1, 0), cur + 1))
    if forced_first:
        f.add(0)
    return sorted(f)


def candidate_blocks(r: int, n_blocks: int, mode: str, forced: list[int]) -> list[int]:
    """C_r: complete history blocks that are not forced ([P2] §2.1, §4.1)."""
    history = range(r) if mode == "prefill" else range(n_blocks - 1)
    fs = set(forced)
    return [j for j in history if j not in fs]


def pooled_scores(q_group: list[np.ndarray], c: np.ndarray, qpool: str) -> np.ndarray:
    """g_j for one query block, all key blocks j (Eq 6 of [P2] §2.1, GQA rule of [P2] §4).

    q_group: one [n_valid_queries, d] array per query head routed together
    (one head for per-head routing; the G heads of a KV head when shared).
    Per head: score every (query, block) pair q_i . c_j, pool over the queries
    (mean or max).  Shared routing then averages the per-head pooled scores.
    """
    per_head = []
    for qh in q_group:
        s = qh.astype(np.float64) @ c.T            # [n_queries, n_blocks]
        if qpool == "mean":
            per_head.append(s.mean(axis=0))
        elif qpool == "max":
            per_head.append(s.max(axis=0))
        else:
            raise ValueError(qpool)
    return np.mean(np.stack(per_head, axis=0), axis=0)


def budget(g: np.ndarray, cands: list[int], forced: list[int], select: str,
           k_b: int, k_min: int, tau_rel: float) -> int:
    """K_r: total selected blocks for the row (forced included).

    top-k: K_r = k_b.  threshold ([P2] Eq 7 with a relative-to-max tau):
    tau = max_{j in C} g_j - tau_rel;  count = |F| + #{j in C : g_j >= tau};
    K_r = min(k_b, max(k_min, count)).
    """
    if select == "topk":
        return k_b
    if select != "threshold":
        raise ValueError(select)
    if cands:
        tau = max(g[j] for j in cands) - tau_rel
        above = sum(1 for j in cands if g[j] >= tau)
    else:
        above = 0
    count = len(forced) + above
    return min(k_b, max(k_min, count))


def select_row(g: np.ndarray, cands: list[int], forced: list[int], select: str,
               k_b: int, k_min: int, tau_rel: float) -> list[int]:
    """One J row: forced blocks (ascending), then the top D candidates, -1 padded.

    D = min(max(K_r - |F|, 0), |C|); candidates ranked by (score descending,
    block id ascending) -- the stable tie rule of [P1]'s top-k note and the
    "ties broken by lower index" setting.  Pinned against brute-force subset
    enumeration in tests.
    """
    k_r = budget(g, cands, forced, select, k_b, k_min, tau_rel)
    d_r = min(max(k_r - len(forced), 0), len(cands))
    ranked = sorted(cands, key=lambda j: (-g[j], j))
    row = list(forced) + ranked[:d_r]
    if len(row) > k_b:
        raise ValueError("forced blocks exceed the row width")
    return row + [-1] * (k_b - len(row))


def route_sequence(q: np.ndarray, k: np.ndarray, length: int, b: int, mode: str,
                   qpool: str, share_gqa: bool, select: str, k_b: int, k_min: int,
                   tau_rel: float, forced_first: bool, return_scores: bool = False, window: int = 1,
                   kpool: str = "mean"):
    """J for one sequence: [H_r, N_q, k_b] int64 (N_q = 1 in decode).

    q: [Hq, n_q_tokens, d] (prefill: n_q_tokens >= length; decode: 1 query);
    k: [Hkv, n_k_tokens, d] with `length` valid keys (decode: cached length L).
    Returns (J, scores) with scores[h_r][r] = (g over all blocks, C_r, F_r)
    when return_scores is set, for tie-band checks.
    """
    hq, hkv = q.shape[0], k.shape[0]
    group = hq // hkv
    n_blk = num_blocks(length, b)
    summaries = [block_summaries(k[h], length, b, kpool) for h in range(hkv)]
    route_heads = hkv if share_gqa else hq
    n_rows = n_blk if mode == "prefill" else 1
    J = np.full((route_heads, n_rows, k_b), -1, dtype=np.int64)
    scores = [[None] * n_rows for _ in range(route_heads)]
    for hr in range(route_heads):
        if share_gqa:
            heads = list(range(hr * group, (hr + 1) * group))
            kvh = hr
        else:
            heads = [hr]
            kvh = hr // group
        # every (query, block) score of every head at once, then pool per query block
        pooled = []
        for h in heads:
            n_tok = length if mode == "prefill" else 1
            s = q[h, :n_tok].astype(np.float64) @ summaries[kvh].T     # [tokens, N]
            rows = []
            for r in range(n_rows):
                lo, hi = (r * b, min((r + 1) * b, length)) if mode == "prefill" else (0, 1)
                rows.append(s[lo:hi].mean(axis=0) if qpool == "mean" else s[lo:hi].max(axis=0))
            pooled.append(np.stack(rows))
        g_rows = np.mean(np.stack(pooled), axis=0)                      # mean over the head group
        for r in range(n_rows):
            cur = r if mode == "prefill" else n_blk - 1
            forced = forced_blocks(cur, n_blk, mode, forced_first, window)
            cands = candidate_blocks(cur, n_blk, mode, forced)
            g = g_rows[r]
            J[hr, r] = select_row(g, cands, forced, select, k_b, k_min, tau_rel)
            scores[hr][r] = (g, cands, forced)
    if return_scores:
        return J, scores
    return J
