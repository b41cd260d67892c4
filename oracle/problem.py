"""Oracle: whole-problem drivers over per-sequence arrays.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rows are enumerated in (sequence, routing head, query block) row-major order:
the order of J's leading dimensions [B, H, N_q, k_b] in [P2]'s opening
paragraph, with sequences of a packed batch concatenated.  In decode each
(sequence, routing head) is one row whose current block is the last one.

Pinned (tests/test_oracle_problem.py): row_table against a hand-written row
list for ragged sequences (prefill and decode); the decode branch of
attention_rows against torch's fp64 SDPA over all cached keys (partial last
blocks, mixed cache lengths) and against plain loops on a sparse block list;
a packed ragged batch against its sequences done one at a time; a packed
batch with empty sequences against the same batch without them.

Inputs are per-sequence float64 arrays:
  qs[s]  [Hq, n_q_tokens, d]   (decode: n_q_tokens = 1)
  ks[s], vs[s]  [Hkv, n_k_tokens, d]
  lengths[s]    valid tokens of sequence s (decode: cached length L)
"""
from __future__ import annotations

import numpy as np

from . import attention as att
from . import routing
from . import worklist as wl


def row_table(lengths, b: int, mode: str, route_heads: int):
    """[(s, h_r, r, n_k)] in row order."""
    rows = []
    for s, length in enumerate(lengths):
        n_k = routing.num_blocks(length, b)
        n_rows = n_k if mode == "prefill" else 1
        for h in range(route_heads):
            for r in range(n_rows):
                rows.append((s, h, r if mode == "prefill" else n_k - 1, n_k))
    return rows


def row_meta(lengths, b: int, mode: str, route_heads: int, forced_first: bool, window: int = 1):
    """(n_k, r, mode, F_r) per row, for the worklist builder."""
    return [(n_k, r, mode, routing.forced_blocks(r, n_k, mode, forced_first, window))
            for (_s, _h, r, n_k) in row_table(lengths, b, mode, route_heads)]


def route(qs, ks, lengths, b, mode, qpool, share_gqa, select, k_b, k_min, tau_rel,
          forced_first, seqs=None, window: int = 1, kpool: str = "mean"):
    """J rows [R, k_b] plus per-row (g, C_r, F_r) for the chosen sequences.

    seqs: subset of sequence ids to route (others left as None rows).
    Returns (J_rows or None-filled list, scores list aligned with row_table).
    """
    first = next(i for i, x in enumerate(qs) if x is not None)
    hq, hkv = qs[first].shape[0], ks[first].shape[0]
    route_heads = hkv if share_gqa else hq
    table = row_table(lengths, b, mode, route_heads)
    j_rows = [None] * len(table)
    scores = [None] * len(table)
    index = {(s, h, r): i for i, (s, h, r, _n) in enumerate(table)}
    for s, length in enumerate(lengths):
        if seqs is not None and s not in seqs:
            continue
        if length == 0:   # a sequence of no tokens has no query blocks, so no rows
            continue
        J, sc = routing.route_sequence(qs[s], ks[s], length, b, mode, qpool, share_gqa,
                                       select, k_b, k_min, tau_rel, forced_first,
                                       return_scores=True, window=window, kpool=kpool)
        for h in range(route_heads):
            for r in range(J.shape[1]):
                rr = r if mode == "prefill" else routing.num_blocks(length, b) - 1
                i = index[(s, h, rr)]
                j_rows[i] = J[h, r]
                scores[i] = sc[h][r]
    return j_rows, scores


def worklist(j_rows, lengths, b, mode, route_heads, forced_first, width_max, window: int = 1):
    meta = row_meta(lengths, b, mode, route_heads, forced_first, window)
    return wl.build(np.asarray(j_rows, dtype=np.int64).reshape(len(meta), -1), meta, width_max)


def attention_rows(qs, ks, vs, lengths, b, mode, share_gqa, row_ids, row_blocks):
    """Masked attention for selected rows.

    row_blocks[i]: the worklist set W of row i.  Returns {row id: list over the
    row's query heads of (head, query token indices, masked_attention dict)}.
    """
    first = next(i for i, x in enumerate(qs) if x is not None)
    hq, hkv = qs[first].shape[0], ks[first].shape[0]
    group = hq // hkv
    route_heads = hkv if share_gqa else hq
    table = row_table(lengths, b, mode, route_heads)
    out = {}
    for i in row_ids:
        s, h, r, _n = table[i]
        length = lengths[s]
        heads = list(range(h * group, (h + 1) * group)) if share_gqa else [h]
        res = []
        for hh in heads:
            kvh = hh // group
            if mode == "prefill":
                toks = np.arange(r * b, min((r + 1) * b, length))
                q_rows = qs[s][hh, toks]
                q_pos = toks
                causal = True
            else:
                toks = np.array([0])
                q_rows = qs[s][hh, 0:1]
                q_pos = np.array([length - 1])
                causal = False
            res.append((hh, toks, att.masked_attention(q_rows, q_pos, ks[s][kvh], vs[s][kvh],
                                                       length, b, row_blocks[i], causal)))
        out[i] = res
    return out
