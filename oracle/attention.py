"""Oracle: exact attention restricted to the selected key blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method computes exact attention inside the selected blocks ([P2] opening
paragraph: exact QK, causal mask, online softmax and AV in the selected tiles;
[P2] §3.2: O_u = Attn(Q_u, concat K_v, concat V_v) over the candidate set).
For query token i of block r, the attended set is

  A_i = { p : block(p) in W(row), p < length, and p <= i in prefill }

and O_i = sum_{p in A_i} softmax_p(q_i . k_p / sqrt(d)) v_p.

`masked_attention` is the plain definition, written the way [P3] "verifying
the kernel" asks for a reference: materialise the full score rows over every
key, set the entries outside A_i to -inf, then softmax and AV.  A boolean mask
cannot count a duplicated block twice ([P2] §1.2).

`streaming_attention` evaluates the same quantity tile by tile with the
online-softmax merge of [P2] §1.2 Eq (3)-(5), over any tile order and any
grouping into split partials.  It exists to pin the order / split invariance
that [P2] §1.2 and [P3] "sparse softmax numerics" state, and to exercise the
merge rule the GPU decode path uses.
"""
from __future__ import annotations

import numpy as np


def allowed_mask(q_pos: np.ndarray, length: int, b: int, blocks, causal: bool) -> np.ndarray:
    """Boolean [len(q_pos), length]: key p is attended by the query at q_pos[i]."""
    key_pos = np.arange(length)
    in_w = np.isin(key_pos // b, np.asarray(sorted(set(int(x) for x in blocks)), dtype=np.int64))
    mask = np.broadcast_to(in_w[None, :], (len(q_pos), length)).copy()
    if causal:
        mask &= key_pos[None, :] <= np.asarray(q_pos)[:, None]
    return mask


def masked_attention(q_rows, q_pos, k, v, length: int, b: int, blocks, causal: bool):
    """Full score rows, mask, softmax, AV -- for one head and one set of query rows.

    q_rows [m, d]; k, v [>= length, d].  Returns dict with o [m, d], the row max
    m (of the scaled logits), the exp-sum l, lse = m + ln l, and the
    probability matrix p [m, length] (zeros outside A_i).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    kk = np.asarray(k[:length], dtype=np.float64)
    vv = np.asarray(v[:length], dtype=np.float64)
    scale = 1.0 / np.sqrt(q_rows.shape[1])
    s = (q_rows @ kk.T) * scale                     # [P2] Eq 2, every key
    mask = allowed_mask(q_pos, length, b, blocks, causal)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ vv
    return dict(o=o, m=m, l=l, lse=m + np.log(l), p=p)


def _tile_state(q_rows, q_pos, k, v, length, b, j, causal, scale):
    """(m_hat, l_hat, u_hat) of one key block j: the new-block terms of Eq 3-5."""
    lo, hi = j * b, min((j + 1) * b, length)
    s = (q_rows @ np.asarray(k[lo:hi], np.float64).T) * scale
    if causal:
        s = np.where(np.arange(lo, hi)[None, :] <= np.asarray(q_pos)[:, None], s, -np.inf)
    m_hat = s.max(axis=1)
    safe = np.where(np.isfinite(m_hat), m_hat, 0.0)
    e = np.exp(s - safe[:, None])
    return m_hat, e.sum(axis=1), e @ np.asarray(v[lo:hi], np.float64)


def merge(state_a, state_b):
    """Online-softmax merge of [P2] §1.2 Eq (3)-(5) for two partial states."""
    m_a, l_a, u_a = state_a
    m_b, l_b, u_b = state_b
    m = np.maximum(m_a, m_b)                                   # Eq 3
    safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(m_a), np.exp(m_a - safe), 0.0)
    wb = np.where(np.isfinite(m_b), np.exp(m_b - safe), 0.0)
    l = wa * l_a + wb * l_b                                    # Eq 4
    u = wa[:, None] * u_a + wb[:, None] * u_b                  # Eq 5
    return m, l, u


def streaming_attention(q_rows, q_pos, k, v, length: int, b: int, tiles, causal: bool,
                        splits: int = 1):
    """Eq 3-5 over `tiles` in the given order, cut into `splits` contiguous groups.

    Each group is folded tile by tile into its own (m, l, u); the group states
    are then merged by the same rule and the output is u / l.  `tiles` must
    already be deduplicated (the worklist's job).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    scale = 1.0 / np.sqrt(q_rows.shape[1])
    m_rows, d = q_rows.shape[0], q_rows.shape[1]
    empty = (np.full(m_rows, -np.inf), np.zeros(m_rows), np.zeros((m_rows, d)))
    tiles = list(tiles)
    per = -(-len(tiles) // splits) if tiles else 0
    total = empty
    for g in range(splits):
        part = empty
        for j in tiles[g * per:(g + 1) * per]:
            part = merge(part, _tile_state(q_rows, q_pos, k, v, length, b, j, causal, scale))
        total = merge(total, part)
    m, l, u = total
    return u / l[:, None]
