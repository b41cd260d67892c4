"""Pins for oracle.problem (row order, decode branch, packed batches) and
oracle.counting.effective_pairs_prefill, against things other than the oracle.

* row_table for two ragged sequences and two heads equals a hand-written list
  of (s, h, r, n_k) in the (sequence, routing head, query block) order of J's
  leading dimensions [B, H, N_q, k_b] ([P2] opening paragraph); decode has one
  row per (sequence, head) whose block is the last cached one
* the decode branch of attention_rows with every cached block listed equals
  torch's fp64 SDPA of the single query over all L cached keys (no causal
  mask: the query is the newest token, [P2] §2.2 decode), for caches with a
  partial last block and of different lengths in one batch
* the decode branch on a sparse block list equals a plain-loop softmax over
  exactly the keys of the listed blocks
* a packed 3-sequence ragged batch routed, worklisted and attended as one
  problem equals each sequence done alone, concatenated in row order; a
  packed batch with empty sequences equals the batch without them
* effective_pairs_prefill with every causal block listed equals Eq 8's
  n (n + 1) / 2 printed for n = 8192 ([P2] §2.2 "a recomputable block
  budget"), and with the diagonal block alone the closed form N b (b + 1) / 2
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import counting, problem, routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_row_table_hand_written_order():
    # lengths 130 (3 blocks of 64, the last partial) and 64 (1 block), 2 heads
    got = problem.row_table([130, 64], 64, "prefill", 2)
    want = [(0, 0, 0, 3), (0, 0, 1, 3), (0, 0, 2, 3),
            (0, 1, 0, 3), (0, 1, 1, 3), (0, 1, 2, 3),
            (1, 0, 0, 1),
            (1, 1, 0, 1)]
    assert got == want
    got_d = problem.row_table([130, 64, 1], 64, "decode", 2)
    want_d = [(0, 0, 2, 3), (0, 1, 2, 3), (1, 0, 0, 1), (1, 1, 0, 1), (2, 0, 0, 1), (2, 1, 0, 1)]
    assert got_d == want_d


@pytest.mark.parametrize("lengths,hq,hkv,d,b", [([130], 4, 2, 8, 64), ([1, 5, 64, 200], 2, 1, 16, 64),
                                                ([37, 16], 3, 3, 4, 8)])
def test_decode_all_blocks_equals_sdpa(lengths, hq, hkv, d, b):
    qs = [_rand((hq, 1, d), 10 + s) for s in range(len(lengths))]
    ks = [_rand((hkv, L, d), 20 + s) for s, L in enumerate(lengths)]
    vs = [_rand((hkv, L, d), 30 + s) for s, L in enumerate(lengths)]
    rows = problem.row_table(lengths, b, "decode", hq)
    blocks = [list(range(routing.num_blocks(lengths[s], b))) for (s, _h, _r, _n) in rows]
    res = problem.attention_rows(qs, ks, vs, lengths, b, "decode", False, list(range(len(rows))), blocks)
    group = hq // hkv
    for i, (s, h, r, n_k) in enumerate(rows):
        assert r == n_k - 1
        [(hh, toks, out)] = res[i]
        assert hh == h and list(toks) == [0]
        q = torch.from_numpy(qs[s][h, 0:1])[None, None]              # [1, 1, 1, d]
        k = torch.from_numpy(ks[s][h // group])[None, None]          # [1, 1, L, d]
        v = torch.from_numpy(vs[s][h // group])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=False)[0, 0].numpy()
        assert np.max(np.abs(out["o"] - ref)) < 1e-12
        # lse of the scaled logits over all L keys
        logits = (qs[s][h, 0] @ ks[s][h // group].T) / math.sqrt(d)
        lse = np.log(np.sum(np.exp(logits - logits.max()))) + logits.max()
        assert abs(out["lse"][0] - lse) < 1e-12


def test_decode_sparse_blocks_plain_loops():
    d, b, L = 4, 8, 45          # 6 blocks, the last holding 5 keys
    q = _rand((1, 1, d), 1)
    k = _rand((1, L, d), 2)
    v = _rand((1, L, d), 3)
    listed = [0, 3, 5]
    res = problem.attention_rows([q], [k], [v], [L], b, "decode", False, [0], [listed])
    [(_hh, _toks, out)] = res[0]
    # plain loops: softmax over the keys of blocks 0, 3 and 5 only
    keys = [p for p in range(L) if p // b in listed]
    logits = []
    for p in keys:
        acc = 0.0
        for e in range(d):
            acc += q[0, 0, e] * k[0, p, e]
        logits.append(acc / math.sqrt(d))
    mx = max(logits)
    w = [math.exp(x - mx) for x in logits]
    tot = sum(w)
    ref = [sum(w[i] * v[0, p, e] for i, p in enumerate(keys)) / tot for e in range(d)]
    assert np.max(np.abs(out["o"][0] - np.array(ref))) < 1e-12
    assert abs(out["lse"][0] - (mx + math.log(tot))) < 1e-12
    # keys 40..44 (block 5) count: 3 blocks = 8 + 8 + 5 keys
    assert len(keys) == 21 and np.count_nonzero(out["p"][0]) == 21


@pytest.mark.parametrize("share", [False, True])
def test_packed_batch_equals_sequences_alone(share):
    b, d, hq, hkv = 8, 4, 4, 2
    lengths = [37, 8, 20]       # 5 blocks (last partial), 1 block, 3 blocks (last partial)
    qs = [_rand((hq, L, d), 40 + s) for s, L in enumerate(lengths)]
    ks = [_rand((hkv, L, d), 50 + s) for s, L in enumerate(lengths)]
    vs = [_rand((hkv, L, d), 60 + s) for s, L in enumerate(lengths)]
    hr = hkv if share else hq
    args = dict(qpool="mean", share_gqa=share, select="topk", k_b=3, k_min=1, tau_rel=2.0,
                forced_first=False)

    def run(qs_, ks_, vs_, lens_):
        J, _ = problem.route(qs_, ks_, lens_, b, "prefill", args["qpool"], share, args["select"],
                             args["k_b"], args["k_min"], args["tau_rel"], args["forced_first"])
        w = problem.worklist(J, lens_, b, "prefill", hr, False, args["k_b"] + 1)
        rows = list(range(len(J)))
        blocks = [w["col_idx"][w["row_ptr"][i]:w["row_ptr"][i + 1]].tolist() for i in rows]
        att = problem.attention_rows(qs_, ks_, vs_, lens_, b, "prefill", share, rows, blocks)
        return J, blocks, att

    J_all, bl_all, att_all = run(qs, ks, vs, lengths)
    table = problem.row_table(lengths, b, "prefill", hr)
    i = 0
    for s in range(len(lengths)):
        J_s, bl_s, att_s = run([qs[s]], [ks[s]], [vs[s]], [lengths[s]])
        for j in range(len(J_s)):
            assert table[i][0] == s
            assert list(J_all[i]) == list(J_s[j])
            assert bl_all[i] == bl_s[j]
            for (h1, t1, o1), (h2, t2, o2) in zip(att_all[i], att_s[j]):
                assert h1 == h2 and list(t1) == list(t2)
                assert np.array_equal(o1["o"], o2["o"])
            i += 1
    assert i == len(J_all)


def test_packed_batch_with_empty_sequences():
    """Sequences of no tokens contribute no rows: the batch with them routes,
    worklists and attends exactly like the batch without them."""
    b, d, hq, hkv = 8, 4, 4, 2
    full = [37, 0, 20, 0, 0, 9]
    qs = [_rand((hq, L, d), 70 + s) for s, L in enumerate(full)]
    ks = [_rand((hkv, L, d), 80 + s) for s, L in enumerate(full)]
    vs = [_rand((hkv, L, d), 90 + s) for s, L in enumerate(full)]
    keep = [s for s, L in enumerate(full) if L]

    def run(idx):
        lens = [full[s] for s in idx]
        J, _ = problem.route([qs[s] for s in idx], [ks[s] for s in idx], lens, b, "prefill", "mean", True,
                             "topk", 3, 1, 2.0, True)
        w = problem.worklist(J, lens, b, "prefill", hkv, True, 5)
        rows = list(range(len(J)))
        blocks = [w["col_idx"][w["row_ptr"][i]:w["row_ptr"][i + 1]].tolist() for i in rows]
        att = problem.attention_rows([qs[s] for s in idx], [ks[s] for s in idx], [vs[s] for s in idx], lens, b,
                                     "prefill", True, rows, blocks)
        return J, w, att

    Ja, wa, aa = run(list(range(len(full))))
    Jb, wb, ab = run(keep)
    assert len(Ja) == len(Jb) == sum(-(-L // b) for L in full) * hkv
    assert all(list(x) == list(y) for x, y in zip(Ja, Jb))
    for key in ("row_ptr", "col_idx", "row_perm", "bucket_ptr"):
        assert np.array_equal(wa[key], wb[key]), key
    for i in aa:
        for (h1, t1, o1), (h2, t2, o2) in zip(aa[i], ab[i]):
            assert h1 == h2 and np.array_equal(o1["o"], o2["o"])


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "budget_counts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


def test_effective_pairs_all_blocks_is_eq8_and_diagonal_closed_form():
    g = _golden()
    n, b = g["n"], g["block"]
    nb = n // b
    all_rows = [(r, list(range(r + 1))) for r in range(nb)]
    assert counting.effective_pairs_prefill(all_rows, n, b) == g["dense_causal_pairs"]
    diag = [(r, [r]) for r in range(nb)]
    assert counting.effective_pairs_prefill(diag, n, b) == nb * b * (b + 1) // 2
    # a partial last block: n = 100, b = 64 -> block 1 holds 36 queries and keys
    assert counting.effective_pairs_prefill([(0, [0]), (1, [0, 1])], 100, 64) == 64 * 65 // 2 + 36 * 64 + 36 * 37 // 2
