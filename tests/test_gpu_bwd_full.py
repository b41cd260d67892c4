"""Backward parity at the benchmark's full sizes, on sampled outputs.

The prefill settings the bench times (8192-token MHA, 16 heads; 2 x 32768-token
GQA, 32 query heads on 8 KV heads with shared routing) go through route,
worklist, fwd and sparse_attn_bwd on the GPU exactly as bench.py runs them.
The oracle ([P2] §4 training paragraph, [P3]: gradients over the forward's
block selection) then recomputes, one by one:

* dQ of sampled worklist rows: the fp64 gradient of that row's queries over
  the row's blocks (its keys are only those, so one oracle call is exact);
* dK and dV of sampled key blocks, among them the block listed by the most
  rows: the sum, over every row whose list holds the block and every query
  head the row serves, of that row's gradient restricted to the block.

Tolerance as in the small-size backward test (same derivation): |err| <=
8e-3 |ref| + 4e-3 max|ref| per sampled tensor.
"""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from dynamic_block_sparse_amd import workloads as wk
from oracle import backward as obwd

pytestmark = pytest.mark.gpu

B = 64
RTOL, STOL = 8e-3, 4e-3


def _check(label, got, ref):
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    worst = float(np.max(err - (RTOL * np.abs(ref) + STOL * scale)))
    print(f"  {label}: scale {scale:.3e} max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    assert worst <= 0, label


@pytest.mark.parametrize("w", [wk.PREFILL_MHA, wk.PREFILL_GQA], ids=lambda w: w.name)
def test_bwd_full_size_sampled(w):
    dev = torch.device("cuda:0")
    print(f"bwd full size {w.name}", flush=True)
    inp = wk.make_inputs(w, dev)
    prob, cfg = dbs.problem_for(w, inp), dbs.config_for(w)
    J, _s = dbs.route(prob, cfg, inp.q, inp.k)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, inp.q, inp.k, inp.v)
    g = torch.Generator(device=dev).manual_seed(17)
    dout = torch.randn(inp.q.shape, generator=g, device=dev).to(inp.q.dtype)
    dq, dk, dv = dbs.bwd(prob, cfg, wl, inp.q, inp.k, inp.v, o, lse, dout)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0

    n, hq, hkv = w.seqlen, w.heads_q, w.heads_kv
    nb = n // B
    group = hq // hkv
    share = w.share_gqa
    hr = hkv if share else hq
    rows = J.shape[0]
    rp = wl.row_ptr[:rows + 1].cpu().numpy()
    ci = wl.col_idx[:int(rp[-1])].cpu().numpy()

    def row_of(s, h, r):
        return (s * hr + h) * nb + r

    cache, kvcache = {}, {}

    def kv(s, kvh):
        if (s, kvh) not in kvcache:
            kvcache[(s, kvh)] = (inp.k[s, kvh].double().cpu().numpy(), inp.v[s, kvh].double().cpu().numpy())
        return kvcache[(s, kvh)]

    def grads(s, h_row, r, hh):
        """Oracle gradients of query head hh over row (s, h_row, r), on the
        row's own blocks only: the listed blocks are packed in ascending order
        (the query block r, the largest, last) and the queries keep their
        offset inside that last block, so every earlier packed block is wholly
        before them and the causal mask is the same as on the full sequence.
        Returns (dq [64, d], {block id: (dk [64, d], dv [64, d])})."""
        key = (s, h_row, r, hh)
        if key not in cache:
            i = row_of(s, h_row, r)
            blocks = ci[rp[i]:rp[i + 1]].tolist()
            assert blocks[-1] == r
            kk, vv = kv(s, hh // group)
            idx = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
            m = len(blocks)
            qpos = (m - 1) * B + np.arange(B)
            qh = inp.q[s, hh, r * B:(r + 1) * B].double().cpu().numpy()
            do = dout[s, hh, r * B:(r + 1) * B].double().cpu().numpy()
            gq, gk, gv = obwd.masked_attention_grads(qh, qpos, kk[idx], vv[idx], m * B, B, list(range(m)), True, do)
            cache[key] = (gq, {b: (gk[t * B:(t + 1) * B], gv[t * B:(t + 1) * B]) for t, b in enumerate(blocks)})
        return cache[key]

    rng = np.random.default_rng(3)
    # dQ of sampled rows: the first, the last and two random ones
    picks = [(0, 0, 0), (w.batch - 1, hr - 1, nb - 1)]
    picks += [(int(rng.integers(w.batch)), int(rng.integers(hr)), int(rng.integers(nb))) for _ in range(2)]
    for s, h, r in picks:
        heads = range(h * group, (h + 1) * group) if share else [h]
        for hh in heads:
            gq, _kv = grads(s, h, r, hh)
            got = dq[s, hh, r * B:(r + 1) * B].float().cpu().numpy().astype(np.float64)
            _check(f"dq s={s} head={hh} r={r}", got, gq)

    # dK, dV of sampled key blocks: the most listed one of (sequence 0, KV head 0) and a random one
    def listing_rows(s, kvh, j):
        hrs = [kvh] if share else list(range(kvh * group, (kvh + 1) * group))
        out = []
        for h in hrs:
            for r in range(j, nb):
                i = row_of(s, h, r)
                lst = ci[rp[i]:rp[i + 1]]
                if np.searchsorted(lst, j) < len(lst) and lst[np.searchsorted(lst, j)] == j:
                    out.append((h, r))
        return out

    counts = np.zeros(nb, dtype=np.int64)
    for h in ([0] if share else range(group)):
        for r in range(nb):
            i = row_of(0, h, r)
            np.add.at(counts, ci[rp[i]:rp[i + 1]], 1)
    blocks = [(0, 0, int(np.argmax(counts))),
              (int(rng.integers(w.batch)), int(rng.integers(hkv)), int(rng.integers(nb)))]
    for s, kvh, j in blocks:
        lr = listing_rows(s, kvh, j)
        print(f"  key block s={s} kvh={kvh} j={j}: listed by {len(lr)} rows", flush=True)
        rk = np.zeros((B, w.head_dim))
        rv = np.zeros((B, w.head_dim))
        for h, r in lr:
            heads = range(h * group, (h + 1) * group) if share else [h]
            for hh in heads:
                gk, gv = grads(s, h, r, hh)[1][j]
                rk += gk
                rv += gv
        gotk = dk[s, kvh, j * B:(j + 1) * B].float().cpu().numpy().astype(np.float64)
        gotv = dv[s, kvh, j * B:(j + 1) * B].float().cpu().numpy().astype(np.float64)
        _check(f"dk s={s} kvh={kvh} j={j}", gotk, rk)
        _check(f"dv s={s} kvh={kvh} j={j}", gotv, rv)
    del inp, J, wl, o, lse, dout, dq, dk, dv
    torch.cuda.empty_cache()
