"""GPU parity of chunked prefill: the queries of one chunk, tokens
[q_start, n) of each sequence, routed against every earlier block of the
sequence (a cached prefix plus the chunk itself) and attended over the K/V
cache ([P2] §3.1: summaries are cache state; block ids stay sequence-local).

Each GPU row (sequence, routing head, query block r >= q_start / b) is
checked against the oracle's row for the same query block of the whole
sequence: router set (tie band), worklist set and error bits, output and
log-sum-exp, at the parity tolerances.  Four routing paths: mean pooling
through the score tiles (MHA), GQA with the sink and a local window, max
pooling (per-row score kernel), and fp32 d = 64.
"""
import types

import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import problem as oprob
from oracle import routing as orout
from oracle import worklist as owl
from parity import LSE_TOL, TOL, check_router_row

pytestmark = pytest.mark.gpu

B = 64
CASES = [
    # name, dtype, d, batch, hq, hkv, n, q_start, cap, k_b, qpool, share, first, window
    ("mha_mean_tiles", "bf16", 128, 2, 4, 4, 1500, 960, 2048, 8, "mean", False, False, 1),
    ("gqa_first_win2", "bf16", 128, 1, 8, 2, 2000, 1024, 2048, 10, "mean", True, True, 2),
    ("mha_maxpool", "bf16", 128, 1, 2, 2, 900, 512, 900, 5, "max", False, False, 1),
    ("f32_d64", "f32", 64, 1, 2, 2, 700, 448, 768, 4, "mean", False, False, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_chunked_prefill(case):
    name, dtype, d, bsz, hq, hkv, n, q0, cap, k_b, qpool, share, first, window = case
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"chunked prefill {name}: n={n} q_start={q0} cap={cap} k_b={k_b}", flush=True)
    g = torch.Generator().manual_seed(31)
    q_full = torch.randn((bsz, hq, n, d), generator=g).to(tdt)
    k = torch.randn((bsz, hkv, cap, d), generator=g).to(tdt)
    v = torch.randn((bsz, hkv, cap, d), generator=g).to(tdt)
    prob = dbs.Problem.fixed(bsz, hq, hkv, d, n, dtype, kv_capacity=cap, q_start=q0)
    cfg = dbs.RouteConfig(k_b=k_b, qpool=qpool, share_gqa=share, force_first=first, window=window)
    qd = q_full[:, :, q0:].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    J, _summ = dbs.route(prob, cfg, qd, kd)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, qd, kd, vd)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0

    # oracle over the whole sequences; GPU row i <-> oracle row of the same (s, h, r)
    qs = [q_full[s].double().numpy() for s in range(bsz)]
    ks = [k[s, :, :n].double().numpy() for s in range(bsz)]
    vs = [v[s, :, :n].double().numpy() for s in range(bsz)]
    hr = hkv if share else hq
    _j, scores = oprob.route(qs, ks, [n] * bsz, B, "prefill", qpool, share, "topk", k_b, 4, 2.0, first,
                             window=window)
    table = oprob.row_table([n] * bsz, B, "prefill", hr)
    index = {(s, h, r): i for i, (s, h, r, _n) in enumerate(table)}
    nb, r0 = -(-n // B), q0 // B
    gpu_rows = [(s, h, r) for s in range(bsz) for h in range(hr) for r in range(r0, nb)]
    Jh = J.cpu().numpy()
    assert Jh.shape[0] == len(gpu_rows)
    rule = types.SimpleNamespace(select="topk", k_b=k_b)
    rp, ci = wl.row_ptr.cpu().numpy(), wl.col_idx.cpu().numpy()
    blocks = {}
    for i, (s, h, r) in enumerate(gpu_rows):
        ok, _nd = check_router_row(Jh[i], scores[index[(s, h, r)]], rule)
        assert ok, (name, s, h, r, Jh[i])
        forced = orout.forced_blocks(r, nb, "prefill", first, window)
        want, err = owl.row_set(Jh[i], nb, r, "prefill", forced)
        assert err == 0 and ci[rp[i]:rp[i + 1]].tolist() == want, (name, s, h, r)
        blocks[index[(s, h, r)]] = want
    # row_perm: a permutation sorted by (length bucket, row)
    perm = wl.row_perm.cpu().numpy()[:len(gpu_rows)]
    lens = rp[1:len(gpu_rows) + 1] - rp[:len(gpu_rows)]
    bucket = [owl.bucket_index(int(x)) for x in lens]
    assert sorted(perm.tolist()) == list(range(len(gpu_rows)))
    assert [(bucket[p], p) for p in perm] == sorted((bucket[p], p) for p in perm)

    res = oprob.attention_rows(qs, ks, vs, [n] * bsz, B, "prefill", share, sorted(blocks), blocks)
    on, ln = o.float().cpu().numpy(), lse.cpu().numpy()
    errs, lerr = [], 0.0
    for oi, heads in res.items():
        s = table[oi][0]
        for hh, toks, ref in heads:
            errs.append(np.abs(on[s, hh, toks - q0] - ref["o"]))
            lerr = max(lerr, float(np.max(np.abs(ln[s, hh, toks - q0] - ref["lse"]))))
    e = np.concatenate(errs)
    mx, mean = TOL[dtype]
    print(f"chunked prefill {name}: rows {len(gpu_rows)} max-abs {e.max():.3e} mean-abs {e.mean():.3e} "
          f"lse {lerr:.2e}", flush=True)
    assert e.max() <= mx and e.mean() <= mean
    assert lerr <= LSE_TOL[dtype]
