"""GPU parity of sparse_attn_append_kv: appending K/V rows to a decode cache and
keeping the block summaries current with the Eq (11) running-mean update
([P2] §3.1), checked against the oracle (oracle/cache.py, oracle/routing.py).

  cache      bit-exact: rows [0, L) equal the appended rows, rows past L keep
             their previous contents
  summaries  blocks below ceil(L / b) within 1e-5 of the oracle's fp64 block
             means of the grown cache (the GPU sums in fp32); blocks past it
             untouched
  decode     routing on the maintained summaries, the worklist and the decode
             attention over a cache with spare capacity (strides follow
             kv_capacity) match the oracle on the grown cache, to the router
             tie band and the output tolerances of the other parity tests

Inputs: N(0, 1) rows from a seeded torch generator, rounded once to the
problem's dtype; the append sizes cross, start and end on block edges.
"""
import types

import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import cache as ocache
from oracle import problem as oprob
from parity import TOL, check_router_row

pytestmark = pytest.mark.gpu

B = 64
SENT_KV = 7.0      # cache rows never written
SENT_SUM = -3.0    # summary slots never written
SUM_TOL = 1e-5


def _run(dtype, d, S=3, hq=4, hkv=2, cap=700, len0=100, chunks=(1, 27, 1, 64, 100, 0, 37), k_b=4, seed=0):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"append_kv case dtype={dtype} d={d} S={S} hq={hq} hkv={hkv} cap={cap} len0={len0} "
          f"chunks={chunks}", flush=True)
    g = torch.Generator().manual_seed(seed)
    k_all = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    v_all = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    q = torch.randn((S, hq, d), generator=g).to(tdt).to(dev)
    kc = torch.full((S, hkv, cap, d), SENT_KV, dtype=tdt)
    vc = torch.full((S, hkv, cap, d), SENT_KV, dtype=tdt)
    kc[:, :, :len0] = k_all[:, :, :len0]
    vc[:, :, :len0] = v_all[:, :, :len0]
    kc, vc = kc.to(dev), vc.to(dev)
    cfg = dbs.RouteConfig(k_b=k_b, share_gqa=True)
    prob = dbs.Problem.decode(S, hq, hkv, d, len0, dtype, kv_capacity=cap)
    summ = torch.full(dbs.summaries_shape(prob), SENT_SUM, dtype=torch.float32, device=dev)
    dbs.route(prob, cfg, q, kc, summaries=summ)          # summaries of the first len0 tokens
    L = len0
    for n in chunks:
        prob = dbs.Problem.decode(S, hq, hkv, d, L, dtype, kv_capacity=cap)
        dbs.append_kv(prob, k_all[:, :, L:L + n].contiguous().to(dev), v_all[:, :, L:L + n].contiguous().to(dev),
                      kc, vc, summ)
        L += n
        torch.cuda.synchronize()
        kh, vh = kc.cpu(), vc.cpu()
        assert torch.equal(kh[:, :, :L], k_all[:, :, :L]) and torch.equal(vh[:, :, :L], v_all[:, :, :L])
        assert bool((kh[:, :, L:] == SENT_KV).all()) and bool((vh[:, :, L:] == SENT_KV).all())
        nb = -(-L // B)
        sh = summ.cpu().double().numpy()
        err = 0.0
        for s in range(S):
            for h in range(hkv):
                ref = ocache.summaries_after(k_all[s, h].double().numpy(), L, B)
                err = max(err, float(np.max(np.abs(sh[s, h, :nb] - ref))))
        assert err <= SUM_TOL, (L, err)
        assert bool((summ[:, :, nb:] == SENT_SUM).all().item())

    # decode over the grown cache: route on the maintained summaries, worklist, attention
    prob = dbs.Problem.decode(S, hq, hkv, d, L, dtype, kv_capacity=cap)
    J, _ = dbs.route(prob, cfg, q, None, summaries=summ, summaries_in=True)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, q, kc, vc)
    torch.cuda.synchronize()
    qs = [q[s].unsqueeze(1).double().cpu().numpy() for s in range(S)]
    ks = [k_all[s, :, :L].double().numpy() for s in range(S)]
    vs = [v_all[s, :, :L].double().numpy() for s in range(S)]
    _j, scores = oprob.route(qs, ks, [L] * S, B, "decode", "mean", True, "topk", k_b, 4, 2.0, False)
    rule = types.SimpleNamespace(select="topk", k_b=k_b)
    Jh = J.cpu().numpy()
    for i in range(Jh.shape[0]):
        ok, _nd = check_router_row(Jh[i], scores[i], rule)
        assert ok, (i, Jh[i])
    rows = Jh.shape[0]
    rp = wl.row_ptr.cpu().numpy()
    ci = wl.col_idx.cpu().numpy()
    blocks = {i: ci[rp[i]:rp[i + 1]].tolist() for i in range(rows)}
    res = oprob.attention_rows(qs, ks, vs, [L] * S, B, "decode", True, list(range(rows)), blocks)
    mx, mean = TOL[dtype]
    errs = []
    for i in range(rows):
        s = i // hkv
        for hh, _toks, ref in res[i]:
            errs.append(np.abs(o[s, hh].float().cpu().numpy().astype(np.float64) - ref["o"][0]))
    e = np.concatenate(errs)
    assert e.max() <= mx and e.mean() <= mean, (e.max(), e.mean())
    return L


def test_append_bf16_d128():
    assert _run("bf16", 128) == 330


def test_append_f32_d64_from_empty_block_edge():
    # starts on a block edge (len0 = 128), one-token appends, a chunk of exactly one block
    assert _run("f32", 64, S=2, hq=2, hkv=2, cap=400, len0=128, chunks=(1, 1, 62, 64, 3, 130)) == 389


def test_append_rejects_past_capacity():
    dev = torch.device("cuda:0")
    prob = dbs.Problem.decode(1, 2, 2, 128, 60, "bf16", kv_capacity=64)
    kc = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=dev)
    summ = torch.zeros(dbs.summaries_shape(prob), dtype=torch.float32, device=dev)
    new = torch.zeros((1, 2, 5, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(dbs.SAError):
        dbs.append_kv(prob, new, new, kc, kc.clone(), summ)


def test_append_graph_replay_matches_eager():
    """The append captured in a HIP graph and replayed three times (state reset
    by eager copies between replays) gives the eager call's cache and
    summaries bit for bit."""
    dev = torch.device("cuda:0")
    S, hkv, d, cap, len0, n = 4, 2, 128, 300, 70, 90
    print(f"append_kv graph replay S={S} hkv={hkv} cap={cap} len0={len0} n={n}", flush=True)
    g = torch.Generator(device=dev).manual_seed(3)
    k0 = torch.randn((S, hkv, cap, d), generator=g, device=dev).to(torch.bfloat16)
    v0 = torch.randn((S, hkv, cap, d), generator=g, device=dev).to(torch.bfloat16)
    prob = dbs.Problem.decode(S, 4, hkv, d, len0, "bf16", kv_capacity=cap)
    s0 = torch.randn(dbs.summaries_shape(prob), generator=g, device=dev)
    kn = torch.randn((S, hkv, n, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((S, hkv, n, d), generator=g, device=dev).to(torch.bfloat16)
    ke, ve, se = k0.clone(), v0.clone(), s0.clone()
    dbs.append_kv(prob, kn, vn, ke, ve, se)
    kc, vc, sc = k0.clone(), v0.clone(), s0.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        dbs.append_kv(prob, kn, vn, kc, vc, sc)      # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dbs.append_kv(prob, kn, vn, kc, vc, sc)
    for _ in range(3):
        kc.copy_(k0); vc.copy_(v0); sc.copy_(s0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(kc, ke) and torch.equal(vc, ve) and torch.equal(sc, se)


def test_summary_pass_stays_inside_a_cache_with_spare_capacity():
    """Regression: with kv_capacity > seqlen the summary pass must launch one
    wavefront per valid block only.  It once launched one per allocated slot,
    mapped (sequence, block) over the valid blocks, and so read K and wrote
    summaries past the last sequence.  Guard rows after the summaries buffer
    must stay untouched and every valid block must match the oracle."""
    dev = torch.device("cuda:0")
    S, hq, hkv, d, L, cap = 3, 4, 2, 128, 100, 700
    print(f"summary pass, capacity {cap} > length {L}", flush=True)
    g = torch.Generator().manual_seed(9)
    k = torch.randn((S + 8, hkv, cap, d), generator=g).to(torch.bfloat16).to(dev)   # rows past S: guard
    q = torch.randn((S, hq, d), generator=g).to(torch.bfloat16).to(dev)
    prob = dbs.Problem.decode(S, hq, hkv, d, L, "bf16", kv_capacity=cap)
    shape = dbs.summaries_shape(prob)
    big = torch.full((S + 8,) + tuple(shape[1:]), SENT_SUM, dtype=torch.float32, device=dev)
    summ = big[:S]
    dbs.route(prob, dbs.RouteConfig(k_b=2, share_gqa=True), q, k[:S], summaries=summ)
    torch.cuda.synchronize()
    assert bool((big[S:] == SENT_SUM).all().item()), "summary pass wrote past the last sequence"
    nb = -(-L // B)
    assert bool((summ[:, :, nb:] == SENT_SUM).all().item())
    kh = k[:S].double().cpu().numpy()
    sh = summ.double().cpu().numpy()
    for s in range(S):
        for h in range(hkv):
            ref = ocache.summaries_after(kh[s, h], L, B)
            assert np.max(np.abs(sh[s, h, :nb] - ref)) <= SUM_TOL

