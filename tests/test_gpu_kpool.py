"""GPU parity of max-pooled key summaries ([P2] §2.1 and §4: the
per-dimension maximum over a block's valid keys, set against the Eq 6 mean).

Summaries are maxima of bf16 (or fp32) inputs, which fp32 holds exactly, so
the GPU's summaries must equal the oracle's bit for bit (valid blocks; a
ragged last block takes only its valid keys).  Routing is checked row by row
against the oracle's scores on those summaries (tie band of the parity
helpers), the worklist set exactly, and the attention output at the parity
tolerances.  Decode keeps max-pooled summaries with the cache: an append
takes the per-dimension maximum with the new keys, checked against the
oracle's append.
"""
import types

import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import cache as ocache
from oracle import problem as oprob
from oracle import routing as orout
from oracle import worklist as owl
from parity import TOL, check_router_row

pytestmark = pytest.mark.gpu

B = 64
CASES = [
    # name, dtype, d, batch, hq, hkv, n, k_b, qpool, share, first, window
    ("mha_meanq_tiles", "bf16", 128, 1, 4, 4, 1000, 6, "mean", False, False, 1),
    ("gqa_maxq_sink", "bf16", 128, 2, 8, 2, 700, 5, "max", True, True, 2),
    ("f32_d64", "f32", 64, 1, 2, 2, 650, 4, "mean", False, False, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_max_key_summaries_prefill(case):
    name, dtype, d, bsz, hq, hkv, n, k_b, qpool, share, first, window = case
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"max key summaries {name}: n={n} k_b={k_b} qpool={qpool}", flush=True)
    g = torch.Generator().manual_seed(51)
    q = torch.randn((bsz, hq, n, d), generator=g).to(tdt)
    k = torch.randn((bsz, hkv, n, d), generator=g).to(tdt)
    v = torch.randn((bsz, hkv, n, d), generator=g).to(tdt)
    prob = dbs.Problem.fixed(bsz, hq, hkv, d, n, dtype)
    cfg = dbs.RouteConfig(k_b=k_b, qpool=qpool, share_gqa=share, force_first=first, window=window,
                          kpool="max")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    J, summ = dbs.route(prob, cfg, qd, kd)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, qd, kd, vd)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0
    nb = -(-n // B)
    sg = summ.cpu().numpy()
    for s in range(bsz):
        for h in range(hkv):
            want = orout.block_summaries(k[s, h].double().numpy(), n, B, "max")
            assert np.array_equal(sg[s, h, :nb].astype(np.float64), want), (name, s, h)

    qs = [q[s].double().numpy() for s in range(bsz)]
    ks = [k[s].double().numpy() for s in range(bsz)]
    vs = [v[s].double().numpy() for s in range(bsz)]
    hr = hkv if share else hq
    _j, scores = oprob.route(qs, ks, [n] * bsz, B, "prefill", qpool, share, "topk", k_b, 4, 2.0, first,
                             window=window, kpool="max")
    table = oprob.row_table([n] * bsz, B, "prefill", hr)
    Jh = J.cpu().numpy()
    rp, ci = wl.row_ptr.cpu().numpy(), wl.col_idx.cpu().numpy()
    rule = types.SimpleNamespace(select="topk", k_b=k_b)
    blocks = {}
    for i, (s, h, r, _n) in enumerate(table):
        ok, _nd = check_router_row(Jh[i], scores[i], rule)
        assert ok, (name, s, h, r, Jh[i])
        forced = orout.forced_blocks(r, nb, "prefill", first, window)
        want, err = owl.row_set(Jh[i], nb, r, "prefill", forced)
        assert err == 0 and ci[rp[i]:rp[i + 1]].tolist() == want, (name, s, h, r)
        blocks[i] = want
    res = oprob.attention_rows(qs, ks, vs, [n] * bsz, B, "prefill", share, sorted(blocks), blocks)
    on = o.float().cpu().numpy()
    errs = []
    for oi, heads in res.items():
        s = table[oi][0]
        for hh, toks, ref in heads:
            errs.append(np.abs(on[s, hh, toks] - ref["o"]))
    e = np.concatenate(errs)
    mx, mean = TOL[dtype]
    print(f"max key summaries {name}: rows {len(table)} max-abs {e.max():.3e} mean-abs {e.mean():.3e}",
          flush=True)
    assert e.max() <= mx and e.mean() <= mean


def test_max_key_summaries_decode_and_append():
    """Decode routes on max-pooled summaries built from the cache, then an
    append of 70 tokens (crossing a block boundary) updates them by maxima."""
    dev = torch.device("cuda:0")
    S, hq, hkv, d, L, cap = 3, 8, 2, 128, 900, 1024
    print(f"max key summaries decode: S={S} L={L} cap={cap}", flush=True)
    g = torch.Generator().manual_seed(52)
    k = torch.randn((S, hkv, cap, d), generator=g).to(torch.bfloat16)
    v = torch.randn((S, hkv, cap, d), generator=g).to(torch.bfloat16)
    q = torch.randn((S, hq, d), generator=g).to(torch.bfloat16)
    prob = dbs.Problem.decode(S, hq, hkv, d, L, "bf16", kv_capacity=cap)
    cfg = dbs.RouteConfig(k_b=6, share_gqa=True, window=2, kpool="max")
    kd, vd, qd = k.to(dev), v.to(dev), q.to(dev)
    J, summ = dbs.route(prob, cfg, qd, kd)
    wl = dbs.build_worklist(prob, cfg, J)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0
    nb = -(-L // B)
    sg = summ.cpu().numpy()
    want = {}
    for s in range(S):
        for h in range(hkv):
            want[(s, h)] = orout.block_summaries(k[s, h].double().numpy(), L, B, "max")
            assert np.array_equal(sg[s, h, :nb].astype(np.float64), want[(s, h)])
    qs = [q[s].unsqueeze(1).double().numpy() for s in range(S)]
    ks = [k[s, :, :L].double().numpy() for s in range(S)]
    _j, scores = oprob.route(qs, ks, [L] * S, B, "decode", "mean", True, "topk", 6, 4, 2.0, False,
                             window=2, kpool="max")
    rule = types.SimpleNamespace(select="topk", k_b=6)
    Jh = J.cpu().numpy()
    for i in range(Jh.shape[0]):
        ok, _nd = check_router_row(Jh[i], scores[i], rule)
        assert ok, (i, Jh[i])

    n = 70
    kn = torch.randn((S, hkv, n, d), generator=g).to(torch.bfloat16)
    vn = torch.randn((S, hkv, n, d), generator=g).to(torch.bfloat16)
    dbs.append_kv(prob, kn.to(dev), vn.to(dev), kd, vd, summ, kpool="max")
    torch.cuda.synchronize()
    sg2 = summ.cpu().numpy()
    nb2 = -(-(L + n) // B)
    for s in range(S):
        for h in range(hkv):
            _k2, _v2, c2 = ocache.append_kv(k[s, h].double().numpy(), v[s, h].double().numpy(),
                                            sg[s, h].astype(np.float64), L, kn[s, h].double().numpy(),
                                            vn[s, h].double().numpy(), B, kpool="max")
            assert np.array_equal(sg2[s, h, :nb2].astype(np.float64), c2[:nb2]), (s, h)
            assert np.array_equal(c2[:nb2], ocache.summaries_after(
                torch.cat([k[s, h, :L], kn[s, h]]).double().numpy(), L + n, B, "max"))


def test_max_key_summaries_packed_varlen():
    """Packed varlen prefill: each sequence's summary slots (from its first
    block slot on) hold the per-dimension maxima of its own keys, ragged and
    one-block sequences included; router rows match the oracle's scores."""
    dev = torch.device("cuda:0")
    lengths, hq, hkv, d = [300, 64, 577], 4, 2, 128
    print(f"max key summaries varlen: lengths={lengths}", flush=True)
    g = torch.Generator().manual_seed(53)
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = torch.randn((hq, total, d), generator=g).to(torch.bfloat16)
    k = torch.randn((hkv, total, d), generator=g).to(torch.bfloat16)
    prob = dbs.Problem.varlen(lengths, hq, hkv, d, torch.tensor(cu, dtype=torch.int32, device=dev), "bf16")
    cfg = dbs.RouteConfig(k_b=4, share_gqa=True, kpool="max")
    J, summ = dbs.route(prob, cfg, q.to(dev), k.to(dev))
    wl = dbs.build_worklist(prob, cfg, J)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0
    sg = summ.cpu().numpy()
    blk0 = 0
    qs, ks = [], []
    for s, ln in enumerate(lengths):
        nb = -(-ln // B)
        for h in range(hkv):
            want = orout.block_summaries(k[h, cu[s]:cu[s] + ln].double().numpy(), ln, B, "max")
            assert np.array_equal(sg[h, blk0:blk0 + nb].astype(np.float64), want), (s, h)
        blk0 += nb
        qs.append(q[:, cu[s]:cu[s] + ln].double().numpy())
        ks.append(k[:, cu[s]:cu[s] + ln].double().numpy())
    _j, scores = oprob.route(qs, ks, lengths, B, "prefill", "mean", True, "topk", 4, 4, 2.0, False, kpool="max")
    rule = types.SimpleNamespace(select="topk", k_b=4)
    Jh = J.cpu().numpy()
    for i in range(Jh.shape[0]):
        ok, _nd = check_router_row(Jh[i], scores[i], rule)
        assert ok, (i, Jh[i])
