"""GPU parity of decode over sequences with different cached lengths
(sa_problem.seq_lens; [P3] "From index output to worklist": the requests of a
decode batch differ in history length).

Every sequence s has its own length L_s: its summaries cover blocks
0 .. ceil(L_s / b) - 1, its row routes over the complete blocks before the
last one, which is forced and masked to its valid keys.  The lengths mix a
one-token cache, exactly one block, a block plus one token, partial last
blocks and long histories.  K/V rows past each L_s hold NaN and summary slots
past each sequence's blocks hold NaN: any read of them would show in the
results.

  summaries  within 1e-5 of the oracle's fp64 block summaries; slots past the
             sequence's blocks untouched
  router     each row against the oracle routed on that sequence alone
             (the 1e-5 relative tie band of the other parity tests)
  worklist   bit-exact against the oracle's worklist of the GPU's J
  output     every row against the oracle's masked attention (bf16 2e-2
             max-abs / 5e-3 mean-abs; fp32 1e-5), lse to the same bounds as
             the other parity tests
  append     per-sequence start rows (0, 1, 63, 64, ...): caches bit-exact,
             summaries within 1e-5 of the oracle's, then decode on the
             maintained summaries as above
  paged      the same ragged batch through a block table: bit-identical to
             the contiguous cache
  lengths    entries outside [1, seqlen] are clamped and reported
             (SA_WL_ERR_LENGTH): results equal those of the clamped lengths
"""
import types

import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import cache as ocache
from oracle import problem as oprob
from parity import LSE_TOL, TOL, check_router_row

pytestmark = pytest.mark.gpu

B = 64
SUM_TOL = 1e-5
LENGTHS = [1, 64, 65, 130, 700, 1000, 2, 129]
CAP = 1088


def _inputs(dtype, d, hq, hkv, lengths, cap, seed):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(seed)
    S = len(lengths)
    k = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    v = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    q = torch.randn((S, hq, d), generator=g).to(tdt)
    for s, L in enumerate(lengths):   # rows past each length are never read
        k[s, :, L:] = float("nan")
        v[s, :, L:] = float("nan")
    return q, k, v


def _lens(lengths, dev):
    return torch.tensor(lengths, dtype=torch.int32, device=dev)


def _same_worklist(a, b):
    """Bit-identical worklists (col_idx up to the entry count: the tail is unwritten)."""
    nnz = int(a.row_ptr[-1].item())
    assert torch.equal(a.row_ptr, b.row_ptr)
    assert torch.equal(a.col_idx[:nnz], b.col_idx[:nnz])
    for key in ("row_perm", "bucket_ptr"):
        assert torch.equal(getattr(a, key), getattr(b, key)), key


def _run(prob, cfg, q, k, v, summ=None, summaries_in=False, num_splits=0):
    J, summ = dbs.route(prob, cfg, q, k, summaries=summ, summaries_in=summaries_in)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, q, k, v, num_splits=num_splits)
    torch.cuda.synchronize()
    return J, summ, wl, o, lse


def _check_decode(cfg, dtype, lengths, q, k, v, J, wl, o, lse):
    """Router rows, worklist and output of a ragged decode batch against the oracle."""
    S = len(lengths)
    hq, hkv = q.shape[1], k.shape[1]
    hr = hkv if cfg.share_gqa else hq
    qs = [q[s].unsqueeze(1).double().cpu().numpy() for s in range(S)]
    ks = [k[s, :, :lengths[s]].double().cpu().numpy() for s in range(S)]
    vs = [v[s, :, :lengths[s]].double().cpu().numpy() for s in range(S)]
    _j, scores = oprob.route(qs, ks, lengths, B, "decode", cfg.qpool, cfg.share_gqa, cfg.select, cfg.k_b,
                             cfg.k_min, cfg.tau_rel, cfg.force_first, window=cfg.window, kpool=cfg.kpool)
    rule = types.SimpleNamespace(select=cfg.select, k_b=cfg.k_b, k_min=cfg.k_min, tau_rel=cfg.tau_rel)
    Jh = J.cpu().numpy()
    rows = Jh.shape[0]
    assert rows == S * hr
    for i in range(rows):
        ok, _nd = check_router_row(Jh[i], scores[i], rule)
        assert ok, (i, Jh[i])
    width = cfg.k_b + max(cfg.window, 1) + (1 if cfg.force_first else 0)
    ref = oprob.worklist(Jh, lengths, B, "decode", hr, cfg.force_first, width, window=cfg.window)
    rp = wl.row_ptr.cpu().numpy()
    nnz = int(rp[-1])
    got = dict(row_ptr=rp, col_idx=wl.col_idx[:nnz].cpu().numpy(), row_perm=wl.row_perm[:rows].cpu().numpy(),
               bucket_ptr=wl.bucket_ptr.cpu().numpy())
    for key in ("row_ptr", "col_idx", "row_perm", "bucket_ptr"):
        assert np.array_equal(np.asarray(got[key], np.int64), ref[key]), key
    assert int(wl.err.item()) == ref["err"] == 0
    blocks = {i: got["col_idx"][rp[i]:rp[i + 1]].tolist() for i in range(rows)}
    res = oprob.attention_rows(qs, ks, vs, lengths, B, "decode", cfg.share_gqa, list(range(rows)), blocks)
    table = oprob.row_table(lengths, B, "decode", hr)
    mx, mean = TOL[dtype]
    errs, lse_err = [], 0.0
    for i in range(rows):
        s = table[i][0]
        for hh, _toks, r in res[i]:
            errs.append(np.abs(o[s, hh].float().cpu().numpy().astype(np.float64) - r["o"][0]))
            lse_err = max(lse_err, abs(float(lse[s, hh].item()) - float(r["lse"][0])))
    e = np.concatenate(errs)
    print(f"ragged decode: max-abs {e.max():.3e} mean-abs {e.mean():.3e} lse {lse_err:.3e}", flush=True)
    assert e.max() <= mx and e.mean() <= mean, (e.max(), e.mean())
    assert lse_err <= LSE_TOL[dtype]


def _check_summaries(summ, k, lengths, kpool):
    sh = summ.cpu().double().numpy()
    kh = k.cpu()
    err = 0.0
    for s, L in enumerate(lengths):
        nb = -(-L // B)
        for h in range(k.shape[1]):
            ref = ocache.summaries_after(kh[s, h, :L].double().numpy(), L, B, kpool)
            err = max(err, float(np.max(np.abs(sh[s, h, :nb] - ref))))
        assert np.isnan(sh[s, :, nb:]).all(), s   # slots past the sequence's blocks untouched
    assert err <= SUM_TOL, err


CASES = [
    # name, dtype, d, hq, hkv, config, splits
    ("bf16_shared_topk", "bf16", 128, 8, 2, dict(k_b=6, share_gqa=True), 0),
    ("bf16_shared_topk_3splits", "bf16", 128, 8, 2, dict(k_b=6, share_gqa=True), 3),
    ("bf16_heads_window_sink", "bf16", 128, 4, 2, dict(k_b=5, window=2, force_first=True), 0),
    ("bf16_shared_threshold", "bf16", 128, 8, 2, dict(k_b=8, share_gqa=True, select="threshold", k_min=3,
                                                      tau_rel=0.5), 0),
    ("bf16_maxpool", "bf16", 128, 8, 2, dict(k_b=6, share_gqa=True, qpool="max", kpool="max"), 0),
    ("f32_d64_heads", "f32", 64, 4, 2, dict(k_b=4), 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_ragged_decode_matches_oracle(case):
    name, dtype, d, hq, hkv, cfgkw, splits = case
    dev = torch.device("cuda:0")
    print(f"ragged decode {name} lengths={LENGTHS} cap={CAP}", flush=True)
    q, k, v = _inputs(dtype, d, hq, hkv, LENGTHS, CAP, seed=31)
    cfg = dbs.RouteConfig(**cfgkw)
    prob = dbs.Problem.decode(len(LENGTHS), hq, hkv, d, max(LENGTHS), dtype, kv_capacity=CAP,
                              seq_lens=_lens(LENGTHS, dev))
    summ = torch.full(dbs.summaries_shape(prob), float("nan"), dtype=torch.float32, device=dev)
    J, summ, wl, o, lse = _run(prob, cfg, q.to(dev), k.to(dev), v.to(dev), summ=summ, num_splits=splits)
    _check_summaries(summ, k, LENGTHS, cfg.kpool)
    _check_decode(cfg, dtype, LENGTHS, q, k, v, J, wl, o, lse)


def test_ragged_paged_equals_contiguous():
    dev = torch.device("cuda:0")
    hq, hkv, d = 8, 2, 128
    S = len(LENGTHS)
    print(f"ragged paged decode lengths={LENGTHS}", flush=True)
    q, k, v = _inputs("bf16", d, hq, hkv, LENGTHS, CAP, seed=37)
    nbc = CAP // B
    pool = S * nbc + 5
    g = torch.Generator().manual_seed(3)
    table = torch.randperm(pool, generator=g)[:S * nbc].reshape(S, nbc).to(torch.int32)
    kp = torch.randn((pool, hkv, B, d), generator=g).to(torch.bfloat16)
    vp = torch.randn((pool, hkv, B, d), generator=g).to(torch.bfloat16)
    for s in range(S):
        for j in range(nbc):
            kp[table[s, j]] = k[s, :, j * B:(j + 1) * B]
            vp[table[s, j]] = v[s, :, j * B:(j + 1) * B]
    cfg = dbs.RouteConfig(k_b=6, share_gqa=True, window=2)
    lens = _lens(LENGTHS, dev)
    pc = dbs.Problem.decode(S, hq, hkv, d, max(LENGTHS), "bf16", kv_capacity=CAP, seq_lens=lens)
    pp = dbs.Problem.decode(S, hq, hkv, d, max(LENGTHS), "bf16", kv_capacity=CAP, block_table=table.to(dev),
                            pool_blocks=pool, seq_lens=lens)
    qd = q.to(dev)
    rc = _run(pc, cfg, qd, k.to(dev), v.to(dev))
    rp = _run(pp, cfg, qd, kp.to(dev), vp.to(dev))
    for s, L in enumerate(LENGTHS):
        nb = -(-L // B)
        assert torch.equal(rc[1][s, :, :nb], rp[1][s, :, :nb])
    assert torch.equal(rc[0], rp[0])
    _same_worklist(rc[2], rp[2])
    assert torch.equal(rc[2].err, rp[2].err)
    assert torch.equal(rc[3], rp[3]) and torch.equal(rc[4], rp[4])
    _check_decode(cfg, "bf16", LENGTHS, q, k, v, rc[0], rc[2], rc[3], rc[4])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_ragged_append_then_decode(dtype, d):
    dev = torch.device("cuda:0")
    hq, hkv, cap = 4, 2, 448
    len0 = [0, 1, 63, 64, 100, 5]
    chunks = (1, 70, 1, 64)
    S = len(len0)
    print(f"ragged append dtype={dtype} d={d} len0={len0} chunks={chunks}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(41)
    total = [a + sum(chunks) for a in len0]
    assert max(total) <= cap
    k_all = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    v_all = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    q = torch.randn((S, hq, d), generator=g).to(tdt).to(dev)
    sent = 7.0
    kc = torch.full((S, hkv, cap, d), sent, dtype=tdt)
    vc = torch.full((S, hkv, cap, d), sent, dtype=tdt)
    for s, L in enumerate(len0):
        kc[s, :, :L] = k_all[s, :, :L]
        vc[s, :, :L] = v_all[s, :, :L]
    kc, vc = kc.to(dev), vc.to(dev)
    cfg = dbs.RouteConfig(k_b=4, share_gqa=True)
    # summaries of the cached prefixes (a zero-length cache routes as one token:
    # its block 0 is rewritten by the first append, which starts from the new keys)
    start = [max(L, 1) for L in len0]
    prob = dbs.Problem.decode(S, hq, hkv, d, max(start), dtype, kv_capacity=cap, seq_lens=_lens(start, dev))
    summ = torch.full(dbs.summaries_shape(prob), -3.0, dtype=torch.float32, device=dev)
    dbs.route(prob, cfg, q, kc, summaries=summ)
    lens = list(len0)
    for n in chunks:
        prob = dbs.Problem.decode(S, hq, hkv, d, max(lens), dtype, kv_capacity=cap, seq_lens=_lens(lens, dev))
        k_new = torch.stack([k_all[s, :, lens[s]:lens[s] + n] for s in range(S)]).contiguous()
        v_new = torch.stack([v_all[s, :, lens[s]:lens[s] + n] for s in range(S)]).contiguous()
        dbs.append_kv(prob, k_new.to(dev), v_new.to(dev), kc, vc, summ)
        lens = [L + n for L in lens]
        torch.cuda.synchronize()
        kh, vh, sh = kc.cpu(), vc.cpu(), summ.cpu().double().numpy()
        err = 0.0
        for s, L in enumerate(lens):
            assert torch.equal(kh[s, :, :L], k_all[s, :, :L]) and torch.equal(vh[s, :, :L], v_all[s, :, :L])
            assert bool((kh[s, :, L:] == sent).all()) and bool((vh[s, :, L:] == sent).all())
            nb = -(-L // B)
            for h in range(hkv):
                ref = ocache.summaries_after(k_all[s, h, :L].double().numpy(), L, B)
                err = max(err, float(np.max(np.abs(sh[s, h, :nb] - ref))))
            assert (sh[s, :, nb:] == -3.0).all(), (s, L)
        assert err <= SUM_TOL, (lens, err)
    prob = dbs.Problem.decode(S, hq, hkv, d, max(lens), dtype, kv_capacity=cap, seq_lens=_lens(lens, dev))
    J, _s = dbs.route(prob, cfg, q, None, summaries=summ, summaries_in=True)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, q, kc, vc)
    torch.cuda.synchronize()
    _check_decode(cfg, dtype, lens, q.cpu(), k_all, v_all, J, wl, o, lse)


def test_lengths_outside_the_bound_are_clamped_and_reported():
    dev = torch.device("cuda:0")
    hq, hkv, d, n, cap = 8, 2, 128, 300, 320
    q, k, v = _inputs("bf16", d, hq, hkv, [cap, cap], cap, seed=43)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    cfg = dbs.RouteConfig(k_b=3, share_gqa=True)
    print("ragged decode: lengths 0 and 5000 against a bound of 300", flush=True)
    bad = dbs.Problem.decode(2, hq, hkv, d, n, "bf16", kv_capacity=cap, seq_lens=_lens([0, 5000], dev))
    good = dbs.Problem.decode(2, hq, hkv, d, n, "bf16", kv_capacity=cap, seq_lens=_lens([1, n], dev))
    rb, rg = _run(bad, cfg, q, k, v), _run(good, cfg, q, k, v)
    assert int(rb[2].err.item()) == dbs.SA_WL_ERR_LENGTH and int(rg[2].err.item()) == 0
    assert torch.equal(rb[0], rg[0])
    _same_worklist(rb[2], rg[2])
    assert torch.equal(rb[3], rg[3]) and torch.equal(rb[4], rg[4])
