"""sparse_attn_fwd_dense: dense causal attention through the sparse kernels.

Every query block attends every key block 0 .. r of its sequence ([P2] §3.1
dense fallback; the dense side of the sparse / dense comparison).  Checked
against the oracle's masked attention with every causal block listed (which
the oracle's pins tie to torch's fp64 causal SDPA), bit for bit against the
sparse call on a worklist that lists every block, and on rows longer than
any worklist row can be (256 blocks)."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import problem as oprob

pytestmark = pytest.mark.gpu

B = 64
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}


def _inputs(lengths, hq, hkv, d, dtype, dev, seed, fixed_n=None, cap=0, q0=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if fixed_n is not None:
        bsz = len(lengths)
        kcap = cap or fixed_n
        q = torch.randn((bsz, hq, fixed_n - q0, d), generator=g).to(tdt)
        k = torch.randn((bsz, hkv, kcap, d), generator=g).to(tdt)
        v = torch.randn((bsz, hkv, kcap, d), generator=g).to(tdt)
        prob = dbs.Problem.fixed(bsz, hq, hkv, d, fixed_n, dtype, kv_capacity=cap, q_start=q0)
        return prob, q, k, v, None
    T = sum(lengths)
    q = torch.randn((hq, T, d), generator=g).to(tdt)
    k = torch.randn((hkv, T, d), generator=g).to(tdt)
    v = torch.randn((hkv, T, d), generator=g).to(tdt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    prob = dbs.Problem.varlen(lengths, hq, hkv, d, cu, dtype)
    return prob, q, k, v, cu


def _seq_views(prob, q, k, v, lengths, q0=0):
    """Per-sequence fp64 numpy arrays for the oracle (queries padded back to the
    whole sequence for chunked prefill: rows before q0 are never compared)."""
    qs, ks, vs = [], [], []
    offs = np.concatenate([[0], np.cumsum(lengths)])
    for s, L in enumerate(lengths):
        if prob.cu_seqlens is None:
            qq = torch.zeros((q.shape[1], L, q.shape[3]), dtype=torch.float64)
            qq[:, q0:] = q[s].double()
            qs.append(qq.numpy())
            ks.append(k[s, :, :L].double().numpy())
            vs.append(v[s, :, :L].double().numpy())
        else:
            a, e = int(offs[s]), int(offs[s + 1])
            qs.append(q[:, a:e].double().numpy())
            ks.append(k[:, a:e].double().numpy())
            vs.append(v[:, a:e].double().numpy())
    return qs, ks, vs


def _check(prob, cfg, q, k, v, lengths, o, lse, dtype, rows=None, q0=0):
    share = cfg.share_gqa
    hr = prob.heads_kv if share else prob.heads_q
    table = oprob.row_table(lengths, B, "prefill", hr)
    if rows is None:
        rows = [i for i, t in enumerate(table) if t[2] * B >= q0]
    qs, ks, vs = _seq_views(prob, q, k, v, lengths, q0)
    blocks = {i: list(range(table[i][2] + 1)) for i in rows}
    res = oprob.attention_rows(qs, ks, vs, lengths, B, "prefill", share, rows, blocks)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    mx, mean_tol = TOL[dtype]
    worst, tot, cnt = 0.0, 0.0, 0
    for i in rows:
        s = table[i][0]
        for hh, toks, ref in res[i]:
            if prob.cu_seqlens is None:
                got = o[s, hh, toks - q0].float().cpu().numpy()
                gl = lse[s, hh, toks - q0].cpu().numpy()
            else:
                got = o[hh, int(offs[s]) + toks].float().cpu().numpy()
                gl = lse[hh, int(offs[s]) + toks].cpu().numpy()
            err = np.abs(got.astype(np.float64) - ref["o"])
            worst = max(worst, float(err.max()))
            tot += float(err.sum())
            cnt += err.size
            assert np.max(np.abs(gl - ref["lse"])) <= (1e-2 if dtype == "bf16" else 1e-5)
    print(f"dense: max-abs {worst:.3e} mean-abs {tot / cnt:.3e} over {cnt}", flush=True)
    assert worst <= mx and tot / cnt <= mean_tol


CASES = [
    # name, dtype, d, lengths, hq, hkv, share, fixed, cap, q0
    ("mha_n500", "bf16", 128, [500], 2, 2, False, True, 0, 0),
    ("gqa_shared_n700_b2", "bf16", 128, [700, 700], 8, 2, True, True, 0, 0),
    ("gqa_pairs_n300", "bf16", 128, [300], 4, 2, True, True, 0, 0),
    ("varlen_gqa", "bf16", 128, [64, 130, 300, 1], 8, 2, True, False, 0, 0),
    ("varlen_mha", "bf16", 128, [200, 64, 77], 2, 2, False, False, 0, 0),
    ("f32_d64_n300", "f32", 64, [300], 2, 2, False, True, 0, 0),
    ("chunked_q128_cap448", "bf16", 128, [400], 4, 4, False, True, 448, 128),
    ("gqa8_shared_n500", "bf16", 128, [500], 16, 2, True, True, 0, 0),
    ("varlen_empty_seqs", "bf16", 128, [64, 0, 300, 0, 1], 8, 2, True, False, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_dense_matches_oracle(case):
    name, dtype, d, lengths, hq, hkv, share, fixed, cap, q0 = case
    dev = torch.device("cuda:0")
    print(f"dense {name}", flush=True)
    prob, q, k, v, _cu = _inputs(lengths, hq, hkv, d, dtype, dev, 7, fixed_n=lengths[0] if fixed else None,
                                 cap=cap, q0=q0)
    cfg = dbs.RouteConfig(k_b=1, share_gqa=share)
    o, lse = dbs.fwd_dense(prob, cfg, q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    _check(prob, cfg, q, k, v, lengths, o.cpu(), lse.cpu(), dtype, q0=q0)


@pytest.mark.parametrize("share,hq,hkv", [(False, 2, 2), (True, 8, 2)])
def test_dense_equals_sparse_with_every_block_listed(share, hq, hkv):
    """A worklist with every causal block (k_b >= N) makes the sparse call visit
    the same tiles in the same order with the same kernel: bit-identical."""
    dev = torch.device("cuda:0")
    n = 1000   # 16 blocks, the last partial
    prob, q, k, v, _ = _inputs([n], hq, hkv, 128, "bf16", dev, 11, fixed_n=n)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    cfg = dbs.RouteConfig(k_b=16, share_gqa=share)
    J, _ = dbs.route(prob, cfg, q, k)
    wl = dbs.build_worklist(prob, cfg, J)
    o_s, lse_s = dbs.fwd(prob, cfg, wl, q, k, v)
    o_d, lse_d = dbs.fwd_dense(prob, cfg, q, k, v)
    torch.cuda.synchronize()
    rp = wl.row_ptr.cpu().numpy()
    assert int(rp[-1]) == sum(r + 1 for r in range(16)) * (hkv if share else hq)   # every causal tile listed
    assert torch.equal(o_s, o_d) and torch.equal(lse_s, lse_d)


@pytest.mark.parametrize("share,hq,hkv,lengths", [
    (False, 16, 16, [8192]),        # 2048 one-head rows: a persistent grid, two passes, 128-row groups
    (True, 8, 2, [2048, 2048]),     # four-head rows, 4 (sequence, head) pairs of 32 rows
    (False, 4, 4, [4096, 4096]),    # one-head rows, 8 pairs of 64 rows (not a multiple of 128)
])
def test_dense_walk_orders_cover_every_row(share, hq, hkv, lengths):
    """The dense call's row orders (longest-first groups of query blocks over
    the (sequence, head) pairs, mirrored passes of a persistent grid) reach
    every row: outputs start as NaN and none is left.  Every row computes its
    own result from its id, so reaching each row is what the order has to get
    right; the values are then checked bit for bit against the sparse call with
    every causal block listed, or, where a row has more blocks than a worklist
    row holds (128 with the forced current block), on sampled query blocks
    against the oracle."""
    dev = torch.device("cuda:0")
    n = lengths[0]
    prob, q, k, v, _ = _inputs(lengths, hq, hkv, 128, "bf16", dev, 17, fixed_n=n)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    nb = n // B
    print(f"dense walk orders: share={share} hq={hq} lengths={lengths}", flush=True)
    nan_o = lambda: torch.full_like(qd, float("nan"))
    nan_l = lambda: torch.full(qd.shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    cfg = dbs.RouteConfig(k_b=min(nb, 127), share_gqa=share)
    o_d, lse_d = dbs.fwd_dense(prob, cfg, qd, kd, vd, o=nan_o(), lse=nan_l())
    torch.cuda.synchronize()
    assert not torch.isnan(o_d).any() and not torch.isnan(lse_d).any()
    if nb <= 127:
        J, _ = dbs.route(prob, cfg, qd, kd)
        wl = dbs.build_worklist(prob, cfg, J)
        o_s, lse_s = dbs.fwd(prob, cfg, wl, qd, kd, vd, o=nan_o(), lse=nan_l())
        torch.cuda.synchronize()
        heads = hkv if share else hq
        assert int(wl.row_ptr[-1].item()) == len(lengths) * heads * nb * (nb + 1) // 2   # every causal tile
        assert torch.equal(o_s, o_d) and torch.equal(lse_s, lse_d)
    else:
        # the sparse call on the same shape (k_b = 16) takes the same mirrored
        # passes over its worklist rows: every row is written
        cfg16 = dbs.RouteConfig(k_b=16, share_gqa=share)
        J, _ = dbs.route(prob, cfg16, qd, kd)
        wl = dbs.build_worklist(prob, cfg16, J)
        o_s, lse_s = dbs.fwd(prob, cfg16, wl, qd, kd, vd, o=nan_o(), lse=nan_l())
        torch.cuda.synchronize()
        assert not torch.isnan(o_s).any() and not torch.isnan(lse_s).any()
        nrows = len(lengths) * (hkv if share else hq) * nb   # (sequence, routing head, query block)
        rows = sorted({0, nb - 1, nb, nrows - 1} | set(np.random.default_rng(1).integers(0, nrows, size=6).tolist()))
        _check(prob, cfg, q, k, v, lengths, o_d.cpu(), lse_d.cpu(), "bf16", rows=rows)


def test_dense_rows_longer_than_a_worklist_row():
    """n = 16384: rows of up to 256 blocks (a worklist row holds at most 128);
    sampled rows (first, last and random query blocks) against the oracle."""
    dev = torch.device("cuda:0")
    n, hq, hkv = 16384, 4, 1
    prob, q, k, v, _ = _inputs([n], hq, hkv, 128, "bf16", dev, 13, fixed_n=n)
    cfg = dbs.RouteConfig(k_b=1, share_gqa=True)
    o, lse = dbs.fwd_dense(prob, cfg, q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = sorted({0, 1, 255} | set(rng.integers(0, 256, size=4).tolist()))
    _check(prob, cfg, q, k, v, [n], o.cpu(), lse.cpu(), "bf16", rows=rows)
