"""GPU parity of the paged decode cache: K/V in a pool of [pool, Hkv, b, d]
pages addressed through a per-sequence block table ([P2] §3.1: block ids
stay sequence-local logical ids; where a block lives is the cache's business).

The same logical cache is run twice, stored contiguously and scattered over
randomly permuted pages: routing (summaries computed from the pool), the
worklist, the decode attention and an append must agree bit for bit, and the
output must match the oracle on the logical cache.  A table entry outside
the pool is reported by the worklist builder (SA_WL_ERR_PAGE); the kernels
clamp page ids, so no access leaves the pool.
"""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import problem as oprob
from parity import TOL

pytestmark = pytest.mark.gpu

B = 64


def _paged_case(dtype, d, S, hq, hkv, L, cap, pool, seed):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    v = torch.randn((S, hkv, cap, d), generator=g).to(tdt)
    q = torch.randn((S, hq, d), generator=g).to(tdt)
    nbc = cap // B
    table = torch.randperm(pool, generator=g)[:S * nbc].reshape(S, nbc).to(torch.int32)
    kp = torch.randn((pool, hkv, B, d), generator=g).to(tdt)   # unused pages hold noise
    vp = torch.randn((pool, hkv, B, d), generator=g).to(tdt)
    for s in range(S):
        for j in range(nbc):
            kp[table[s, j]] = k[s, :, j * B:(j + 1) * B]
            vp[table[s, j]] = v[s, :, j * B:(j + 1) * B]
    return dev, q.to(dev), k.to(dev), v.to(dev), kp.to(dev), vp.to(dev), table.to(dev)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_paged_decode_matches_contiguous_and_oracle(dtype, d):
    S, hq, hkv, L, cap, pool = 3, 8, 2, 950, 1024, 64
    print(f"paged decode dtype={dtype} d={d} S={S} L={L} cap={cap} pool={pool}", flush=True)
    dev, q, k, v, kp, vp, table = _paged_case(dtype, d, S, hq, hkv, L, cap, pool, seed=21)
    cfg = dbs.RouteConfig(k_b=6, share_gqa=True, window=2)
    pc = dbs.Problem.decode(S, hq, hkv, d, L, dtype, kv_capacity=cap)
    pp = dbs.Problem.decode(S, hq, hkv, d, L, dtype, kv_capacity=cap, block_table=table, pool_blocks=pool)
    out = {}
    for name, prob, kk, vv in (("contiguous", pc, k, v), ("paged", pp, kp, vp)):
        J, summ = dbs.route(prob, cfg, q, kk)
        wl = dbs.build_worklist(prob, cfg, J)
        o, lse = dbs.fwd(prob, cfg, wl, q, kk, vv)
        torch.cuda.synchronize()
        out[name] = (J, summ, wl, o, lse)
    (Jc, sc, wc, oc, lc), (Jp, sp, wp, op, lp) = out["contiguous"], out["paged"]
    nb = -(-L // B)   # summary slots past the valid blocks are never written
    assert torch.equal(Jc, Jp) and torch.equal(sc[:, :, :nb], sp[:, :, :nb])
    nnz = int(wc.row_ptr[-1].item())
    for key in ("row_ptr", "row_perm", "bucket_ptr", "err"):
        assert torch.equal(getattr(wc, key), getattr(wp, key)), key
    assert torch.equal(wc.col_idx[:nnz], wp.col_idx[:nnz])
    assert int(wp.err.item()) == 0
    assert torch.equal(oc, op) and torch.equal(lc, lp)
    # the paged output against the oracle on the logical cache
    qs = [q[s].unsqueeze(1).double().cpu().numpy() for s in range(S)]
    ks = [k[s, :, :L].double().cpu().numpy() for s in range(S)]
    vs = [v[s, :, :L].double().cpu().numpy() for s in range(S)]
    rows = Jp.shape[0]
    rp, ci = wp.row_ptr.cpu().numpy(), wp.col_idx.cpu().numpy()
    blocks = {i: ci[rp[i]:rp[i + 1]].tolist() for i in range(rows)}
    res = oprob.attention_rows(qs, ks, vs, [L] * S, B, "decode", True, list(range(rows)), blocks)
    errs = [np.abs(op[i // hkv, hh].float().cpu().numpy().astype(np.float64) - ref["o"][0])
            for i in range(rows) for hh, _t, ref in res[i]]
    e = np.concatenate(errs)
    mx, mean = TOL[dtype]
    assert e.max() <= mx and e.mean() <= mean, (e.max(), e.mean())

    # append 40 tokens (blocks 14 and 15) into both layouts
    n = 40
    g = torch.Generator().manual_seed(22)
    tdt = k.dtype
    kn = torch.randn((S, hkv, n, d), generator=g).to(tdt).to(dev)
    vn = torch.randn((S, hkv, n, d), generator=g).to(tdt).to(dev)
    dbs.append_kv(pc, kn, vn, k, v, sc)
    dbs.append_kv(pp, kn, vn, kp, vp, sp)
    torch.cuda.synchronize()
    assert torch.equal(sc, sp)
    tb = table.cpu()
    for s in range(S):
        for j in range(cap // B):
            assert torch.equal(kp[tb[s, j]], k[s, :, j * B:(j + 1) * B])
            assert torch.equal(vp[tb[s, j]], v[s, :, j * B:(j + 1) * B])


def test_page_outside_pool_is_reported():
    S, hq, hkv, d, L, cap, pool = 2, 8, 2, 128, 640, 640, 32
    dev, q, k, v, kp, vp, table = _paged_case("bf16", d, S, hq, hkv, L, cap, pool, seed=23)
    bad = table.clone()
    bad[1, 9] = pool + 5            # the current (last) block of sequence 1: always in its row
    print("paged decode with one page id outside the pool", flush=True)
    prob = dbs.Problem.decode(S, hq, hkv, d, L, "bf16", kv_capacity=cap, block_table=bad, pool_blocks=pool)
    cfg = dbs.RouteConfig(k_b=4, share_gqa=True)
    J, _summ = dbs.route(prob, cfg, q, kp)
    wl = dbs.build_worklist(prob, cfg, J)
    torch.cuda.synchronize()
    assert int(wl.err.item()) & dbs.SA_WL_ERR_PAGE
    rp, ci = wl.row_ptr.cpu().numpy(), wl.col_idx.cpu().numpy()
    for i in range(hkv, 2 * hkv):   # sequence 1's rows: block 9 dropped
        assert 9 not in ci[rp[i]:rp[i + 1]].tolist()
    for i in range(hkv):            # sequence 0's rows keep their current block
        assert 9 in ci[rp[i]:rp[i + 1]].tolist()
