"""GPU parity of the backward pass (sparse_attn_bwd) against the oracle's
gradients ([P2] §4 training paragraph, [P3]: the backward reuses the
forward's block selection).

The forward runs on the GPU (route, worklist, fwd); its worklist is the block
selection, which the forward parity tests already check bit for bit against
the oracle.  For every worklist row the oracle differentiates the plain
masked attention of that row's queries (fp64 autograd of the definition) over
the row's blocks; dQ of those queries is the row's dq, and dK, dV of a key are
the sums over every row (and, under shared GQA routing, every query head of
the group) that attends it.

Tolerances, per tensor with scale = max |reference|:
  bf16  |err| <= 8e-3 |ref| + 4e-3 scale.  The kernel reads the same bf16
        inputs the oracle sees and accumulates in fp32; the error is the bf16
        rounding of the result (<= 2^-9 |ref|, taken with a factor 4) plus
        terms of order 2^-9 scale from the bf16 operands P and dS of the
        second products and the bf16 output O inside D_i = dO . O.
  fp32  |err| <= 1e-4 |ref| + 2e-5 scale: fp32 accumulation over up to a few
        thousand terms, in an order the atomics do not fix; the absolute part
        covers the cancellation in dP - D near zeros of the gradient.
"""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from oracle import attention as oatt
from oracle import backward as obwd
from oracle import problem as oprob

pytestmark = pytest.mark.gpu

B = 64
RTOL = {"bf16": (8e-3, 4e-3), "f32": (1e-4, 2e-5)}

CASES = [
    # name, dtype, d, lengths (None: fixed), batch, hq, hkv, n, q_start, cap, k_b, share, first, window
    ("mha_bf16", "bf16", 128, None, 2, 2, 2, 700, 0, 0, 4, False, False, 1),
    ("gqa_shared_sink_win2", "bf16", 128, None, 1, 8, 2, 600, 0, 0, 3, True, True, 2),
    ("gqa_per_head", "bf16", 128, None, 1, 4, 2, 450, 0, 0, 3, False, False, 1),
    ("varlen_f32_d64", "f32", 64, [300, 577, 64], 3, 2, 1, 0, 0, 0, 3, False, True, 1),
    ("chunked_bf16", "bf16", 128, None, 1, 2, 2, 900, 512, 1024, 4, False, False, 1),
    ("varlen_bf16_gqa", "bf16", 128, [300, 577, 64, 1000], 4, 8, 2, 0, 0, 0, 4, True, True, 2),
    ("varlen_bf16_per_head", "bf16", 128, [700, 130], 2, 4, 2, 0, 0, 0, 3, False, False, 1),
    ("gqa8_shared", "bf16", 128, None, 1, 16, 2, 500, 0, 0, 4, True, False, 1),
    ("varlen_empty_seqs", "bf16", 128, [64, 0, 300, 0, 1], 5, 8, 2, 0, 0, 0, 4, True, True, 1),
    # groups of 3 and 6 query heads per KV head (the forward pads its last head quad)
    ("gqa3_shared", "bf16", 128, None, 1, 6, 2, 500, 0, 0, 4, True, True, 1),
    ("gqa6_shared_varlen", "bf16", 128, [300, 450], 2, 12, 2, 0, 0, 0, 4, True, False, 2),
    # key block 0 (forced for every row) listed by more pairs than the dK/dV
    # split target (at least 64): 35 rows x 4 heads = 140 pairs -> 3 chunks,
    # and 71 one-head rows -> 2 chunks
    ("gqa_shared_first_split", "bf16", 128, None, 1, 8, 2, 2200, 0, 0, 4, True, True, 1),
    ("mha_first_split", "bf16", 128, None, 1, 2, 2, 4500, 0, 0, 4, False, True, 1),
]


def _inputs(case, dev):
    name, dtype, d, lengths, bsz, hq, hkv, n, q0, cap, k_b, share, first, window = case
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(41)
    cfg = dbs.RouteConfig(k_b=k_b, share_gqa=share, force_first=first, window=window)
    if lengths is not None:
        total = sum(lengths)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
        q = torch.randn((hq, total, d), generator=g).to(tdt)
        k = torch.randn((hkv, total, d), generator=g).to(tdt)
        v = torch.randn((hkv, total, d), generator=g).to(tdt)
        do = torch.randn((hq, total, d), generator=g).to(tdt)
        prob = dbs.Problem.varlen(lengths, hq, hkv, d, cu.to(dev), dtype)
        # per-sequence views [H, len, d] for the oracle, token offset of each sequence
        views = [(int(cu[s]), lengths[s]) for s in range(bsz)]
        q_in = q
    else:
        kvn = cap or n
        q = torch.randn((bsz, hq, n, d), generator=g).to(tdt)
        k = torch.randn((bsz, hkv, kvn, d), generator=g).to(tdt)
        v = torch.randn((bsz, hkv, kvn, d), generator=g).to(tdt)
        do = torch.randn((bsz, hq, n - q0, d), generator=g).to(tdt)
        prob = dbs.Problem.fixed(bsz, hq, hkv, d, n, dtype, kv_capacity=cap, q_start=q0)
        views = None
        q_in = q[:, :, q0:].contiguous()
    return prob, cfg, q, q_in, k, v, do, views


def _seq(x, s, views):
    """[H, len, d] of sequence s (fp64 numpy)."""
    if views is None:
        return x[s].double().numpy()
    t0, ln = views[s]
    return x[:, t0:t0 + ln].double().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_bwd_matches_oracle(case):
    name, dtype, d, lengths, bsz, hq, hkv, n, q0, cap, k_b, share, first, window = case
    dev = torch.device("cuda:0")
    print(f"bwd {name}: dtype={dtype} d={d} batch={bsz} hq={hq} hkv={hkv} n={n} lengths={lengths} "
          f"q_start={q0} cap={cap}", flush=True)
    prob, cfg, q, q_in, k, v, do, views = _inputs(case, dev)
    qd, kd, vd, dod = q_in.to(dev), k.to(dev), v.to(dev), do.to(dev)
    J, _summ = dbs.route(prob, cfg, qd, kd)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, qd, kd, vd)
    dq, dk, dv = dbs.bwd(prob, cfg, wl, qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    assert int(wl.err.item()) == 0

    lens = lengths if lengths is not None else [n] * bsz
    hr = hkv if share else hq
    group = hq // hkv
    table = oprob.row_table(lens, B, "prefill", hr)
    r0 = q0 // B
    gpu_rows = [t for t in table if t[2] >= r0]
    rp, ci = wl.row_ptr.cpu().numpy(), wl.col_idx.cpu().numpy()
    assert J.shape[0] == len(gpu_rows)
    if name.endswith("_split"):
        # (row, head) pairs per (sequence, KV head, key block): the case must
        # put more than the split target's floor (64) on one block
        pairs = {}
        for i, (s, h, _r, _nk) in enumerate(gpu_rows):
            for b in ci[rp[i]:rp[i + 1]].tolist():
                key = (s, h if share else h // group, b)
                pairs[key] = pairs.get(key, 0) + (group if share else 1)
        assert max(pairs.values()) > 64, max(pairs.values())

    ref_dq = np.zeros(dq.shape, dtype=np.float64)
    ref_dk = np.zeros(dk.shape, dtype=np.float64)
    ref_dv = np.zeros(dv.shape, dtype=np.float64)
    # The kernels take D = dO . O from the O that the forward stored (bf16 or
    # fp32), not from the exact O.  A relative error e of O's elements moves
    # D_i by at most e sum_d |dO_id O_id|, and dQ_i (= c sum_j P_ij (dP_ij -
    # D_i) k_j) by c dD_i sum_j P_ij |k_j|.  A row with few keys does not
    # average that out (row 0's first query attends to one key: its exact dQ
    # is 0), so the bound on dQ carries this term, with e = 2^-8 for bf16 (the
    # rounding to 8 significant bits, plus the forward's fp32 sums).
    slack_dq = np.zeros(dq.shape, dtype=np.float64)
    e_o = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -20
    seqs = {}
    for i, (s, h, r, _nk) in enumerate(gpu_rows):
        if s not in seqs:
            seqs[s] = tuple(_seq(x, s, views) for x in (q, k, v))
        qs, ks, vs = seqs[s]
        length = lens[s]
        toks = np.arange(r * B, min((r + 1) * B, length))
        blocks = ci[rp[i]:rp[i + 1]].tolist()
        heads = range(h * group, (h + 1) * group) if share else [h]
        for hh in heads:
            kvh = hh // group
            if views is None:
                dout = do[s, hh, toks - q0].double().numpy()
            else:
                dout = do[hh, views[s][0] + toks].double().numpy()
            gq, gk, gv = obwd.masked_attention_grads(qs[hh, toks], toks, ks[kvh], vs[kvh], length, B, blocks,
                                                     True, dout)
            fw = oatt.masked_attention(qs[hh, toks], toks, ks[kvh], vs[kvh], length, B, blocks, True)
            d_err = e_o * np.abs(dout * fw["o"]).sum(axis=1)
            sq = d_err[:, None] * (fw["p"] @ np.abs(ks[kvh][:length])) / np.sqrt(d)
            if views is None:
                slack_dq[s, hh, toks - q0] = sq
            else:
                slack_dq[hh, views[s][0] + toks] = sq
            if views is None:
                ref_dq[s, hh, toks - q0] = gq
                ref_dk[s, kvh, :length] += gk
                ref_dv[s, kvh, :length] += gv
            else:
                t0 = views[s][0]
                ref_dq[hh, t0 + toks] = gq
                ref_dk[kvh, t0:t0 + length] += gk
                ref_dv[kvh, t0:t0 + length] += gv

    rtol, stol = RTOL[dtype]
    for label, got, ref in (("dq", dq, ref_dq), ("dk", dk, ref_dk), ("dv", dv, ref_dv)):
        g64 = got.float().cpu().numpy().astype(np.float64)
        scale = float(np.max(np.abs(ref)))
        err = np.abs(g64 - ref)
        bound = rtol * np.abs(ref) + stol * scale + (slack_dq if label == "dq" else 0.0)
        worst = float(np.max(err - bound))
        print(f"bwd {name} {label}: scale {scale:.3e} max-abs {err.max():.3e} mean-abs {err.mean():.3e}",
              flush=True)
        assert worst <= 0, (name, label, np.unravel_index(np.argmax(err - bound), err.shape))
    if dtype == "bf16":
        # dQ has no atomics: a second call repeats every bit.  dK, dV of a key
        # block shared by several workgroups are summed in atomic order, so
        # they may differ in the last bf16 bit.
        dq2, dk2, dv2 = dbs.bwd(prob, cfg, wl, qd, kd, vd, o, lse, dod)
        assert torch.equal(dq, dq2)
        for a, b in ((dk, dk2), (dv, dv2)):
            assert torch.allclose(a.float(), b.float(), rtol=2 ** -7, atol=1e-6)
    # keys past the sequence end (capacity tail) get exactly zero
    if cap:
        assert not dk[:, :, n:].any() and not dv[:, :, n:].any()


def test_bwd_rejects_decode_and_other_head_dims():
    dev = torch.device("cuda:0")
    prob = dbs.Problem.fixed(1, 2, 2, 64, 128, "bf16")
    cfg = dbs.RouteConfig(k_b=2)
    x = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device=dev)
    J, _ = dbs.route(prob, cfg, x, x)
    wl = dbs.build_worklist(prob, cfg, J)
    lse = torch.zeros((1, 2, 128), dtype=torch.float32, device=dev)
    with pytest.raises(dbs.SAError):
        dbs.bwd(prob, cfg, wl, x, x, x, x, lse, x)


def test_bwd_graph_replay_matches_eager():
    """The backward enqueues kernels only (its counters and accumulators are
    cleared by fill kernels), so it can be captured in a HIP graph: three
    replays, with eager work on the same buffers between them, must each
    reproduce the eager result bit for bit (no key block is shared here)."""
    dev = torch.device("cuda:0")
    bsz, hq, hkv, d, n = 1, 2, 2, 128, 450
    print(f"bwd graph replay: n={n}", flush=True)
    g = torch.Generator().manual_seed(43)
    q, k, v, do = (torch.randn((bsz, h, n, d), generator=g).to(torch.bfloat16).to(dev)
                   for h in (hq, hkv, hkv, hq))
    prob = dbs.Problem.fixed(bsz, hq, hkv, d, n, "bf16")
    cfg = dbs.RouteConfig(k_b=3)
    J, _s = dbs.route(prob, cfg, q, k)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, q, k, v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(dbs.workspace_size(prob, cfg, 3), dtype=torch.uint8, device=dev)
    dbs.bwd(prob, cfg, wl, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dbs.bwd(prob, cfg, wl, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dbs.bwd(prob, cfg, wl, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws)
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(float(rep + 1))          # eager work between replays
        ws.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(t, r), (rep, name)
