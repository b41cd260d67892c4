"""Router quality of the GPU routing at the 8192-token MHA setting, measured by
the oracle (oracle/quality.py; [P2] §4): recall of the planted blocks and the
Eq (10) coverage of the dense causal attention.  Statistical sanity, not
parity: the inputs are N(0, 1) with 8 planted earlier blocks per head (K +=
2 u on them, Q += u), so

  recall    every planted block j < r must be in row r's worklist (its pooled
            score ~2 u.u = 2 stands far above the unplanted ones)
  coverage  the selected keys must hold more dense attention mass than their
            share of the causal keys (the planted keys draw extra weight)

The figures are printed for the record."""
import numpy as np
import pytest
import torch

from dynamic_block_sparse_amd import workloads as wk
from oracle import problem as oprob
from oracle import quality
from parity import run_gpu

pytestmark = pytest.mark.gpu


def test_router_quality_planted_mha():
    w = wk.PREFILL_MHA
    print(f"router quality on {w.name}", flush=True)
    inp = wk.make_inputs(w, torch.device("cuda:0"))
    run = run_gpu(w, inp)
    rp, ci = run.wl["row_ptr"], run.wl["col_idx"]
    table = oprob.row_table(inp.lengths, w.block, w.mode, w.route_heads)
    recalls = []
    for i, (s, h, r, _n) in enumerate(table):
        relevant = [int(j) for j in inp.planted[(s, h)] if j < r]
        recalls.append(quality.recall(ci[rp[i]:rp[i + 1]], relevant))
    recalls = np.array(recalls)
    q = inp.q[0].double().cpu().numpy()
    k = inp.k[0].double().cpu().numpy()
    index = {(s, h, r): i for i, (s, h, r, _n) in enumerate(table)}
    covs, ratios = [], []
    for h in range(w.heads_q):
        for r in (16, 64, 127):
            i = index[(0, h, r)]
            blocks = ci[rp[i]:rp[i + 1]].tolist()
            pos = np.arange(r * w.block, (r + 1) * w.block)
            c = quality.coverage(q[h, pos], pos, k[h], w.seqlen, w.block, blocks)
            attended = np.array([sum(min(w.block, p + 1 - j * w.block) for j in blocks if j * w.block <= p)
                                 for p in pos])
            covs.append(c)
            ratios.append(c / (attended / (pos + 1)))
    covs, ratios = np.concatenate(covs), np.concatenate(ratios)
    print(f"planted recall: mean {recalls.mean():.4f} min {recalls.min():.3f} over {len(recalls)} rows; "
          f"coverage (rows of blocks 16, 64, 127 of every head): mean {covs.mean():.4f} "
          f"min {covs.min():.4f}; coverage / share of causal keys: mean {ratios.mean():.3f}", flush=True)
    assert recalls.min() == 1.0
    assert ratios.mean() > 1.0
