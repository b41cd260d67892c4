"""GPU-vs-oracle comparison helpers (test infrastructure).

Acceptance rules:
  router     per row, the selected set may differ from the oracle's only among
             candidates whose exact (fp64) score lies within a 1e-5 relative band
             of the selection boundary: the D-th / (D+1)-th score for top-k, and
             tau for Eq 7's count; forced blocks must be present
  worklist   bit-exact: row_ptr, col_idx, row_perm, bucket_ptr and err equal
             the oracle's worklist built from the GPU's own J
  output     against the oracle's masked attention on the GPU worklist:
             bf16 max-abs <= 2e-2 and mean-abs <= 5e-3; fp32 max-abs <= 1e-5
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import dynamic_block_sparse_amd as dbs
from dynamic_block_sparse_amd import workloads as wk
from oracle import problem as oprob
from oracle import routing as orout

TIE_REL = 1e-5
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}
# log-sum-exp, natural log units.  bf16 path: Q is rounded to bf16 after the
# log2(e)/sqrt(d) pre-scale (score error ~1e-3) and the normaliser sums the
# bf16-rounded weights (relative error <= 2^-9); 1e-2 bounds both.  fp32 path:
# fp32 rounding only.
LSE_TOL = {"bf16": 1e-2, "f32": 1e-5}


@dataclasses.dataclass
class GpuRun:
    J: np.ndarray
    summaries: torch.Tensor
    wl: dict
    o: torch.Tensor
    lse: torch.Tensor


def run_gpu(w, inp, num_splits: int = 0) -> GpuRun:
    prob = dbs.problem_for(w, inp)
    cfg = dbs.config_for(w)
    J, summ = dbs.route(prob, cfg, inp.q, inp.k)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, inp.q, inp.k, inp.v, num_splits=num_splits)
    torch.cuda.synchronize()
    rows = J.shape[0]
    nnz = int(wl.row_ptr[rows].item())
    wld = dict(row_ptr=wl.row_ptr.cpu().numpy(), col_idx=wl.col_idx[:nnz].cpu().numpy(),
               row_perm=wl.row_perm[:rows].cpu().numpy(), bucket_ptr=wl.bucket_ptr.cpu().numpy(),
               err=int(wl.err.item()))
    return GpuRun(J.cpu().numpy(), summ, wld, o, lse)


def check_worklist(w, inp, run: GpuRun):
    """Bit-exact worklist equality against the oracle applied to the GPU's J."""
    sz = dbs.sizes(dbs.problem_for(w, inp), dbs.config_for(w))
    ref = oprob.worklist(run.J, inp.lengths, w.block, w.mode, w.route_heads, w.forced_first,
                         sz.width_max, window=w.window)
    for key in ("row_ptr", "col_idx", "row_perm", "bucket_ptr"):
        assert np.array_equal(np.asarray(run.wl[key], np.int64), ref[key]), key
    assert run.wl["err"] == ref["err"]
    return ref


def _boundary_ok(picks, g, cands, d):
    ranked = sorted(cands, key=lambda j: (-g[j], j))
    ref = set(ranked[:d])
    if picks == ref:
        return True, 0
    if d == 0 or d >= len(ranked):
        return False, len(picks ^ ref)
    t, t2 = g[ranked[d - 1]], g[ranked[d]]
    band = TIE_REL * max(abs(t), abs(t2))
    for j in picks - ref:      # picked by the GPU, not by the oracle: must be tied with the boundary
        if g[j] < t - band:
            return False, len(picks ^ ref)
    for j in ref - picks:      # dropped: must not be clearly above the boundary
        if g[j] > t2 + band:
            return False, len(picks ^ ref)
    return True, len(picks ^ ref)


def check_router_row(j_row, scores, w):
    """Returns (ok, n_tie_differences) for one row."""
    g, cands, forced = scores
    got = set(int(x) for x in j_row if x != -1)
    if not set(forced) <= got:
        return False, -1
    picks = got - set(forced)
    if not picks <= set(cands):
        return False, -1
    if w.select == "topk":
        dset = {min(max(w.k_b - len(forced), 0), len(cands))}
    else:
        # Eq 7 count: candidates within the band around tau may fall either way
        if cands:
            gmax = max(g[j] for j in cands)
            tau = gmax - w.tau_rel
            band = TIE_REL * max(abs(tau), abs(gmax))
            lo = sum(1 for j in cands if g[j] >= tau + band)
            hi = sum(1 for j in cands if g[j] >= tau - band)
        else:
            lo = hi = 0
        dset = set()
        for cnt in range(lo, hi + 1):
            k_r = min(w.k_b, max(w.k_min, len(forced) + cnt))
            dset.add(min(max(k_r - len(forced), 0), len(cands)))
    if len(picks) not in dset:
        return False, -1
    return _boundary_ok(picks, g, cands, len(picks))


def check_router(w, inp, run: GpuRun, seqs=None):
    """Route on the oracle for `seqs` (all by default) and compare every row."""
    if seqs is None:
        qs, ks, _vs = wk.per_sequence(inp)
    else:
        qs, ks, _vs = wk.per_sequence_subset(inp, seqs)
    lengths = inp.lengths
    _j, scores = oprob.route(qs_full(qs, seqs, len(lengths)), qs_full(ks, seqs, len(lengths)),
                             lengths, w.block, w.mode, w.qpool, w.share_gqa, w.select, w.k_b,
                             w.k_min, w.tau_rel, w.forced_first, seqs=seqs, window=w.window)
    bad, ties, checked = [], 0, 0
    for i, sc in enumerate(scores):
        if sc is None:
            continue
        ok, nd = check_router_row(run.J[i], sc, w)
        checked += 1
        if not ok:
            bad.append(i)
        elif nd > 0:
            ties += 1
    return dict(checked=checked, bad=bad, tie_rows=ties)


def qs_full(parts, seqs, n):
    if seqs is None:
        return parts
    out = [None] * n
    for s, x in zip(seqs, parts):
        out[s] = x
    return out



def check_output(w, inp, run: GpuRun, row_ids, wl_ref=None):
    """Compare O (and LSE) of the given rows with the oracle's masked attention."""
    wl = wl_ref if wl_ref is not None else run.wl
    rp, ci = wl["row_ptr"], wl["col_idx"]
    table = oprob.row_table(inp.lengths, w.block, w.mode, w.route_heads)
    seqs = sorted(set(table[i][0] for i in row_ids))
    parts = wk.per_sequence_subset(inp, seqs)
    qs, ks, vs = (qs_full(p, seqs, len(inp.lengths)) for p in parts)
    blocks = {i: ci[rp[i]:rp[i + 1]].tolist() for i in row_ids}
    res = oprob.attention_rows(qs, ks, vs, inp.lengths, w.block, w.mode, w.share_gqa, row_ids,
                               blocks)
    max_err, sum_err, cnt, lse_err = 0.0, 0.0, 0, 0.0
    offs = np.concatenate([[0], np.cumsum(inp.lengths)])
    for i in row_ids:
        s = table[i][0]
        for hh, toks, ref in res[i]:
            if w.mode == "decode":
                got = run.o[s, hh].float().cpu().numpy()[None]
                gl = run.lse[s, hh].float().cpu().numpy()[None]
            elif w.varlen:
                a = int(offs[s])
                got = run.o[hh, a + toks].float().cpu().numpy()
                gl = run.lse[hh, a + toks].float().cpu().numpy()
            else:
                got = run.o[s, hh, toks].float().cpu().numpy()
                gl = run.lse[s, hh, toks].float().cpu().numpy()
            err = np.abs(got.astype(np.float64) - ref["o"])
            max_err = max(max_err, float(err.max()))
            sum_err += float(err.sum())
            cnt += err.size
            lse_err = max(lse_err, float(np.max(np.abs(gl - ref["lse"]))))
    return dict(max_abs=max_err, mean_abs=sum_err / max(cnt, 1), lse_max_abs=lse_err, n=cnt)


def sample_rows(w, inp, per_seq_head: int = 3, seed: int = 0, seqs=None):
    """Rows of blocks 0, 1, N-1 plus random ones, for each (sequence, routing head)."""
    rng = np.random.default_rng(seed)
    table = oprob.row_table(inp.lengths, w.block, w.mode, w.route_heads)
    by = {}
    for i, (s, h, r, n_k) in enumerate(table):
        if seqs is not None and s not in seqs:
            continue
        by.setdefault((s, h), []).append((r, i, n_k))
    out = []
    for (s, h), lst in by.items():
        n_k = lst[0][2]
        if w.mode == "decode":
            out.extend(i for _r, i, _n in lst)
            continue
        want = {0, 1, n_k - 1} | set(rng.integers(0, n_k, size=per_seq_head).tolist())
        out.extend(i for r, i, _n in lst if r in want)
    return sorted(out)
