"""GPU: the three calls captured in a HIP graph replay to the eager results.

The library enqueues only kernels on the caller's stream (no memset, no
allocation, no synchronisation), so route + worklist + fwd can be captured
once and replayed.  Each replay follows eager work on other buffers and a
synchronisation, and must reproduce the eager J, worklist, output and
log-sum-exp bit for bit (the path is deterministic).
"""
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from dynamic_block_sparse_amd import workloads as wk

pytestmark = pytest.mark.gpu


class _Step:
    def __init__(self, w, inp, summaries_in=False):
        self.w, self.inp = w, inp
        self.prob, self.cfg = dbs.problem_for(w, inp), dbs.config_for(w)
        dev = inp.q.device
        sz = dbs.sizes(self.prob, self.cfg)
        self.J = torch.empty((sz.rows, w.k_b), dtype=torch.int32, device=dev)
        self.summ = torch.empty(dbs.summaries_shape(self.prob), dtype=torch.float32, device=dev)
        self.wl = dbs.alloc_worklist(self.prob, self.cfg, dev)
        self.o = torch.empty_like(inp.q)
        self.lse = torch.empty(inp.q.shape[:-1], dtype=torch.float32, device=dev)
        self.ws = [torch.empty(max(dbs.workspace_size(self.prob, self.cfg, i, 0), 1), dtype=torch.uint8,
                               device=dev) for i in range(3)]
        self.summaries_in = summaries_in
        if summaries_in:
            dbs.route(self.prob, self.cfg, inp.q, inp.k, summaries=self.summ, J=self.J, workspace=self.ws[0])

    def __call__(self):
        dbs.route(self.prob, self.cfg, self.inp.q, None if self.summaries_in else self.inp.k,
                  summaries=self.summ, summaries_in=self.summaries_in, J=self.J, workspace=self.ws[0])
        dbs.build_worklist(self.prob, self.cfg, self.J, out=self.wl, workspace=self.ws[1])
        dbs.fwd(self.prob, self.cfg, self.wl, self.inp.q, self.inp.k, self.inp.v, o=self.o, lse=self.lse,
                workspace=self.ws[2])

    def outputs(self):
        rows = self.J.shape[0]
        nnz = int(self.wl.row_ptr[rows].item())   # col_idx is written up to nnz only
        return {"J": self.J.clone(), "row_ptr": self.wl.row_ptr.clone(),
                "col_idx": self.wl.col_idx[:nnz].clone(), "row_perm": self.wl.row_perm[:rows].clone(),
                "bucket_ptr": self.wl.bucket_ptr.clone(), "err": self.wl.err.clone(),
                "o": self.o.clone(), "lse": self.lse.clone()}


@pytest.mark.parametrize("w", [
    wk.PREFILL_MHA.replace(name="graph_mha", heads_q=4, heads_kv=4, seqlen=2048),
    wk.PREFILL_GQA.replace(name="graph_gqa", batch=1, heads_q=8, heads_kv=2, seqlen=4096),
    wk.DECODE.replace(name="graph_decode", batch=4, seqlen=16384),
], ids=lambda w: w.name)
def test_graph_replay_matches_eager(w):
    dev = torch.device("cuda:0")
    dbs.load_library()
    inp = wk.make_inputs(w, dev)
    step = _Step(w, inp, summaries_in=(w.mode == "decode"))
    step()
    torch.cuda.synchronize()
    ref = step.outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        # eager work between replays, then clobber the outputs
        other.mul_(1.5).add_(rep)
        for x in (step.J, step.wl.col_idx, step.o, step.lse):
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for name in ref:
            assert torch.equal(got[name], ref[name]), f"replay {rep}: {name} differs"
