#!/usr/bin/env python3
"""Benchmark: one hot-path step of dynamic block-sparse attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM:

    sparse_attn_route -> sparse_attn_build_worklist -> sparse_attn_fwd

on the 8192-token MHA prefill setting (B=1, H=16, n=8192, d=128, b=64,
k_b=16, bf16, planted relevance).  `value` is the selected-tile FLOPs of the
step (4*b*b*d per (query head, tile) visit of the worklist) divided by the
whole step's time, in TFLOP/s.  The attention kernel alone is reported in
`roofline` against the bf16 dense MFMA peak; routing and worklist times are
reported separately in `stages_ms`.  The split-KV decode setting (64 x
131072-token caches, Hq=32, Hkv=8, k_b=64) is timed too and reported under
`decode` as KV GB/s against the HBM peak.

The fp64 CPU oracle is timed on a bounded sample of the same prefill input
(`cpu_baseline`): a reported baseline, not a target.

    python bench.py [--steps K] [--warmup W] [--no-decode] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd TFLOP/s on selected tiles (% MFMA peak); decode KV GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha256") != source_sha(rec["source"]):
        return None
    return rec["bytes_per_launch"]


class Stepper:
    """Preallocated buffers and the three calls of one step."""

    def __init__(self, dbs, w, inp, summaries_in=False, num_splits=0):
        import torch
        self.dbs, self.w, self.inp = dbs, w, inp
        self.prob, self.cfg = dbs.problem_for(w, inp), dbs.config_for(w)
        dev = inp.q.device
        sz = dbs.sizes(self.prob, self.cfg)
        self.sz = sz
        self.J = torch.empty((sz.rows, w.k_b), dtype=torch.int32, device=dev)
        self.summ = torch.empty(dbs.summaries_shape(self.prob), dtype=torch.float32, device=dev)
        self.wl = dbs.alloc_worklist(self.prob, self.cfg, dev)
        self.o = torch.empty_like(inp.q)
        self.lse = torch.empty(inp.q.shape[:-1], dtype=torch.float32, device=dev)
        mk = lambda n: torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        self.ws = [mk(dbs.workspace_size(self.prob, self.cfg, i, num_splits)) for i in range(3)]
        self.summaries_in = summaries_in
        self.num_splits = num_splits
        if summaries_in:   # summaries are cache state: build them once, outside any timing
            dbs.route(self.prob, self.cfg, inp.q, inp.k, summaries=self.summ, J=self.J, workspace=self.ws[0])

    def route(self):
        self.dbs.route(self.prob, self.cfg, self.inp.q, None if self.summaries_in else self.inp.k,
                       summaries=self.summ, summaries_in=self.summaries_in, J=self.J,
                       workspace=self.ws[0])

    def worklist(self):
        self.dbs.build_worklist(self.prob, self.cfg, self.J, out=self.wl, workspace=self.ws[1])

    def fwd(self):
        self.dbs.fwd(self.prob, self.cfg, self.wl, self.inp.q, self.inp.k, self.inp.v, o=self.o,
                     lse=self.lse, num_splits=self.num_splits, workspace=self.ws[2])

    def step(self, ev=None):
        if ev is not None:
            ev[0].record()
        self.route()
        if ev is not None:
            ev[1].record()
        self.worklist()
        if ev is not None:
            ev[2].record()
        self.fwd()
        if ev is not None:
            ev[3].record()

    def tile_visits(self):
        """Sum over rows of unique tiles times the query heads each row serves."""
        nnz = int(self.wl.row_ptr[self.sz.rows].item())
        return nnz * (self.w.group if self.w.share_gqa else 1)


def timed(stepper, steps, warmup):
    import torch
    for _ in range(warmup):
        stepper.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        stepper.step(evs[i])
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    stage = [sum(e[k].elapsed_time(e[k + 1]) for e in evs) / steps for k in range(3)]
    fwd_all = sorted(e[2].elapsed_time(e[3]) for e in evs)
    return total / steps, stage, fwd_all


def graph_timed(stepper, steps, warmup):
    """The whole step (route, worklist, fwd) captured once in a HIP graph and
    replayed: the same kernels on the same resident buffers, without the host
    launch gaps between the seven small launches of an eager step."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stepper.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stepper.step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(w, inp, heads):
    """The fp64 oracle on `heads` heads of the prefill input: route, worklist, attention."""
    import numpy as np
    from oracle import problem as oprob
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:   # threadpoolctl absent: report the affinity mask
        cores = len(os.sched_getaffinity(0))
    q = inp.q[0, :heads].double().cpu().numpy()
    k = inp.k[0, :heads].double().cpu().numpy()
    v = inp.v[0, :heads].double().cpu().numpy()
    lengths = [w.seqlen]
    t0 = time.perf_counter()
    J, _ = oprob.route([q], [k], lengths, w.block, w.mode, w.qpool, w.share_gqa, w.select, w.k_b,
                       w.k_min, w.tau_rel, w.forced_first)
    t1 = time.perf_counter()
    wl = oprob.worklist(J, lengths, w.block, w.mode, heads, w.forced_first, w.k_b + 1)
    t2 = time.perf_counter()
    rows = list(range(len(J)))
    blocks = {i: wl["col_idx"][wl["row_ptr"][i]:wl["row_ptr"][i + 1]].tolist() for i in rows}
    oprob.attention_rows([q], [k], [v], lengths, w.block, w.mode, w.share_gqa, rows, blocks)
    t3 = time.perf_counter()
    flops = int(wl["row_ptr"][-1]) * 4 * w.block * w.block * w.head_dim
    return dict(value=round(flops / (t3 - t0) / 1e12, 6), unit="TFLOP/s", cores=int(cores),
                kind="oracle",
                sample=f"{heads} of {w.heads_q} heads of the prefill input, all {len(rows) // heads} "
                       f"query blocks: route {t1 - t0:.2f}s, worklist {t2 - t1:.2f}s, "
                       f"masked attention {t3 - t2:.2f}s ({flops / 1e9:.2f} GFLOP of selected tiles)",
                seconds=round(t3 - t0, 3))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--decode-splits", type=int, default=0)
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all",
                    help="profiling aid: time one setting only (the JSON line then lacks the other)")
    ap.add_argument("--no-graph", action="store_true",
                    help="profiling aid: time eager steps only (value then comes from eager steps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="profiling aid: run a plain device copy of this many MiB (5 times) first, "
                         "the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import dynamic_block_sparse_amd as dbs
    from dynamic_block_sparse_amd import workloads as wk

    dev = torch.device("cuda:0")
    dbs.load_library()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log(f"copy calibration: 5 copies of {args.copy_calibration} MiB")
    w = wk.PREFILL_MHA
    out = {}
    if args.only == "decode":
        return run_decode(args, dbs, wk, dev, out, None, w)
    log(f"generating {w.name}")
    inp = wk.make_inputs(w, dev)
    st = Stepper(dbs, w, inp)
    log("timing prefill steps")
    eager_ms, stage, fwd_all = timed(st, args.steps, args.warmup)
    ms = eager_ms if args.no_graph else graph_timed(st, args.steps, args.warmup)
    visits = st.tile_visits()
    flops = visits * 4 * w.block * w.block * w.head_dim
    fwd_ms = stage[2]
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    err = int(st.wl.err.item())
    out.update({
        "metric": METRIC,
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V with planted relevance; no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seqlen": w.seqlen, "head_dim": w.head_dim, "block": w.block, "k_b": w.k_b,
                   "qpool": w.qpool, "tile_visits": visits, "selected_tile_flops": flops},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<1>",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("prefill_bf16_kernel")},
        "step": ("eager steps (--no-graph)" if args.no_graph else
                 "HIP graph replay of route + worklist + fwd") +
                "; eager_ms_per_step: the step launched call by call, stages_ms: its per-call split",
        "eager_ms_per_step": round(eager_ms, 5),
        "stages_ms": {"route": round(stage[0], 5), "worklist": round(stage[1], 5),
                      "fwd": round(stage[2], 5), "fwd_p10": round(fwd_all[len(fwd_all) // 10], 5),
                      "fwd_p90": round(fwd_all[(len(fwd_all) * 9) // 10], 5)},
        "worklist_err": err,
    })
    del st
    run_decode(args, dbs, wk, dev, out, inp, w)


def run_decode(args, dbs, wk, dev, out, inp, w):
    import torch
    if not args.no_decode and args.only != "prefill":
        wd = wk.DECODE
        log(f"generating {wd.name}")
        inp_d = wk.make_inputs(wd, dev)
        sd = Stepper(dbs, wd, inp_d, summaries_in=True, num_splits=args.decode_splits)
        log("timing decode steps")
        eager_msd, stage_d, _ = timed(sd, max(args.steps // 2, 10), args.warmup)
        msd = eager_msd if args.no_graph else graph_timed(sd, max(args.steps // 2, 10), args.warmup)
        nnz = int(sd.wl.row_ptr[sd.sz.rows].item())
        kv_bytes = nnz * wd.block * wd.head_dim * 2 * 2
        qo_bytes = 2 * wd.batch * wd.heads_q * wd.head_dim * 2
        gbs = (kv_bytes + qo_bytes) / (stage_d[2] * 1e-3) / 1e9
        route_bytes = wd.batch * wd.heads_kv * (wd.seqlen // wd.block) * wd.head_dim * 4
        out["decode"] = {
            "workload": wd.name, "ms_per_step": round(msd, 5), "eager_ms_per_step": round(eager_msd, 5),
            "stages_ms": {"route": round(stage_d[0], 5), "worklist": round(stage_d[1], 5),
                          "fwd": round(stage_d[2], 5)},
            "kv_bytes": kv_bytes, "kv_gbs": round(gbs, 1),
            "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<4> + decode_merge_kernel",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for("decode_split_kernel")},
            "route_summary_gbs": round(route_bytes / (stage_d[0] * 1e-3) / 1e9, 1),
        }
        del sd, inp_d
        torch.cuda.empty_cache()
    if not args.no_cpu and inp is not None:
        log(f"timing the oracle on {args.cpu_heads} heads")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
