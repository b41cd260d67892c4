#!/usr/bin/env python3
"""Benchmark: one hot-path step of dynamic block-sparse attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM:

    sparse_attn_route -> sparse_attn_build_worklist -> sparse_attn_fwd

The JSON line's `value` is the step on the packed variable-length setting, the
largest prefill workload that fits one GPU (8 sequences of 2K-64K tokens drawn
from a seed, Hq=32, Hkv=8, d=128, b=64, Eq 7 threshold routing with k_max=64,
bf16, planted relevance): selected-tile FLOPs of the step (4*b*b*d per (query
head, tile) visit of the worklist) divided by the step's time, the step
replayed as one HIP graph, in TFLOP/s.  The attention kernel alone is reported
in `roofline` against the bf16 dense MFMA peak: its mean launch time over every
timed call (events on the stream the library launches on), warm and after a
last-level cache flush (a 512 MB buffer read outside the events).

The other settings are timed the same way and reported under `settings`, each
with its own `roofline`: the 8192-token MHA prefill (B=1, H=16, k_b=16), the
32768-token GQA prefill (B=2, Hq=32, Hkv=8, k_b=32, sink forced) and split-KV
decode (64 x 131072-token caches, Hq=32, Hkv=8, k_b=64) as KV GB/s against the
HBM peak.  The backward pass is timed on the prefill settings, and each
prefill setting (plus the GQA shape at 65536 tokens) is also run densely
(`dense`): the sparse/dense crossover.

The fp64 CPU oracle is timed on a bounded, seeded sample of the headline
setting (`cpu_baseline`): a reported baseline, not a target.

    python bench.py [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-bwd]
    python bench.py --workload NAME     # time one setting only (it becomes the headline)
    python bench.py --no-dense          # skips the dense causal comparison (`dense`)
    python bench.py --crossover         # adds a k_b sweep against the dense call (`crossover`)
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
FLUSH_BYTES = 512 << 20        # twice the 256 MB last-level (MALL) cache


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload`, from committed rocprofv3
    counter runs (profiles/traffic.json, keyed "kernel|workload"), or None when
    that pair was never measured or the kernel's source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(f"{kernel}|{workload}")
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

    def fwd_kernel_name(self):
        """The attention kernel the library picks: by query heads per worklist row."""
        hpr = self.w.group if self.w.share_gqa else 1
        return {1: "prefill_bf16_kernel<1,2>", 2: "prefill_bf16_kernel<2,0>",
                4: "prefill_bf16_pp_kernel<4>"}.get(hpr, f"heads per row {hpr}")

    def worklist_stats(self):
        """Rows per length bucket and the tiles per row (max and mean)."""
        rp = self.wl.row_ptr[:self.sz.rows + 1].cpu()
        lens = (rp[1:] - rp[:-1]).double()
        bp = self.wl.bucket_ptr.cpu().tolist()
        return {"bucket_rows": [bp[i + 1] - bp[i] for i in range(len(bp) - 1)],
                "tiles_per_row_max": int(lens.max().item()),
                "tiles_per_row_mean": round(float(lens.mean().item()), 3)}

    def tile_visits(self):
        """Sum over rows of unique tiles times the query heads each row serves."""
        nnz = int(self.wl.row_ptr[self.sz.rows].item())
        return nnz * (self.w.group if self.w.share_gqa else 1)


def timed(stepper, steps, warmup, flush=None):
    """Eager steps, each call bracketed by events on the current stream.

    With `flush` (a device buffer larger than the 256 MB last-level cache) the
    buffer is read (summed) before every step, outside the events, so no step
    finds the previous step's inputs in cache.  A read leaves no dirty lines,
    whose write-back would otherwise land on the first call after it.  The
    mean over the loop then includes the flushes and only the per-call times
    are meaningful."""
    import torch
    for _ in range(warmup):
        stepper.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        if flush is not None:
            flush.sum()
        stepper.step(evs[i])
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    per_call = [[e[k].elapsed_time(e[k + 1]) for e in evs] for k in range(3)]
    return total / steps, per_call


def spread(xs):
    """Mean, median, p10 and p90 of a list of times (ms)."""
    ys = sorted(xs)
    n = len(ys)
    return {"mean": round(sum(ys) / n, 5), "median": round(ys[n // 2], 5),
            "p10": round(ys[n // 10], 5), "p90": round(ys[(n * 9) // 10], 5)}


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


def pipelined_timed(steppers, steps, warmup):
    """Two independent batches in flight: each stepper (its own J, worklist,
    outputs and workspaces over the same resident inputs) has its step
    captured in a HIP graph, and the graphs are replayed alternately on two
    streams.  Every step still runs route, worklist and fwd over its batch; a
    step's kernels may overlap the other batch's.  Throughput only: one
    step's latency is the serial graph replay."""
    import torch
    graphs = []
    for st in steppers:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            st.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.step()
        graphs.append(g)
    streams = [torch.cuda.Stream() for _ in steppers]
    n = len(steppers)

    def run(k):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for i in range(k):
            with torch.cuda.stream(streams[i % n]):
                graphs[i % n].replay()
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)

    run(warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run(steps)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


PIPELINED_NOTE = ("two batches in flight: the step's HIP graph of each of two steppers (own buffers, same inputs) "
                  "replayed alternately on two streams, so one batch's route and worklist can overlap the other's "
                  "attention; throughput only (a step's latency is ms_per_step)")
# Two batches in flight only pay where a step is short enough that launch gaps
# and the small routing grids leave the chip idle; on longer steps the
# attention kernel already fills it, and the two batches' overlapping
# dispatches would only blur that kernel's per-launch durations in a trace.
PIPELINE_MAX_STEP_MS = 1.0


def _host_info():
    """Threads numpy's BLAS uses, the BLAS library, and the host CPU model."""
    import numpy  # noqa: F401  (loads the BLAS so threadpoolctl can see it)
    cores, blas = len(os.sched_getaffinity(0)), "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            cores = max(p.get("num_threads", 1) for p in pools)
            blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')})"
                             for p in pools)
    except Exception:   # threadpoolctl absent: the affinity mask
        pass
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return int(cores), blas, model


def cpu_baseline(w, inp, n_blocks, seed=0):
    """The fp64 oracle as it stands, on a bounded seeded sample of the prefill input.

    Sample: the shortest sequence of the batch, routed and worklisted whole
    (every routing head and query block), and the masked attention of the rows
    of `n_blocks` of its query blocks (blocks 0, 1, N-1 and seeded random ones;
    0 = all of them) for every routing head.  The rate counts the selected-tile FLOPs of the
    attended rows against the attention time plus their share (by rows) of
    the routing and worklist time."""
    import numpy as np
    from oracle import problem as oprob
    from dynamic_block_sparse_amd import workloads as wk
    cores, blas, model = _host_info()
    s = int(np.argmin(inp.lengths))
    L = inp.lengths[s]
    q, k, v = (x[0] for x in wk.per_sequence_subset(inp, [s]))
    t0 = time.perf_counter()
    J, _ = oprob.route([q], [k], [L], w.block, w.mode, w.qpool, w.share_gqa, w.select, w.k_b,
                       w.k_min, w.tau_rel, w.forced_first, window=w.window, kpool=w.kpool)
    t1 = time.perf_counter()
    wl = oprob.worklist(J, [L], w.block, w.mode, w.route_heads, w.forced_first,
                        w.k_b + max(w.window, 1) + int(w.forced_first), window=w.window)
    t2 = time.perf_counter()
    nq = -(-L // w.block)
    rng = np.random.default_rng(seed)
    n_blocks = nq if n_blocks <= 0 else min(n_blocks, nq)
    pick = {0, 1, nq - 1} if n_blocks >= 3 else set(range(n_blocks))
    while len(pick) < n_blocks:
        pick.add(int(rng.integers(0, nq)))
    table = oprob.row_table([L], w.block, w.mode, w.route_heads)
    rows = [i for i, (_s, _h, r, _n) in enumerate(table) if r in pick]
    blocks = {i: wl["col_idx"][wl["row_ptr"][i]:wl["row_ptr"][i + 1]].tolist() for i in rows}
    t3 = time.perf_counter()
    oprob.attention_rows([q], [k], [v], [L], w.block, w.mode, w.share_gqa, rows, blocks)
    t4 = time.perf_counter()
    hpr = w.group if w.share_gqa else 1
    tiles = sum(len(blocks[i]) for i in rows)
    flops = tiles * hpr * 4 * w.block * w.block * w.head_dim
    share = len(rows) / len(table)
    secs = (t4 - t3) + share * (t2 - t0)
    return dict(value=round(flops / secs / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=(f"sequence {s} of {w.name} ({L} tokens, the batch's shortest): routed and "
                        f"worklisted whole ({len(table)} rows: route {t1 - t0:.2f}s, worklist {t2 - t1:.2f}s), "
                        f"masked attention of the {len(rows)} rows of {len(pick)} query blocks x "
                        f"{w.route_heads} routing heads x {hpr} query heads ({t4 - t3:.2f}s, "
                        f"{flops / 1e9:.2f} GFLOP of selected tiles); rate = those FLOPs / (attention "
                        f"time + {share:.3f} of the route and worklist time)"),
                seconds=round(t4 - t0, 3), cpu_model=model, blas=blas)


def prefill_flops(st, w):
    """Physical selected-tile FLOPs (4*b*b*d per visit) and the causal-effective
    count in which each diagonal tile holds only its b*(b+1)/2 unmasked pairs."""
    visits = st.tile_visits()
    per = 4 * w.block * w.block * w.head_dim
    diag = st.sz.rows * (w.group if w.share_gqa else 1)
    eff = (visits - diag) * per + diag * 4 * (w.block * (w.block + 1) // 2) * w.head_dim
    return visits, visits * per, eff


def measure_prefill(args, dbs, w, inp, flush):
    import torch
    st = Stepper(dbs, w, inp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.step()
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    log(f"timing {w.name}: warm eager steps")
    eager_ms, warm = timed(st, args.steps, args.warmup)
    log(f"timing {w.name}: steps with the last-level cache flushed before each")
    _, cold = timed(st, args.steps, 2, flush)
    ms = eager_ms if args.no_graph else graph_timed(st, args.steps, args.warmup)
    visits, flops, eff = prefill_flops(st, w)
    # the attention kernel's mean launch time over every timed call, warm and
    # after a flush (what a kernel trace of the same run averages)
    fwd_calls = warm[2] + cold[2]
    fwd_ms = sum(fwd_calls) / len(fwd_calls)
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    kernel = st.fwd_kernel_name()
    rec = {
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "ms_per_step": round(ms, 5),
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seqlen": w.seqlen or f"varlen {w.varlen_min}..{w.varlen_max}",
                   "head_dim": w.head_dim, "block": w.block, "k_b": w.k_b, "select": w.select,
                   "qpool": w.qpool, "tile_visits": visits, "selected_tile_flops": flops,
                   "causal_effective_flops": eff},
        "roofline": {"bound": "mfma", "kernel": kernel,
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(kernel, w.name),
                     "algorithmic_flops_per_launch": flops,
                     "mean_launch_ms": round(fwd_ms, 5),
                     "time": (f"mean of the {len(fwd_calls)} timed sparse_attn_fwd calls (warm, and after a "
                              f"last-level cache flush), events on the launch stream; one attention launch "
                              f"per call" + (" plus the 2 us block-offset kernel of a packed batch"
                                             if w.varlen else ""))},
        "step": ("eager steps (--no-graph)" if args.no_graph else
                 "HIP graph replay of route + worklist + fwd") +
                "; eager_ms_per_step: the step launched call by call",
        "eager_ms_per_step": round(eager_ms, 5),
        "first_step_ms": round(first_ms, 3),
        "stages_ms": {"warm": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), warm)},
                      "cache_flushed": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), cold)}},
        "effective_tflops": round(eff / (fwd_ms * 1e-3) / 1e12, 3),
        "route_worklist_share_of_step": round(1 - fwd_ms / ms, 4) if not args.no_graph else None,
        "worklist_err": int(st.wl.err.item()),
    }
    if w.varlen or w.select == "threshold":
        rec["worklist"] = st.worklist_stats()
    if not args.no_graph and ms < PIPELINE_MAX_STEP_MS:
        log(f"timing {w.name}: two batches in flight on two streams")
        st2 = Stepper(dbs, w, inp)
        msp = pipelined_timed([st, st2], args.steps, args.warmup)
        del st2
        rec["pipelined"] = {"streams": 2, "ms_per_step": round(msp, 5),
                            "value": round(flops / (msp * 1e-3) / 1e12, 3), "note": PIPELINED_NOTE}
    if not args.no_bwd:
        log(f"timing the backward pass on {w.name}")
        rec["backward"] = measure_bwd(args, dbs, st, visits)
    del st
    return rec


def measure_bwd(args, dbs, st, visits):
    """sparse_attn_bwd over the step's worklist, output and lse with a seeded
    dO: each call bracketed by events (warm), median over the calls.  FLOPs
    are the five products per selected tile visit (S, dP, dQ, dK, dV: 10 b^2 d);
    the two kernels form S and dP in both, so they execute 14 b^2 d."""
    import torch
    w, inp = st.w, st.inp
    g = torch.Generator(device=inp.q.device).manual_seed(7)
    dout = torch.randn(inp.q.shape, generator=g, device=inp.q.device).to(inp.q.dtype)
    dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)
    ws = torch.empty(max(dbs.workspace_size(st.prob, st.cfg, 3), 1), dtype=torch.uint8, device=inp.q.device)
    call = lambda: dbs.bwd(st.prob, st.cfg, st.wl, inp.q, inp.k, inp.v, st.o, st.lse, dout, dq=dq, dk=dk,
                           dv=dv, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(max(args.steps // 10, 5)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    med = spread(ts)["median"]
    flops = visits * 10 * w.block * w.block * w.head_dim
    tf = flops / (med * 1e-3) / 1e12
    del dout, dq, dk, dv, ws
    return {"median_ms": round(med, 4), "algorithmic_flops": flops, "tflops": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "kernels": ("bwd_dq_rows_bf16_kernel" if w.share_gqa and w.group in (2, 4, 8) else "bwd_dq_bf16_kernel")
                       + " + bwd_dkdv_bf16_kernel",
            "time": "median call, warm (events on the current stream)"}


def measure_dense(args, dbs, w, inp, flush, sparse_rec):
    """The same causal attention done densely, for the sparse/dense crossover
    ([P2] §3.1 dense fallback): sparse_attn_fwd_dense (this library's kernels,
    every causal tile of every row, same layout, dtype and masks) and, for
    fixed-length inputs, torch's flash-attention SDPA (causal, bf16, forced to
    its flash backend; GQA through enable_gqa).  Each call timed after the
    cache flush; medians in ms.  Crossover: the sparse step (route + worklist +
    fwd) costs t_r + t_w + f * (dense time) * c when it keeps a fraction f of
    the causal tiles, c being its measured per-tile cost relative to the
    dense walk; it beats the dense call while f < (t_dense - t_r - t_w) /
    (c t_dense)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    prob, cfg = dbs.problem_for(w, inp), dbs.config_for(w)
    hpr = w.group if w.share_gqa else 1
    nblocks = [-(-L // w.block) for L in inp.lengths]
    dense_visits = sum(nb * (nb + 1) // 2 for nb in nblocks) * w.route_heads * hpr
    o = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[:-1], dtype=torch.float32, device=inp.q.device)
    ws = torch.empty(max(dbs.workspace_size(prob, cfg, 2), 1), dtype=torch.uint8, device=inp.q.device)
    call = lambda: dbs.fwd_dense(prob, cfg, inp.q, inp.k, inp.v, o=o, lse=lse, workspace=ws)
    flash = None
    if not w.varlen:
        gqa = w.heads_q != w.heads_kv
        flash = lambda: torch.nn.functional.scaled_dot_product_attention(
            inp.q, inp.k, inp.v, is_causal=True, enable_gqa=gqa)
    reps = max(min(args.steps // 5, 10), 3)

    def time_calls(fn):
        out = []
        for i in range(reps + 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 1:
                out.append(e0.elapsed_time(e1))
        return spread(out)["median"]

    ours_ms = time_calls(call)
    flash_ms, flash_err = None, None
    if flash is not None:
        try:
            with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
                flash_ms = time_calls(flash)
        except RuntimeError as e:   # no flash kernel for this shape on this build
            flash_err = str(e).splitlines()[0][:160]
    causal = 4 * w.head_dim * w.heads_q * sum(L * (L + 1) // 2 for L in inp.lengths)
    tile_flops = 4 * w.block * w.block * w.head_dim
    st = sparse_rec["stages_ms"]["cache_flushed"]
    t_r, t_w, t_f = st["route"]["median"], st["worklist"]["median"], st["fwd"]["median"]
    sparse_visits = sparse_rec["config"]["tile_visits"]
    frac = sparse_visits / dense_visits
    cost = (t_f / sparse_visits) / (ours_ms / dense_visits)
    f_star = (ours_ms - t_r - t_w) / (cost * ours_ms)
    del o, lse, ws
    return {"dense_fwd_ms": ours_ms, "dense_tile_visits": dense_visits,
            "dense_tflops_tiles": round(dense_visits * tile_flops / (ours_ms * 1e-3) / 1e12, 1),
            "dense_frac_of_peak": round(dense_visits * tile_flops / (ours_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "torch_flash_sdpa_ms": flash_ms,
            "torch_flash_sdpa_tflops_causal": (round(causal / (flash_ms * 1e-3) / 1e12, 1)
                                               if flash_ms else None),
            "torch_flash_note": flash_err or ("not run: packed varlen input" if flash is None else None),
            "sparse_step_ms": round(t_r + t_w + t_f, 5),
            "sparse_tile_fraction": round(frac, 4),
            "sparse_per_tile_cost_vs_dense": round(cost, 3),
            "sparse_speedup_vs_dense": round(ours_ms / (t_r + t_w + t_f), 2),
            "sparse_speedup_vs_flash": round(flash_ms / (t_r + t_w + t_f), 2) if flash_ms else None,
            "fallback_tile_fraction": round(min(f_star, 1.0), 4),
            "fallback_tile_fraction_raw": round(f_star, 4),
            "note": "times: median calls after a cache flush; fallback_tile_fraction: the sparse step "
                    "(route + worklist + fwd) beats the dense call while it keeps fewer than this "
                    "fraction of the causal tiles (raw > 1: a listed tile costs less than a tile of "
                    "the dense walk, so the sparse step wins at any fraction)"}


def measure_crossover(args, dbs, w, inp, flush):
    """Empirical sparse/dense crossover ([P2] §3.1 dense fallback): the sparse
    step (route + worklist + fwd, each after a cache flush, medians) at a range
    of budgets k_b on the same inputs, beside the dense call; the crossover is
    where the step time meets the dense time, interpolated in the tile
    fraction between the two budgets that bracket it."""
    import torch
    prob, cfg = dbs.problem_for(w, inp), dbs.config_for(w)
    nblocks = [-(-L // w.block) for L in inp.lengths]
    hpr = w.group if w.share_gqa else 1
    dense_visits = sum(nb * (nb + 1) // 2 for nb in nblocks) * w.route_heads * hpr
    o = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[:-1], dtype=torch.float32, device=inp.q.device)
    ws = torch.empty(max(dbs.workspace_size(prob, cfg, 2), 1), dtype=torch.uint8, device=inp.q.device)
    times = []
    for i in range(6):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dbs.fwd_dense(prob, cfg, inp.q, inp.k, inp.v, o=o, lse=lse, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        if i:
            times.append(e0.elapsed_time(e1))
    dense_ms = spread(times)["median"]
    del o, lse, ws
    max_kb = 128 - max(w.window, 1) - (1 if w.forced_first else 0)
    budgets = sorted({kb for kb in (4, 8, 16, 32, 48, 64, 80, 96, 112, max_kb) if kb <= max_kb})
    pts = []
    for kb in budgets:
        wk_ = w.replace(name=f"{w.name}_kb{kb}", k_b=kb)
        st = Stepper(dbs, wk_, inp)
        _, cold = timed(st, 10, 2, flush)
        r, wl_, f = (spread(x)["median"] for x in cold)
        frac = st.tile_visits() / dense_visits
        pts.append({"k_b": kb, "tile_fraction": round(frac, 4), "step_ms": round(r + wl_ + f, 5),
                    "route_ms": round(r, 5), "worklist_ms": round(wl_, 5), "fwd_ms": round(f, 5),
                    "step_vs_dense": round((r + wl_ + f) / dense_ms, 3)})
        del st
        torch.cuda.empty_cache()
    cross = None
    for a, b in zip(pts, pts[1:]):
        if a["step_ms"] <= dense_ms < b["step_ms"]:
            t = (dense_ms - a["step_ms"]) / (b["step_ms"] - a["step_ms"])
            cross = round(a["tile_fraction"] + t * (b["tile_fraction"] - a["tile_fraction"]), 4)
    return {"workload": w.name, "dense_fwd_ms": dense_ms, "points": pts,
            "crossover_tile_fraction": cross,
            "note": "crossover_tile_fraction: null when every budget's step beats the dense call "
                    "(the widest row holds at most 128 ids)"}


def measure_decode(args, dbs, wd, dev, flush):
    import torch
    log(f"generating {wd.name}")
    inp_d = wk_make(wd, dev)
    sd = Stepper(dbs, wd, inp_d, summaries_in=True, num_splits=args.decode_splits)
    steps = max(args.steps // 2, 10)
    log(f"timing {wd.name}: warm eager steps")
    eager_msd, warm = timed(sd, steps, args.warmup)
    log(f"timing {wd.name}: steps with the last-level cache flushed before each")
    _, cold = timed(sd, steps, 2, flush)
    msd = eager_msd if args.no_graph else graph_timed(sd, steps, args.warmup)
    nnz = int(sd.wl.row_ptr[sd.sz.rows].item())
    kv_bytes = nnz * wd.block * wd.head_dim * 2 * 2
    qo_bytes = 2 * wd.batch * wd.heads_q * wd.head_dim * 2
    fwd_calls = warm[2] + cold[2]
    fwd_ms = sum(fwd_calls) / len(fwd_calls)
    gbs = (kv_bytes + qo_bytes) / (fwd_ms * 1e-3) / 1e9
    route_bytes = wd.batch * wd.heads_kv * (wd.seqlen // wd.block) * wd.head_dim * 4
    rec = {
        "workload": wd.name, "reading": f"k_b = {wd.k_b} tiles per row, the forced last block counted in",
        "ms_per_step": round(msd, 5), "eager_ms_per_step": round(eager_msd, 5),
        "stages_ms": {"warm": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), warm)},
                      "cache_flushed": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), cold)}},
        "value": round(gbs, 1), "unit": "GB/s",
        "kv_bytes": kv_bytes, "kv_gbs": round(gbs, 1),
        "roofline": {"bound": "hbm", "kernel": "decode_fused_kernel<4>",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for("decode_fused_kernel<4>", wd.name),
                     "algorithmic_bytes_per_launch": kv_bytes + qo_bytes,
                     "mean_launch_ms": round(fwd_ms, 5),
                     "time": f"mean of the {len(fwd_calls)} timed sparse_attn_fwd calls (warm, and after a "
                             f"last-level cache flush), events on the launch stream"},
        "route_summary_gbs": round(route_bytes / (spread(cold[0])["median"] * 1e-3) / 1e9, 1),
    }
    if not args.no_graph and msd < PIPELINE_MAX_STEP_MS:
        log(f"timing {wd.name}: two batches in flight on two streams")
        sd2 = Stepper(dbs, wd, inp_d, summaries_in=True, num_splits=args.decode_splits)
        msp = pipelined_timed([sd, sd2], steps, args.warmup)
        del sd2
        rec["pipelined"] = {"streams": 2, "ms_per_step": round(msp, 5),
                            "kv_gbs_per_step_time": round((kv_bytes + qo_bytes) / (msp * 1e-3) / 1e9, 1),
                            "note": PIPELINED_NOTE}
    del sd
    # the other reading of the setting: k_b blocks routed plus the forced last
    # block (k_b + 1 tiles per row), on the same cache
    w1 = wd.replace(name=wd.name + "_plus_forced", k_b=wd.k_b + 1)
    s1 = Stepper(dbs, w1, inp_d, summaries_in=True, num_splits=args.decode_splits)
    log(f"timing {w1.name}: warm and cache-flushed eager steps")
    eager1, warm1 = timed(s1, steps, args.warmup)
    _, cold1 = timed(s1, steps, 2, flush)
    nnz1 = int(s1.wl.row_ptr[s1.sz.rows].item())
    kv1 = nnz1 * wd.block * wd.head_dim * 2 * 2
    calls1 = warm1[2] + cold1[2]
    fwd1 = sum(calls1) / len(calls1)
    gbs1 = (kv1 + qo_bytes) / (fwd1 * 1e-3) / 1e9
    rec["plus_forced"] = {
        "workload": w1.name, "reading": f"{wd.k_b} routed blocks plus the forced last block "
                                        f"({wd.k_b + 1} tiles per row)",
        "eager_ms_per_step": round(eager1, 5),
        "stages_ms": {"warm": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), warm1)},
                      "cache_flushed": {k: spread(v) for k, v in zip(("route", "worklist", "fwd"), cold1)}},
        "kv_bytes": kv1, "kv_gbs": round(gbs1, 1), "frac": round(gbs1 / PEAK_HBM_GBS, 4),
        "mean_launch_ms": round(fwd1, 5)}
    del s1, inp_d
    torch.cuda.empty_cache()
    rec["append_kv"] = measure_append(args, dbs, wd, dev)
    return rec


def measure_append(args, dbs, wd, dev):
    """sparse_attn_append_kv at the decode shape (S sequences x Hkv heads, d):
    one token per sequence (what a decode step appends) and a 64-token chunk,
    into a cache with room past its 100 valid rows (the cost depends only on
    the appended rows and the blocks they land in, not on the cache length).
    Timed as a HIP graph of R back-to-back calls, so host-side argument
    marshalling is not counted; per call = graph time / R."""
    import torch
    S, hkv, d, cap, len0 = wd.batch, wd.heads_kv, wd.head_dim, 256, 100
    g = torch.Generator(device=dev).manual_seed(5)
    kc = torch.randn((S, hkv, cap, d), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((S, hkv, cap, d), generator=g, device=dev).to(torch.bfloat16)
    prob = dbs.Problem.decode(S, wd.heads_q, hkv, d, len0, "bf16", kv_capacity=cap)
    summ = torch.randn(dbs.summaries_shape(prob), generator=g, device=dev)
    out = {}
    for n in (1, 64):
        kn = torch.randn((S, hkv, n, d), generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn((S, hkv, n, d), generator=g, device=dev).to(torch.bfloat16)
        R = 20
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(max(args.warmup, 1)):
                dbs.append_kv(prob, kn, vn, kc, vc, summ)
        torch.cuda.current_stream(dev).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(R):
                dbs.append_kv(prob, kn, vn, kc, vc, summ)
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(args.steps // 5, 10)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / R)
        del graph
        med = spread(ts)["median"]
        touched = (len0 + n - 1) // 64 - len0 // 64 + 1
        nbytes = S * hkv * (4 * n * d * 2 + 2 * touched * d * 4)   # K/V read + written, summaries read + written
        out[f"{n}_tokens"] = {"median_us": round(med * 1e3, 2), "bytes": nbytes,
                              "gbs": round(nbytes / (med * 1e-3) / 1e9, 1)}
    del kc, vc, summ
    torch.cuda.empty_cache()
    return out


def wk_make(w, dev):
    from dynamic_block_sparse_amd import workloads as wk
    return wk.make_inputs(w, dev)


def main():
    from dynamic_block_sparse_amd import workloads as wk
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode setting")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense comparison (sparse_attn_fwd_dense and torch flash SDPA on "
                         "each prefill setting, and the 65536-token crossover point)")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--crossover", action="store_true",
                    help="also sweep k_b on the MHA and GQA settings against the dense call (empirical "
                         "sparse/dense crossover)")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="query blocks of the oracle's sample (every routing head of each); "
                         "0: every query block of the sampled sequence")
    ap.add_argument("--decode-splits", type=int, default=0)
    ap.add_argument("--workload", choices=[w.name for w in wk.ALL if w.dtype == "bf16"], default=None,
                    help="time this setting only; it becomes the JSON line's headline")
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
    # 512 MB read between timed steps: twice the last-level cache
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    # the headline: the largest prefill setting that fits one GPU, unless one
    # setting is asked for by name
    if args.workload:
        head = wk.BY_NAME[args.workload]
        others = []
    else:
        head = wk.VARLEN
        others = [wk.PREFILL_MHA, wk.PREFILL_GQA] + ([] if args.no_decode else [wk.DECODE])
    out = {"metric": METRIC}
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16"}
    cpu_inp = None
    if head.mode == "decode":
        rec = measure_decode(args, dbs, head, dev, flush)
        out.update({"value": rec.pop("value"), "unit": rec.pop("unit"), **common,
                    "ms_per_step": rec.pop("ms_per_step"),
                    "data": "synthetic (seeded N(0,1) Q/K/V with planted hot blocks; no dataset)",
                    "config": {"workload": head.name}})
        out.update(rec)
    else:
        log(f"generating {head.name}")
        inp = wk.make_inputs(head, dev)
        rec = measure_prefill(args, dbs, head, inp, flush)
        out.update({"value": rec.pop("value"), "unit": "TFLOP/s", **common,
                    "ms_per_step": rec.pop("ms_per_step"),
                    "data": "synthetic (seeded N(0,1) Q/K/V with planted relevance; no dataset)"})
        out.update(rec)
        if not args.no_dense:
            log(f"timing dense causal attention on {head.name}")
            out["dense"] = measure_dense(args, dbs, head, inp, flush, out)
        if not args.no_cpu:
            cpu_inp = inp
        else:
            del inp
        torch.cuda.empty_cache()
    settings = {}
    if not args.workload and not args.no_dense:
        # a longer point for the crossover: the GQA setting at 65536 tokens, one sequence
        others.insert(2, wk.PREFILL_GQA.replace(name="prefill_gqa_b1_hq32_hkv8_n65536_d128_kb32", batch=1,
                                                seqlen=65536))
    for w in others:
        if w.mode == "decode":
            settings[w.name] = measure_decode(args, dbs, w, dev, flush)
        else:
            log(f"generating {w.name}")
            inp_w = wk.make_inputs(w, dev)
            settings[w.name] = measure_prefill(args, dbs, w, inp_w, flush)
            if not args.no_dense:
                log(f"timing dense causal attention on {w.name}")
                settings[w.name]["dense"] = measure_dense(args, dbs, w, inp_w, flush, settings[w.name])
            del inp_w
        torch.cuda.empty_cache()
    if settings:
        out["settings"] = settings
    if args.crossover:
        out["crossover"] = []
        for w in (wk.PREFILL_MHA, wk.PREFILL_GQA):
            log(f"k_b sweep against the dense call on {w.name}")
            inp_w = wk.make_inputs(w, dev)
            out["crossover"].append(measure_crossover(args, dbs, w, inp_w, flush))
            del inp_w
            torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    if cpu_inp is not None:
        log(f"timing the oracle on a sample of {head.name}")
        out["cpu_baseline"] = cpu_baseline(head, cpu_inp, args.cpu_blocks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
