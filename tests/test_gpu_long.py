"""GPU parity for sequences longer than 8192 blocks (524,288 tokens): routing
then selects each row from its scores in memory (prefill: the route
workspace; decode: LDS) instead of registers.  Router sets on every row,
the worklist bit for bit, and the output on sampled rows, against the oracle.
"""
import pytest
import torch

import dynamic_block_sparse_amd as dbs
from dynamic_block_sparse_amd import workloads as wk

from parity import LSE_TOL, TOL, check_output, check_router, check_worklist, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dbs.load_library()
    return torch.device("cuda:0")


def _check(w, inp, run, rows):
    r = check_router(w, inp, run)
    print(f"[{w.name}] router rows checked {r['checked']} tie-band rows {r['tie_rows']}", flush=True)
    assert not r["bad"], f"router mismatches outside the tie band at rows {r['bad'][:10]}"
    check_worklist(w, inp, run)
    o = check_output(w, inp, run, rows)
    mx, mean = TOL[w.dtype]
    print(f"[{w.name}] output max-abs {o['max_abs']:.3e} mean-abs {o['mean_abs']:.3e} "
          f"lse max-abs {o['lse_max_abs']:.3e} over {o['n']} values", flush=True)
    assert o["max_abs"] <= mx and o["mean_abs"] <= mean and o["lse_max_abs"] <= LSE_TOL[w.dtype]


LONG_PREFILL = [
    # 8300 key blocks, ragged last block (the oracle routes it in ~35 s)
    wk.PREFILL_MHA.replace(name="long_mha_h1_n531183_kb16", heads_q=1, heads_kv=1, seqlen=8300 * 64 - 17),
]


@pytest.mark.parametrize("w", LONG_PREFILL, ids=lambda w: w.name)
def test_long_prefill(dev, w):
    print(f"case {w.name}", flush=True)
    inp = wk.make_inputs(w, dev)
    run = run_gpu(w, inp)
    _check(w, inp, run, sample_rows(w, inp, per_seq_head=6, seed=11))


LONG_DECODE = [
    # two caches of 540,000 tokens (8438 blocks, 8437 candidates a row): top-k
    # and the Eq 7 threshold count
    wk.DECODE.replace(name="long_decode_s2_L540000", batch=2, heads_q=8, heads_kv=2, seqlen=540000, k_b=16),
    wk.DECODE.replace(name="long_decode_s2_L540000_thresh", batch=2, heads_q=8, heads_kv=2, seqlen=540000,
                      k_b=24, select="threshold", k_min=4, tau_rel=2.0),
    # 17188 blocks: the score array (69 KB) needs more LDS than the default allowance
    wk.DECODE.replace(name="long_decode_s1_L1100000", batch=1, heads_q=8, heads_kv=2, seqlen=1100000, k_b=16),
]


@pytest.mark.parametrize("w", LONG_DECODE, ids=lambda w: w.name)
def test_long_decode(dev, w):
    print(f"case {w.name}", flush=True)
    inp = wk.make_inputs(w, dev)
    run = run_gpu(w, inp)
    _check(w, inp, run, list(range(run.J.shape[0])))
