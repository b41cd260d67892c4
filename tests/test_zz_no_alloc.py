"""sparse_attn_build_worklist_noalloc against sparse_attn_build_worklist.

The no-allocation entry point takes its workspace from the library's static
device scratch instead of an argument; everything else (inputs, outputs,
error bits) is the regular worklist build's, so the two must agree bit for
bit.  Two calls in a row on the same GPU, the second on a smaller input (so
it runs over scratch the first one left behind): a GQA prefill routed by the
library, then a small packed batch with an adversarial J (duplicates, -1
slots, ids out of range and acausal ids)."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_amd as dbs

pytestmark = pytest.mark.gpu


def _compare(prob, cfg, J):
    ref = dbs.build_worklist(prob, cfg, J)
    got = dbs.alloc_worklist(prob, cfg, J.device)
    # poison the outputs so stale values cannot pass
    for t in (got.row_ptr, got.col_idx, got.row_perm, got.bucket_ptr):
        t.fill_(-7)
    dbs.build_worklist_noalloc(prob, cfg, J, out=got)
    torch.cuda.synchronize()
    sz = dbs.sizes(prob, cfg)
    nnz = int(ref.row_ptr[sz.rows].item())
    assert torch.equal(got.row_ptr, ref.row_ptr)
    assert torch.equal(got.col_idx[:nnz], ref.col_idx[:nnz])
    assert torch.equal(got.row_perm[:sz.rows], ref.row_perm[:sz.rows])
    assert torch.equal(got.bucket_ptr, ref.bucket_ptr)
    assert torch.equal(got.err, ref.err)
    return ref


def test_noalloc_worklist_matches_regular_two_calls():
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    # call 1: GQA prefill, 2 x 4096 tokens, shared routing with the sink forced
    prob = dbs.Problem.fixed(2, 8, 2, 128, 4096, "bf16")
    cfg = dbs.RouteConfig(k_b=16, share_gqa=True, force_first=True)
    q = torch.randn(dbs.q_shape(prob), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(dbs.kv_shape(prob), generator=g, device=dev).to(torch.bfloat16)
    J, _ = dbs.route(prob, cfg, q, k)
    ref1 = _compare(prob, cfg, J)
    assert int(ref1.err.item()) == 0
    # call 2: a smaller packed batch (ragged, a one-block sequence) with an
    # adversarial J; the scratch still holds call 1's rows
    lengths = [200, 64, 130]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    prob2 = dbs.Problem.varlen(lengths, 2, 2, 128, cu, "bf16")
    cfg2 = dbs.RouteConfig(k_b=6, window=2)
    rows = dbs.sizes(prob2, cfg2).rows
    rng = np.random.default_rng(3)
    J2 = rng.integers(-3, 6, size=(rows, cfg2.k_b)).astype(np.int32)   # -3..-2: bad, -1: empty, 4-5: too far
    J2[::3, 1] = J2[::3, 0]                                            # duplicates
    ref2 = _compare(prob2, cfg2, torch.from_numpy(J2).to(dev))
    assert int(ref2.err.item()) & dbs.SA_WL_ERR_RANGE
    assert int(ref2.err.item()) & dbs.SA_WL_ERR_ACAUSAL
    # and once more at the first size, after the smaller call
    _compare(prob, cfg, J)


def test_noalloc_refuses_problems_beyond_the_scratch():
    dev = torch.device("cuda:0")
    prob = dbs.Problem.fixed(1, 128, 128, 128, 65536, "bf16")    # 131072 rows x 512 B > 32 MiB
    cfg = dbs.RouteConfig(k_b=16)
    J = torch.zeros((dbs.sizes(prob, cfg).rows, cfg.k_b), dtype=torch.int32, device=dev)
    out = dbs.alloc_worklist(prob, cfg, dev)
    with pytest.raises(ValueError, match="scratch"):
        dbs.build_worklist_noalloc(prob, cfg, J, out=out)
