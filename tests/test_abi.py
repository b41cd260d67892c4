"""CPU checks of the C-ABI library: it loads, exports every declared symbol,
computes host-side sizes, and rejects bad arguments before touching a GPU.

No call here reaches a kernel launch: every argument set either fails host
validation or goes to the pure-host size queries.
"""
import ctypes
import dataclasses
import os
import re

import pytest

import dynamic_block_sparse_amd as dbs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(sparse_attn_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dbs.LIB_PATH):
        pytest.fail("libsparse_attn.so is not built (python -m dynamic_block_sparse_amd.build)")
    return dbs.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(dbs.EXPORTED) <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name


def _prob(**kw):
    base = dict(batch=1, heads_q=16, heads_kv=16, head_dim=128, seqlen=8192, dtype="bf16", mode="prefill")
    base.update(kw)
    return dbs.Problem(**base)


def test_sizes_prefill_mha(lib):
    s = dbs.sizes(_prob(), dbs.RouteConfig(k_b=16))
    assert s.rows == 16 * 128
    assert s.width_max == 17
    assert s.nnz_cap == 16 * 128 * 17
    assert s.n_buckets == 4          # 4, 8, 16, 32
    assert s.kv_blocks == 128


def test_sizes_gqa_shared_and_decode(lib):
    s = dbs.sizes(_prob(batch=2, heads_q=32, heads_kv=8, seqlen=32768),
                  dbs.RouteConfig(k_b=32, share_gqa=True, force_first=True))
    assert s.rows == 2 * 8 * 512 and s.width_max == 34 and s.n_buckets == 5
    d = dbs.sizes(dbs.Problem.decode(64, 32, 8, 128, 131072), dbs.RouteConfig(k_b=64, share_gqa=True))
    assert d.rows == 64 * 8 and d.width_max == 65 and d.n_buckets == 6 and d.kv_blocks == 64 * 2048


def test_workspace_sizes(lib):
    p, c = _prob(), dbs.RouteConfig(k_b=16)
    # route: one fp32 score per (row, candidate slot), rows x max_blocks
    sz = dbs.sizes(p, c)
    assert dbs.workspace_size(p, c, 0) >= sz.rows * 128 * 4
    assert dbs.workspace_size(p, c, 1) >= 2048 * 128 * 4
    dp = dbs.Problem.decode(64, 32, 8, 128, 131072)
    dc = dbs.RouteConfig(k_b=64, share_gqa=True)
    # decode: up to 8 splits merge in LDS (no workspace); more keep fp32 partial
    # states (u[128], m, l) per (row, split, head) in the workspace
    assert dbs.workspace_size(dp, dc, 2, 8) == 0
    assert dbs.workspace_size(dp, dc, 2, 0) == 0
    assert dbs.workspace_size(dp, dc, 2, 16) >= 512 * 16 * 4 * 130 * 4


@pytest.mark.parametrize("bad,status", [
    (dict(heads_q=12, heads_kv=8), dbs.SA_ERR_INVALID_ARG),     # Hq % Hkv
    (dict(head_dim=96), dbs.SA_ERR_UNSUPPORTED),
    (dict(block=32), dbs.SA_ERR_UNSUPPORTED),
    (dict(seqlen=0), dbs.SA_ERR_INVALID_ARG),                   # fixed length needs n >= 1
    (dict(batch=0), dbs.SA_ERR_INVALID_ARG),
])
def test_invalid_problem_rejected(lib, bad, status):
    with pytest.raises(dbs.SAError) as e:
        dbs.sizes(_prob(**bad), dbs.RouteConfig(k_b=16))
    assert e.value.status == status


@pytest.mark.parametrize("cfg", [
    dbs.RouteConfig(k_b=0),
    dbs.RouteConfig(k_b=1, force_first=True),        # two forced blocks do not fit
    dbs.RouteConfig(k_b=128),                        # row wider than 128 slots
    dbs.RouteConfig(k_b=8, select="threshold", tau_rel=-1.0),
])
def test_invalid_config_rejected(lib, cfg):
    with pytest.raises(dbs.SAError) as e:
        dbs.sizes(_prob(), cfg)
    assert e.value.status == dbs.SA_ERR_INVALID_ARG


def test_calls_validate_before_any_launch(lib):
    """Null pointers / small capacities fail with a status; nothing is enqueued."""
    p, c = _prob().to_c(), dbs.RouteConfig(k_b=16).to_c()
    P, C = ctypes.byref(p), ctypes.byref(c)
    assert lib.sparse_attn_route(P, C, None, None, None, 0, None, None, 0, None) == dbs.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_build_worklist(P, C, 8, 8, 8, 10, 8, 8, 8, 8, 10**9, None) == dbs.SA_ERR_WORKSPACE
    assert lib.sparse_attn_build_worklist(P, C, 8, 8, 8, 10**9, 8, 8, 8, 8, 10, None) == dbs.SA_ERR_WORKSPACE
    assert lib.sparse_attn_fwd(P, C, None, 8, 8, 8, 8, 8, 8, None, 0, None, 0, None) == dbs.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_fwd(P, C, 8, 8, 8, 8, 8, 8, 8, None, -1, None, 0, None) == dbs.SA_ERR_INVALID_ARG
    # bf16 with head_dim 64 is not implemented by the attention kernel
    p64 = _prob(head_dim=64).to_c()
    assert lib.sparse_attn_fwd(ctypes.byref(p64), C, 8, 8, 8, 8, 8, 8, 8, None, 0, None, 0, None) \
        == dbs.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_status_string(dbs.SA_ERR_HIP) == b"HIP launch failed"


def test_decode_capacity_sizes_and_prefill_rejects_capacity(lib):
    d = dbs.sizes(dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500), dbs.RouteConfig(k_b=8, share_gqa=True))
    assert d.kv_blocks == 4 * 24            # summary slots follow the capacity: ceil(1500 / 64)
    assert dbs.summaries_shape(dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500)) == (4, 2, 24, 128)
    for bad in (dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=999),   # capacity below the length
                dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=-1),
                dataclasses.replace(_prob(), kv_capacity=8000)):            # prefill: below the length too
        with pytest.raises(dbs.SAError) as e:
            dbs.sizes(bad, dbs.RouteConfig(k_b=8, share_gqa=True))
        assert e.value.status == dbs.SA_ERR_INVALID_ARG


def test_append_kv_validates_before_any_launch(lib):
    """Every bad argument returns a status on the host; n_new = 0 enqueues nothing."""
    def call(prob, n, ptr=8, kpool=dbs.SA_POOL_MEAN):
        p = prob.to_c()
        return lib.sparse_attn_append_kv(ctypes.byref(p), n, ptr, ptr, ptr, ptr, ptr, kpool, None)
    ok = dbs.Problem.decode(2, 4, 2, 128, 100, kv_capacity=200)
    assert call(ok, 0) == dbs.SA_OK                                            # nothing to do
    assert call(ok, 101) == dbs.SA_ERR_INVALID_ARG                             # past the capacity
    assert call(ok, -1) == dbs.SA_ERR_INVALID_ARG
    assert call(ok, 5, ptr=None) == dbs.SA_ERR_INVALID_ARG                     # null pointers
    assert call(dbs.Problem.decode(2, 4, 2, 128, 100), 1) == dbs.SA_ERR_INVALID_ARG   # no capacity set
    assert call(dataclasses.replace(_prob(), kv_capacity=9000), 1) == dbs.SA_ERR_INVALID_ARG  # prefill
    assert call(dataclasses.replace(ok, q_start=64), 1) == dbs.SA_ERR_INVALID_ARG            # decode: no chunk
    assert call(dbs.Problem.decode(2, 4, 2, 96, 100, kv_capacity=200), 1) == dbs.SA_ERR_UNSUPPORTED
    assert call(dbs.Problem.decode(2, 4, 3, 128, 100, kv_capacity=200), 1) == dbs.SA_ERR_INVALID_ARG
    assert call(ok, 1, kpool=2) == dbs.SA_ERR_INVALID_ARG                      # unknown key pooling


def test_route_cfg_kpool_validated(lib):
    assert dbs.sizes(_prob(), dbs.RouteConfig(k_b=8, kpool="max")).rows > 0
    c = dbs.RouteConfig(k_b=8).to_c()
    c.kpool = 5
    p = _prob().to_c()
    assert lib.sparse_attn_workspace_size(ctypes.byref(p), ctypes.byref(c), 0, 0) == 0


def test_window_sizes_and_limits(lib):
    s = dbs.sizes(_prob(), dbs.RouteConfig(k_b=16, window=4, force_first=True))
    assert s.width_max == 16 + 4 + 1
    for bad in (dbs.RouteConfig(k_b=16, window=-1),
                dbs.RouteConfig(k_b=4, window=5),                  # k_b must cover the forced ids
                dbs.RouteConfig(k_b=100, window=30)):              # row wider than 128 slots
        with pytest.raises(dbs.SAError) as e:
            dbs.sizes(_prob(), bad)
        assert e.value.status == dbs.SA_ERR_INVALID_ARG


def test_block_table_validation(lib):
    import torch
    table = torch.zeros((4, 24), dtype=torch.int32)      # host memory: only the pointer is checked here
    ok = dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500, block_table=table, pool_blocks=96)
    assert dbs.sizes(ok, dbs.RouteConfig(k_b=8, share_gqa=True)).kv_blocks == 4 * 24
    short = dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500, block_table=table[:, :20].contiguous(),
                               pool_blocks=96)                               # stride < ceil(1500 / 64)
    no_pool = dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500, block_table=table, pool_blocks=0)
    prefill = dataclasses.replace(_prob(), block_table=table, pool_blocks=96)
    for bad in (short, no_pool, prefill):
        with pytest.raises(dbs.SAError) as e:
            dbs.sizes(bad, dbs.RouteConfig(k_b=8, share_gqa=True))
        assert e.value.status == dbs.SA_ERR_INVALID_ARG


def test_chunked_prefill_sizes_and_limits(lib):
    cfg = dbs.RouteConfig(k_b=16)
    p = dbs.Problem.fixed(2, 4, 4, 128, 1500, "bf16", kv_capacity=2048, q_start=960)
    s = dbs.sizes(p, cfg)
    assert s.rows == 2 * 4 * (24 - 15)        # query blocks 15 .. 23 of every (sequence, head)
    assert s.kv_blocks == 2 * 32              # summary slots follow the capacity
    assert dbs.summaries_shape(p) == (2, 4, 32, 128)
    for bad in (dataclasses.replace(p, q_start=100),     # not a whole number of blocks
                dataclasses.replace(p, q_start=1536),    # no query left
                dataclasses.replace(p, q_start=-64),
                dataclasses.replace(dbs.Problem.decode(2, 4, 4, 128, 1500), q_start=64)):
        with pytest.raises(dbs.SAError) as e:
            dbs.sizes(bad, cfg)
        assert e.value.status == dbs.SA_ERR_INVALID_ARG



def test_bwd_validates_before_any_launch(lib):
    """sparse_attn_bwd returns its status on the host for a decode problem, an
    unsupported head_dim / dtype pair, null pointers and a short workspace."""
    cfg = dbs.RouteConfig(k_b=8).to_c()

    def call(prob, ws_bytes=1 << 40, ptr=8):
        p = prob.to_c()
        # row_ptr, col_idx, q, k, v, o, lse, dout, dq, dk, dv, ws
        return lib.sparse_attn_bwd(ctypes.byref(p), ctypes.byref(cfg), *([ptr] * 12), ws_bytes, None)
    ok = _prob()
    need = lib.sparse_attn_workspace_size(ctypes.byref(ok.to_c()), ctypes.byref(cfg), 3, 0)
    # D per query (16 heads x 8192 tokens), dK and dV accumulators, two counters per key block and head
    assert need >= 16 * 8192 * 4 + 2 * 16 * 8192 * 128 * 4 + 2 * 128 * 16 * 4
    assert lib.sparse_attn_workspace_size(ctypes.byref(ok.to_c()), ctypes.byref(cfg), 4, 0) == 0
    assert call(dbs.Problem.decode(2, 4, 2, 128, 100)) == dbs.SA_ERR_UNSUPPORTED
    assert call(_prob(head_dim=64)) == dbs.SA_ERR_UNSUPPORTED           # bf16 needs d = 128
    assert call(_prob(dtype="f32")) == dbs.SA_ERR_UNSUPPORTED           # fp32 needs d = 64
    assert call(ok, ptr=None) == dbs.SA_ERR_INVALID_ARG
    assert call(ok, ws_bytes=need - 1) == dbs.SA_ERR_WORKSPACE


def test_noalloc_worklist_rejects_sizes_beyond_scratch(lib):
    # 128 heads x 1024 blocks = 131072 rows need 64 MiB of worklist scratch: refused on
    # the host (SA_ERR_WORKSPACE) before the scratch or any pointer is touched
    p = _prob(heads_q=128, heads_kv=128, seqlen=65536).to_c()
    c = dbs.RouteConfig(k_b=16).to_c()
    need = lib.sparse_attn_workspace_size(ctypes.byref(p), ctypes.byref(c), 1, 0)
    assert need > dbs.NOALLOC_SCRATCH_BYTES
    st = lib.sparse_attn_build_worklist_noalloc(ctypes.byref(p), ctypes.byref(c), None, None, None, 0, None,
                                                None, None, None)
    assert st == dbs.SA_ERR_WORKSPACE
    # an invalid problem is still reported as such first
    bad = _prob(block=32).to_c()
    st = lib.sparse_attn_build_worklist_noalloc(ctypes.byref(bad), ctypes.byref(c), None, None, None, 0, None,
                                                None, None, None)
    assert st == dbs.SA_ERR_UNSUPPORTED


def test_seq_lens_only_for_decode(lib):
    import torch
    lens = torch.ones(4, dtype=torch.int32)           # host memory: only the pointer is checked here
    cfg = dbs.RouteConfig(k_b=8, share_gqa=True)
    ok = dbs.Problem.decode(4, 8, 2, 128, 1000, kv_capacity=1500, seq_lens=lens)
    s = dbs.sizes(ok, cfg)
    assert s.rows == 4 * 2 and s.kv_blocks == 4 * 24   # sized by the bound and the capacity
    for bad in (dataclasses.replace(_prob(), seq_lens=lens),
                dataclasses.replace(dbs.Problem.varlen([64, 64], 8, 2, 128, torch.zeros(3, dtype=torch.int32)),
                                    seq_lens=lens)):
        with pytest.raises(dbs.SAError) as e:
            dbs.sizes(bad, cfg)
        assert e.value.status == dbs.SA_ERR_INVALID_ARG
