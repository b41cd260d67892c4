"""The Python binding refuses bad tensors before anything is enqueued.

The kernels index Q, K, V, O, lse, dO, J and the worklist from the problem's
geometry alone, so a wrong shape, a wrong dtype, a strided view (a stride-0
expanded dO, a slice along the token axis) or a tensor on the host would be
read or written out of place.  Each such input must raise ValueError in the
binding.  These run on the CPU: the checks are host-side and come before any
library call that launches work (the library is loaded only for its host-side
size queries)."""
import dataclasses

import pytest
import torch

import dynamic_block_sparse_amd as dbs

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(dbs.LIB_PATH),
                                reason="libsparse_attn.so not built")

B, HQ, HKV, N, D = 1, 4, 2, 256, 128


def _prob():
    return dbs.Problem.fixed(B, HQ, HKV, D, N, "bf16")


def _cfg():
    return dbs.RouteConfig(k_b=3)


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _wl(prob, cfg):
    sz = dbs.sizes(prob, cfg)
    return dbs.Worklist(row_ptr=_t((sz.rows + 1,), torch.int32), col_idx=_t((sz.nnz_cap,), torch.int32),
                        row_perm=_t((sz.rows,), torch.int32), bucket_ptr=_t((sz.n_buckets + 1,), torch.int32),
                        err=_t((1,), torch.int32))


def test_shapes_follow_the_layouts():
    p = _prob()
    assert dbs.q_shape(p) == (B, HQ, N, D) and dbs.kv_shape(p) == (B, HKV, N, D)
    pc = dbs.Problem.fixed(B, HQ, HKV, D, N, "bf16", kv_capacity=320, q_start=128)
    assert dbs.q_shape(pc) == (B, HQ, N - 128, D) and dbs.kv_shape(pc) == (B, HKV, 320, D)
    pd = dbs.Problem.decode(3, HQ, HKV, D, 100, "bf16", kv_capacity=128)
    assert dbs.q_shape(pd) == (3, HQ, D) and dbs.kv_shape(pd) == (3, HKV, 128, D)
    pv = dbs.Problem.varlen([70, 30], HQ, HKV, D, torch.tensor([0, 70, 100], dtype=torch.int32))
    assert dbs.q_shape(pv) == (HQ, 100, D) and dbs.kv_shape(pv) == (HKV, 100, D)


def test_host_tensors_are_refused():
    p, c = _prob(), _cfg()
    with pytest.raises(ValueError, match="GPU tensor"):
        dbs.route(p, c, _t(dbs.q_shape(p)), _t(dbs.kv_shape(p)))


@pytest.mark.parametrize("bad", ["q_shape", "q_dtype", "k_shape", "summaries", "J"])
def test_route_refuses(bad):
    p, c = _prob(), _cfg()
    q, k = _t(dbs.q_shape(p)), _t(dbs.kv_shape(p))
    summ = _t(dbs.summaries_shape(p), torch.float32)
    J = _t((dbs.sizes(p, c).rows, c.k_b), torch.int32)
    if bad == "q_shape":
        q = _t((B, HQ, N + 64, D))[:, :, 64:]          # a slice along the token axis: not contiguous
        q = q.contiguous()[:, :, :N - 1]
    elif bad == "q_dtype":
        q = q.float()
    elif bad == "k_shape":
        k = _t((B, HQ, N, D))
    elif bad == "summaries":
        summ = summ.to(torch.bfloat16)
    else:
        J = _t((dbs.sizes(p, c).rows, c.k_b + 1), torch.int32)
    with pytest.raises(ValueError, match="must be"):
        dbs.route(p, c, q, k, summaries=summ, J=J)


def test_strided_views_are_refused():
    p, c = _prob(), _cfg()
    big = _t((B, HQ, N + 64, D))
    q_view = big[:, :, 64:]                             # right shape, wrong strides
    assert tuple(q_view.shape) == dbs.q_shape(p)
    with pytest.raises(ValueError, match="contiguous"):
        dbs.fwd(p, c, _wl(p, c), q_view, _t(dbs.kv_shape(p)), _t(dbs.kv_shape(p)))
    # the stride-0 gradient that o.sum().backward() hands to a custom backward
    q, kv = _t(dbs.q_shape(p)), _t(dbs.kv_shape(p))
    dout = torch.ones((), dtype=torch.bfloat16).expand(dbs.q_shape(p))
    lse = _t(dbs.q_shape(p)[:-1], torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        dbs.bwd(p, c, _wl(p, c), q, kv, kv, q, lse, dout)


@pytest.mark.parametrize("bad", ["lse_dtype", "o_shape", "row_ptr", "col_idx_short", "v_dtype"])
def test_fwd_refuses(bad):
    p, c = _prob(), _cfg()
    q, k, v = _t(dbs.q_shape(p)), _t(dbs.kv_shape(p)), _t(dbs.kv_shape(p))
    o, lse = _t(dbs.q_shape(p)), _t(dbs.q_shape(p)[:-1], torch.float32)
    wl = _wl(p, c)
    if bad == "lse_dtype":
        lse = lse.double()
    elif bad == "o_shape":
        o = _t((B, HQ, N, D // 2))
    elif bad == "row_ptr":
        wl.row_ptr = wl.row_ptr[:-1].clone()
    elif bad == "col_idx_short":
        wl.col_idx = wl.col_idx[:-1].clone()
    else:
        v = v.float()
    with pytest.raises(ValueError):
        dbs.fwd(p, c, wl, q, k, v, o=o, lse=lse)


def test_build_worklist_refuses_bad_J_and_outputs():
    p, c = _prob(), _cfg()
    rows = dbs.sizes(p, c).rows
    with pytest.raises(ValueError, match="J"):
        dbs.build_worklist(p, c, _t((rows, c.k_b), torch.int64))
    wl = _wl(p, c)
    wl.bucket_ptr = _t((1,), torch.int32)
    with pytest.raises(ValueError, match="GPU tensor|bucket_ptr"):
        dbs.build_worklist(p, c, _t((rows, c.k_b), torch.int32), out=wl)


def test_packed_problem_tables_checked():
    cu = torch.tensor([0, 70, 100], dtype=torch.int64)   # int64: refused
    p = dbs.Problem.varlen([70, 30], HQ, HKV, D, cu)
    c = _cfg()
    with pytest.raises(ValueError):
        dbs.route(p, c, _t(dbs.q_shape(p)), _t(dbs.kv_shape(p)))


def test_seq_lens_checked():
    p = dbs.Problem.decode(3, HQ, HKV, D, 300, seq_lens=torch.ones(3, dtype=torch.int64))   # int64: refused
    c = _cfg()
    q, kv = _t(dbs.q_shape(p)), _t(dbs.kv_shape(p))
    with pytest.raises(ValueError, match="seq_lens"):
        dbs.route(p, c, q, kv)
    p = dbs.Problem.decode(3, HQ, HKV, D, 300, seq_lens=torch.ones(2, dtype=torch.int32))    # wrong batch
    with pytest.raises(ValueError, match="seq_lens"):
        dbs.route(p, c, q, kv)
    p = dataclasses.replace(dbs.Problem.fixed(1, HQ, HKV, D, 300), seq_lens=torch.ones(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_lens"):
        dbs.route(p, c, _t(dbs.q_shape(p)), _t(dbs.kv_shape(p)))
