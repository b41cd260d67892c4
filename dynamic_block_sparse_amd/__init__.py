"""dynamic_block_sparse_amd -- dynamic block-sparse attention on AMD MI355X (gfx950).

A thin ctypes binding over libsparse_attn.so (C ABI in include/sparse_attn.h).
The binding only marshals arguments: it turns torch tensors into device
pointers, sizes workspaces and raises on a nonzero status.  Every step of the
path (summaries, routing, worklist, attention) runs in the library's HIP
kernels; there is no Python or CPU fallback.  PyTorch provides device memory
and the current stream.

    import dynamic_block_sparse_amd as dbs
    prob = dbs.Problem.fixed(batch=1, heads_q=16, heads_kv=16, head_dim=128, seqlen=8192,
                             dtype="bf16")
    cfg = dbs.RouteConfig(k_b=16)
    J, summ = dbs.route(prob, cfg, q, k)
    wl = dbs.build_worklist(prob, cfg, J)
    o, lse = dbs.fwd(prob, cfg, wl, q, k, v)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = 0, 1, 2, 3, 4
SA_WL_ERR_RANGE, SA_WL_ERR_ACAUSAL, SA_WL_ERR_PAGE, SA_WL_ERR_LENGTH = 1, 2, 4, 8
SA_F32, SA_BF16 = 0, 1
SA_PREFILL, SA_DECODE = 0, 1
SA_POOL_MEAN, SA_POOL_MAX = 0, 1
SA_SELECT_TOPK, SA_SELECT_THRESHOLD = 0, 1
SA_FORCE_CURRENT, SA_FORCE_FIRST = 1, 2

EXPORTED = ["sparse_attn_sizes", "sparse_attn_workspace_size", "sparse_attn_route",
            "sparse_attn_build_worklist", "sparse_attn_fwd", "sparse_attn_append_kv",
            "sparse_attn_bwd", "sparse_attn_status_string", "sparse_attn_build_worklist_noalloc",
            "sparse_attn_fwd_dense"]
NOALLOC_SCRATCH_BYTES = 32 << 20   # SA_NOALLOC_SCRATCH_BYTES


class SAError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed: status {status} ({text})")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("total_tokens", ctypes.c_int32),
                ("total_blocks", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("kv_capacity", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("table_stride", ctypes.c_int32), ("pool_blocks", ctypes.c_int32),
                ("q_start", ctypes.c_int32), ("seq_lens", ctypes.c_void_p)]


class _RouteCfg(ctypes.Structure):
    _fields_ = [("qpool", ctypes.c_int32), ("share_gqa", ctypes.c_int32),
                ("select", ctypes.c_int32), ("k_b", ctypes.c_int32),
                ("k_min", ctypes.c_int32), ("tau_rel", ctypes.c_float),
                ("forced", ctypes.c_uint32), ("window", ctypes.c_int32),
                ("kpool", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsparse_attn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m dynamic_block_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    P, R = ctypes.POINTER(_Problem), ctypes.POINTER(_RouteCfg)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.sparse_attn_sizes.argtypes = [P, R, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                      ctypes.POINTER(i64), ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.sparse_attn_sizes.restype = ctypes.c_int
    lib.sparse_attn_append_kv.argtypes = [P, i32, vp, vp, vp, vp, vp, i32, vp]
    lib.sparse_attn_append_kv.restype = ctypes.c_int
    lib.sparse_attn_bwd.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_bwd.restype = ctypes.c_int
    lib.sparse_attn_workspace_size.argtypes = [P, R, i32, i32]
    lib.sparse_attn_workspace_size.restype = sz
    lib.sparse_attn_route.argtypes = [P, R, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.sparse_attn_route.restype = ctypes.c_int
    lib.sparse_attn_build_worklist.argtypes = [P, R, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_build_worklist.restype = ctypes.c_int
    lib.sparse_attn_build_worklist_noalloc.argtypes = [P, R, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.sparse_attn_build_worklist_noalloc.restype = ctypes.c_int
    lib.sparse_attn_fwd.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.sparse_attn_fwd.restype = ctypes.c_int
    lib.sparse_attn_fwd_dense.argtypes = [P, R, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_fwd_dense.restype = ctypes.c_int
    lib.sparse_attn_status_string.argtypes = [ctypes.c_int]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(call: str, status: int):
    if status != SA_OK:
        text = load_library().sparse_attn_status_string(status).decode()
        raise SAError(call, status, text)


@dataclasses.dataclass
class Problem:
    """Geometry of one call (mirrors sa_problem)."""

    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seqlen: int                  # fixed n / decode L; 0 for packed varlen
    dtype: str = "bf16"          # "bf16" | "f32"
    mode: str = "prefill"        # "prefill" | "decode"
    block: int = 64
    cu_seqlens: Optional[torch.Tensor] = None   # int32 [batch+1] on the device
    lengths: Optional[list] = None              # host copy of the varlen lengths
    kv_capacity: int = 0         # decode: allocated cache tokens (0 = seqlen)
    block_table: Optional[torch.Tensor] = None  # decode, paged: int32 [batch, stride] pages (device)
    pool_blocks: int = 0         # paged: pages in the [pool, Hkv, b, d] K/V pool
    q_start: int = 0             # chunked prefill: first query token (multiple of block)
    seq_lens: Optional[torch.Tensor] = None     # decode: int32 [batch] per-sequence cached lengths
                                                # (device), each <= seqlen; None = all seqlen

    @staticmethod
    def fixed(batch, heads_q, heads_kv, head_dim, seqlen, dtype="bf16", kv_capacity=0, q_start=0):
        return Problem(batch, heads_q, heads_kv, head_dim, seqlen, dtype, "prefill",
                       kv_capacity=kv_capacity, q_start=q_start)

    @staticmethod
    def decode(batch, heads_q, heads_kv, head_dim, cache_len, dtype="bf16", kv_capacity=0,
               block_table=None, pool_blocks=0, seq_lens=None):
        """cache_len: the cached length of every sequence, or with seq_lens (device
        int32 [batch]) an upper bound on each sequence's own length."""
        return Problem(batch, heads_q, heads_kv, head_dim, cache_len, dtype, "decode",
                       kv_capacity=kv_capacity, block_table=block_table, pool_blocks=pool_blocks,
                       seq_lens=seq_lens)

    @staticmethod
    def varlen(lengths, heads_q, heads_kv, head_dim, cu_seqlens, dtype="bf16"):
        return Problem(len(lengths), heads_q, heads_kv, head_dim, 0, dtype, "prefill",
                       cu_seqlens=cu_seqlens, lengths=list(lengths))

    def to_c(self) -> _Problem:
        p = _Problem()
        p.batch, p.heads_q, p.heads_kv, p.head_dim = self.batch, self.heads_q, self.heads_kv, self.head_dim
        p.block, p.seqlen = self.block, self.seqlen
        p.dtype = SA_BF16 if self.dtype == "bf16" else SA_F32
        p.mode = SA_DECODE if self.mode == "decode" else SA_PREFILL
        p.kv_capacity = self.kv_capacity
        p.q_start = self.q_start
        if self.block_table is not None:
            p.block_table = self.block_table.data_ptr()
            p.table_stride = int(self.block_table.shape[1])
            p.pool_blocks = self.pool_blocks
        if self.seq_lens is not None:
            p.seq_lens = self.seq_lens.data_ptr()
        if self.cu_seqlens is not None:
            p.cu_seqlens = self.cu_seqlens.data_ptr()
            nb = [-(-int(x) // self.block) for x in self.lengths]
            p.total_tokens = int(sum(self.lengths))
            p.total_blocks = int(sum(nb))
            p.max_blocks = int(max(nb))
        return p


@dataclasses.dataclass
class RouteConfig:
    """Routing settings (mirrors sa_route_cfg)."""

    k_b: int = 16
    qpool: str = "mean"          # "mean" | "max"
    share_gqa: bool = False
    select: str = "topk"         # "topk" | "threshold"
    k_min: int = 4
    tau_rel: float = 2.0
    force_first: bool = False
    window: int = 1              # local branch: current block + window - 1 before it, forced
    kpool: str = "mean"          # key summaries: "mean" (block mean) | "max" (per-dimension max)

    def to_c(self) -> _RouteCfg:
        c = _RouteCfg()
        c.qpool = SA_POOL_MAX if self.qpool == "max" else SA_POOL_MEAN
        c.share_gqa = int(bool(self.share_gqa))
        c.select = SA_SELECT_THRESHOLD if self.select == "threshold" else SA_SELECT_TOPK
        c.k_b, c.k_min, c.tau_rel = self.k_b, self.k_min, self.tau_rel
        c.forced = SA_FORCE_CURRENT | (SA_FORCE_FIRST if self.force_first else 0)
        c.window = self.window
        c.kpool = SA_POOL_MAX if self.kpool == "max" else SA_POOL_MEAN
        return c


@dataclasses.dataclass
class Sizes:
    rows: int
    width_max: int
    nnz_cap: int
    n_buckets: int
    kv_blocks: int


@dataclasses.dataclass
class Worklist:
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    row_perm: torch.Tensor
    bucket_ptr: torch.Tensor
    err: torch.Tensor


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_of(prob: Problem) -> torch.dtype:
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


def q_shape(prob: Problem):
    """Q / O / dO shape: fixed [B, Hq, n - q_start, d], packed [Hq, T, d], decode [S, Hq, d]."""
    if prob.mode == "decode":
        return (prob.batch, prob.heads_q, prob.head_dim)
    if prob.cu_seqlens is not None:
        return (prob.heads_q, int(sum(prob.lengths)), prob.head_dim)
    return (prob.batch, prob.heads_q, prob.seqlen - prob.q_start, prob.head_dim)


def kv_shape(prob: Problem):
    """K / V shape: fixed and decode [B, Hkv, kv_capacity or n, d], packed [Hkv, T, d],
    paged decode pool [pool_blocks, Hkv, b, d]."""
    if prob.block_table is not None:
        return (prob.pool_blocks, prob.heads_kv, prob.block, prob.head_dim)
    if prob.cu_seqlens is not None:
        return (prob.heads_kv, int(sum(prob.lengths)), prob.head_dim)
    return (prob.batch, prob.heads_kv, prob.kv_capacity or prob.seqlen, prob.head_dim)


def _require(call: str, name: str, t, shape, dtype, device=None, min_numel: bool = False):
    """Raise ValueError unless t is a contiguous `dtype` tensor of `shape` (or,
    with min_numel, a 1-D one holding at least shape[0] elements).  Checked
    before anything is enqueued: the kernels index these buffers from the
    geometry alone.  Where the tensors live is checked once all of them have
    passed (_on_device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{call}: {name} must be a torch.Tensor, got {type(t).__name__}")
    ok_shape = (t.dim() == 1 and t.numel() >= shape[0]) if min_numel else tuple(t.shape) == tuple(shape)
    want = f"at least {shape[0]} elements (1-D)" if min_numel else f"shape {tuple(shape)}"
    if not ok_shape or t.dtype != dtype:
        raise ValueError(f"{call}: {name} must be {dtype} with {want}, got {t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{call}: {name} must be contiguous (strides {t.stride()})")


def _on_device(call: str, device, **tensors):
    """Raise ValueError unless every given tensor is a GPU tensor on `device`."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{call}: {name} must be a GPU tensor, got device {t.device}")
        if t.device != device:
            raise ValueError(f"{call}: {name} is on {t.device}, expected {device}")


def _require_problem(call: str, prob: Problem, device):
    """The device tables a Problem carries: cu_seqlens [B + 1] and block_table [B, stride], int32."""
    if prob.cu_seqlens is not None:
        if prob.lengths is None or len(prob.lengths) != prob.batch:
            raise ValueError(f"{call}: a packed problem needs the host lengths of its {prob.batch} sequences")
        _require(call, "cu_seqlens", prob.cu_seqlens, (prob.batch + 1,), torch.int32, device)
    if prob.block_table is not None:
        bt = prob.block_table
        if bt.dim() != 2 or bt.shape[0] != prob.batch:
            raise ValueError(f"{call}: block_table must be [batch, stride], got {tuple(bt.shape)}")
        _require(call, "block_table", bt, tuple(bt.shape), torch.int32, device)
    if prob.seq_lens is not None:
        if prob.mode != "decode":
            raise ValueError(f"{call}: seq_lens applies to decode problems only")
        _require(call, "seq_lens", prob.seq_lens, (prob.batch,), torch.int32, device)


def _require_worklist(call: str, prob: Problem, cfg: RouteConfig, wl: "Worklist", device, full: bool = True):
    sz = sizes(prob, cfg)
    _require(call, "row_ptr", wl.row_ptr, (sz.rows + 1,), torch.int32, device)
    _require(call, "col_idx", wl.col_idx, (max(sz.nnz_cap, 1),), torch.int32, device, min_numel=True)
    if full:
        _require(call, "row_perm", wl.row_perm, (max(sz.rows, 1),), torch.int32, device, min_numel=True)
        _require(call, "bucket_ptr", wl.bucket_ptr, (sz.n_buckets + 1,), torch.int32, device)
        _require(call, "err", wl.err, (1,), torch.int32, device)
    return sz


def sizes(prob: Problem, cfg: RouteConfig) -> Sizes:
    lib = load_library()
    r, nnz, kv = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    w, nb = ctypes.c_int32(), ctypes.c_int32()
    p, c = prob.to_c(), cfg.to_c()
    _check("sparse_attn_sizes", lib.sparse_attn_sizes(ctypes.byref(p), ctypes.byref(c), ctypes.byref(r),
                                                      ctypes.byref(w), ctypes.byref(nnz), ctypes.byref(nb),
                                                      ctypes.byref(kv)))
    return Sizes(r.value, w.value, nnz.value, nb.value, kv.value)


def workspace_size(prob: Problem, cfg: RouteConfig, which: int, num_splits: int = 0) -> int:
    p, c = prob.to_c(), cfg.to_c()
    return int(load_library().sparse_attn_workspace_size(ctypes.byref(p), ctypes.byref(c), which, num_splits))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _use_workspace(call: str, workspace: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    """The caller's workspace when it is a big enough device buffer on `device`, else a new one."""
    if workspace is None:
        return _workspace(nbytes, device)
    if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"{call}: workspace must be a contiguous tensor on {device}")
    if workspace.numel() * workspace.element_size() < nbytes:
        return _workspace(nbytes, device)
    return workspace


def summaries_shape(prob: Problem):
    if prob.cu_seqlens is not None:
        nb = sum(-(-int(x) // prob.block) for x in prob.lengths)
        return (prob.heads_kv, nb, prob.head_dim)
    n = prob.kv_capacity if prob.kv_capacity else prob.seqlen
    nb = -(-n // prob.block)
    return (prob.batch, prob.heads_kv, nb, prob.head_dim)


def route(prob: Problem, cfg: RouteConfig, q: torch.Tensor, k: Optional[torch.Tensor],
          summaries: Optional[torch.Tensor] = None, summaries_in: bool = False,
          J: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """sparse_attn_route: returns (J int32 [rows, k_b], fp32 summaries)."""
    lib = load_library()
    _require("route", "q", q, q_shape(prob), _dtype_of(prob))
    dev = q.device
    _require_problem("route", prob, dev)
    if not summaries_in:
        _require("route", "k", k, kv_shape(prob), _dtype_of(prob), dev)
    elif summaries is None:
        raise ValueError("route: summaries_in needs the stored summaries")
    if summaries is None:
        summaries = torch.empty(summaries_shape(prob), dtype=torch.float32, device=dev)
    _require("route", "summaries", summaries, summaries_shape(prob), torch.float32, dev)
    rows = sizes(prob, cfg).rows
    if J is None:
        J = torch.empty((rows, cfg.k_b), dtype=torch.int32, device=dev)
    _require("route", "J", J, (rows, cfg.k_b), torch.int32, dev)
    _on_device("route", dev, q=q, k=None if summaries_in else k, summaries=summaries, J=J,
               cu_seqlens=prob.cu_seqlens, block_table=prob.block_table, seq_lens=prob.seq_lens)
    p, c = prob.to_c(), cfg.to_c()
    wsb = workspace_size(prob, cfg, 0)
    ws = _use_workspace("route", workspace, wsb, dev)
    _check("sparse_attn_route", lib.sparse_attn_route(
        ctypes.byref(p), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(summaries), int(summaries_in),
        _ptr(J), _ptr(ws), wsb, _stream(dev)))
    return J, summaries


def alloc_worklist(prob: Problem, cfg: RouteConfig, device) -> Worklist:
    sz = sizes(prob, cfg)
    return Worklist(row_ptr=torch.empty(sz.rows + 1, dtype=torch.int32, device=device),
                    col_idx=torch.empty(max(sz.nnz_cap, 1), dtype=torch.int32, device=device),
                    row_perm=torch.empty(max(sz.rows, 1), dtype=torch.int32, device=device),
                    bucket_ptr=torch.empty(sz.n_buckets + 1, dtype=torch.int32, device=device),
                    err=torch.zeros(1, dtype=torch.int32, device=device))


def build_worklist(prob: Problem, cfg: RouteConfig, J: torch.Tensor, out: Optional[Worklist] = None,
                   workspace: Optional[torch.Tensor] = None) -> Worklist:
    """sparse_attn_build_worklist: returns the CSR worklist (device tensors)."""
    lib = load_library()
    rows = sizes(prob, cfg).rows
    _require("build_worklist", "J", J, (rows, cfg.k_b), torch.int32)
    dev = J.device
    _require_problem("build_worklist", prob, dev)
    if out is None:
        sz = sizes(prob, cfg)
        out = Worklist(row_ptr=torch.empty(sz.rows + 1, dtype=torch.int32, device=dev),
                       col_idx=torch.empty(max(sz.nnz_cap, 1), dtype=torch.int32, device=dev),
                       row_perm=torch.empty(max(sz.rows, 1), dtype=torch.int32, device=dev),
                       bucket_ptr=torch.empty(sz.n_buckets + 1, dtype=torch.int32, device=dev),
                       err=torch.zeros(1, dtype=torch.int32, device=dev))
    else:
        _require_worklist("build_worklist", prob, cfg, out, dev)
    _on_device("build_worklist", dev, J=J, row_ptr=out.row_ptr, col_idx=out.col_idx, row_perm=out.row_perm,
               bucket_ptr=out.bucket_ptr, err=out.err, cu_seqlens=prob.cu_seqlens,
               block_table=prob.block_table, seq_lens=prob.seq_lens)
    p, c = prob.to_c(), cfg.to_c()
    wsb = workspace_size(prob, cfg, 1)
    ws = _use_workspace("build_worklist", workspace, wsb, dev)
    _check("sparse_attn_build_worklist", lib.sparse_attn_build_worklist(
        ctypes.byref(p), ctypes.byref(c), _ptr(J), _ptr(out.row_ptr), _ptr(out.col_idx),
        out.col_idx.numel(), _ptr(out.row_perm), _ptr(out.bucket_ptr), _ptr(out.err),
        _ptr(ws), wsb, _stream(dev)))
    return out


def build_worklist_noalloc(prob: Problem, cfg: RouteConfig, J: torch.Tensor, out: Worklist) -> Worklist:
    """sparse_attn_build_worklist_noalloc: the worklist of build_worklist into the
    caller's preallocated `out` (alloc_worklist), with the library's static device
    scratch in place of a workspace; allocates nothing."""
    lib = load_library()
    rows = sizes(prob, cfg).rows
    _require("build_worklist_noalloc", "J", J, (rows, cfg.k_b), torch.int32)
    dev = J.device
    _require_problem("build_worklist_noalloc", prob, dev)
    _require_worklist("build_worklist_noalloc", prob, cfg, out, dev)
    _on_device("build_worklist_noalloc", dev, J=J, row_ptr=out.row_ptr, col_idx=out.col_idx,
               row_perm=out.row_perm, bucket_ptr=out.bucket_ptr, err=out.err, cu_seqlens=prob.cu_seqlens,
               block_table=prob.block_table, seq_lens=prob.seq_lens)
    need = workspace_size(prob, cfg, 1)
    if need > NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"build_worklist_noalloc: the problem needs {need} bytes of scratch, more than the "
                         f"{NOALLOC_SCRATCH_BYTES} the library holds ({rows} rows)")
    p, c = prob.to_c(), cfg.to_c()
    _check("sparse_attn_build_worklist_noalloc", lib.sparse_attn_build_worklist_noalloc(
        ctypes.byref(p), ctypes.byref(c), _ptr(J), _ptr(out.row_ptr), _ptr(out.col_idx),
        out.col_idx.numel(), _ptr(out.row_perm), _ptr(out.bucket_ptr), _ptr(out.err), _stream(dev)))
    return out


def fwd(prob: Problem, cfg: RouteConfig, wl: Worklist, q, k, v, o=None, lse=None,
        want_lse: bool = True, num_splits: int = 0, workspace: Optional[torch.Tensor] = None):
    """sparse_attn_fwd: returns (O, LSE or None)."""
    lib = load_library()
    dt, qs, kvs = _dtype_of(prob), q_shape(prob), kv_shape(prob)
    _require("fwd", "q", q, qs, dt)
    dev = q.device
    _require_problem("fwd", prob, dev)
    _require("fwd", "k", k, kvs, dt, dev)
    _require("fwd", "v", v, kvs, dt, dev)
    _require_worklist("fwd", prob, cfg, wl, dev, full=False)
    _require("fwd", "row_perm", wl.row_perm, (max(sizes(prob, cfg).rows, 1),), torch.int32, dev, min_numel=True)
    if o is None:
        o = torch.empty_like(q)
    _require("fwd", "o", o, qs, dt, dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    if lse is not None:
        _require("fwd", "lse", lse, qs[:-1], torch.float32, dev)
    _on_device("fwd", dev, q=q, k=k, v=v, o=o, lse=lse, row_ptr=wl.row_ptr, col_idx=wl.col_idx,
               row_perm=wl.row_perm, cu_seqlens=prob.cu_seqlens, block_table=prob.block_table,
               seq_lens=prob.seq_lens)
    p, c = prob.to_c(), cfg.to_c()
    wsb = workspace_size(prob, cfg, 2, num_splits)
    ws = _use_workspace("fwd", workspace, wsb, dev)
    _check("sparse_attn_fwd", lib.sparse_attn_fwd(
        ctypes.byref(p), ctypes.byref(c), _ptr(wl.row_ptr), _ptr(wl.col_idx), _ptr(wl.row_perm),
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), num_splits, _ptr(ws), wsb, _stream(dev)))
    return o, lse


def fwd_dense(prob: Problem, cfg: RouteConfig, q, k, v, o=None, lse=None, want_lse: bool = True,
              workspace: Optional[torch.Tensor] = None):
    """sparse_attn_fwd_dense: dense causal attention with the sparse kernels
    (every query block attends every earlier key block); returns (O, LSE or None)."""
    lib = load_library()
    dt, qs, kvs = _dtype_of(prob), q_shape(prob), kv_shape(prob)
    _require("fwd_dense", "q", q, qs, dt)
    dev = q.device
    _require_problem("fwd_dense", prob, dev)
    _require("fwd_dense", "k", k, kvs, dt, dev)
    _require("fwd_dense", "v", v, kvs, dt, dev)
    if o is None:
        o = torch.empty_like(q)
    _require("fwd_dense", "o", o, qs, dt, dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    if lse is not None:
        _require("fwd_dense", "lse", lse, qs[:-1], torch.float32, dev)
    _on_device("fwd_dense", dev, q=q, k=k, v=v, o=o, lse=lse, cu_seqlens=prob.cu_seqlens)
    p, c = prob.to_c(), cfg.to_c()
    wsb = workspace_size(prob, cfg, 2)
    ws = _use_workspace("fwd_dense", workspace, wsb, dev)
    _check("sparse_attn_fwd_dense", lib.sparse_attn_fwd_dense(
        ctypes.byref(p), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), wsb,
        _stream(dev)))
    return o, lse


def bwd(prob: Problem, cfg: RouteConfig, wl: Worklist, q, k, v, o, lse, dout, dq=None, dk=None, dv=None,
        workspace: Optional[torch.Tensor] = None):
    """sparse_attn_bwd: returns (dQ, dK, dV) for the forward that produced o and lse."""
    lib = load_library()
    dt, qs, kvs = _dtype_of(prob), q_shape(prob), kv_shape(prob)
    _require("bwd", "q", q, qs, dt)
    dev = q.device
    _require_problem("bwd", prob, dev)
    for name, t, shp, tdt in (("k", k, kvs, dt), ("v", v, kvs, dt), ("o", o, qs, dt),
                              ("lse", lse, qs[:-1], torch.float32), ("dout", dout, qs, dt)):
        _require("bwd", name, t, shp, tdt, dev)
    _require_worklist("bwd", prob, cfg, wl, dev, full=False)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, shp in (("dq", dq, qs), ("dk", dk, kvs), ("dv", dv, kvs)):
        _require("bwd", name, t, shp, dt, dev)
    _on_device("bwd", dev, q=q, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, row_ptr=wl.row_ptr,
               col_idx=wl.col_idx, cu_seqlens=prob.cu_seqlens)
    p, c = prob.to_c(), cfg.to_c()
    wsb = workspace_size(prob, cfg, 3)
    ws = _use_workspace("bwd", workspace, wsb, dev)
    _check("sparse_attn_bwd", lib.sparse_attn_bwd(
        ctypes.byref(p), ctypes.byref(c), _ptr(wl.row_ptr), _ptr(wl.col_idx), _ptr(q), _ptr(k), _ptr(v),
        _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsb, _stream(dev)))
    return dq, dk, dv


def append_kv(prob: Problem, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, summaries: torch.Tensor, kpool: str = "mean"):
    """sparse_attn_append_kv: writes k_new / v_new [S, Hkv, n, d] into rows
    [L0, L0 + n) of the caches [S, Hkv, kv_capacity, d] and updates the fp32
    summaries of the blocks they land in (in place; block means, or
    per-dimension maxima with kpool "max").  L0 = prob.seqlen, or sequence s's
    prob.seq_lens[s] when set.  The caller advances them by n afterwards."""
    dt = torch.bfloat16 if prob.dtype == "bf16" else torch.float32
    cap = prob.kv_capacity
    shape_c = (prob.batch, prob.heads_kv, cap, prob.head_dim)
    if prob.block_table is not None:
        shape_c = (prob.pool_blocks, prob.heads_kv, prob.block, prob.head_dim)
    n = k_new.shape[2] if k_new.dim() == 4 else -1
    shape_n = (prob.batch, prob.heads_kv, n, prob.head_dim)
    for name, t, shp, tdt in (("k_new", k_new, shape_n, dt), ("v_new", v_new, shape_n, dt),
                              ("k_cache", k_cache, shape_c, dt), ("v_cache", v_cache, shape_c, dt),
                              ("summaries", summaries, summaries_shape(prob), torch.float32)):
        if tuple(t.shape) != shp or t.dtype != tdt or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"append_kv: {name} must be a contiguous {tdt} device tensor of shape {shp}, "
                             f"got {tuple(t.shape)} {t.dtype}")
    _require_problem("append_kv", prob, k_cache.device)
    _on_device("append_kv", k_cache.device, k_new=k_new, v_new=v_new, v_cache=v_cache, summaries=summaries,
               block_table=prob.block_table, seq_lens=prob.seq_lens)
    p = prob.to_c()
    _check("sparse_attn_append_kv", load_library().sparse_attn_append_kv(
        ctypes.byref(p), n, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(summaries),
        SA_POOL_MAX if kpool == "max" else SA_POOL_MEAN, _stream(k_cache.device)))


def problem_for(w, inp) -> Problem:
    """Problem geometry for a workload's inputs (see workloads.py)."""
    if w.mode == "decode":
        return Problem.decode(w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seqlen, w.dtype)
    if w.varlen:
        return Problem.varlen(inp.lengths, w.heads_q, w.heads_kv, w.head_dim, inp.cu_seqlens, w.dtype)
    return Problem.fixed(w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seqlen, w.dtype)


def config_for(w) -> RouteConfig:
    return RouteConfig(k_b=w.k_b, qpool=w.qpool, share_gqa=w.share_gqa, select=w.select,
                       k_min=w.k_min, tau_rel=w.tau_rel, force_first=w.forced_first, window=w.window,
                       kpool=w.kpool)
