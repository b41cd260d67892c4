"""Seeded synthetic workloads for dynamic block-sparse attention.

This module only *makes inputs*: problem shapes, sequence lengths, and Q/K/V
tensors drawn from N(0, 1) with an optional planted relevance direction.  It
holds none of the method's arithmetic (no summaries, scores, selection,
worklists or attention) and imports neither the HIP path nor the oracle, so
both sides can consume the same tensors.

Layouts (row-major, contiguous):
  fixed-length prefill  q [B, Hq, n, d]   k, v [B, Hkv, n, d]
  packed varlen prefill q [Hq, T, d]      k, v [Hkv, T, d]   cu_seqlens [B+1] int32
  decode                q [S, Hq, d]      k, v [S, Hkv, L, d]  (one query per sequence)

Random draws use torch generators seeded from a (workload seed, tensor id,
sequence, head) key, generated chunk by chunk on the requested device, so a
32 GiB decode cache never needs a host copy.  Values are drawn in fp32, the
planted direction is added in fp32, and the result is rounded once to the
workload dtype (round-to-nearest-even for bf16).

Planting (the pages fix only "random earlier blocks get +alpha*u, Q gets
+gain*u"; the remaining choices are this module's):
  u      = a unit vector drawn per (head) / (batch, kv head) / (sequence)
  blocks = distinct, uniform over [0, N-1) so never the last block
  K      += alpha * u on every token of those blocks (for that kv head)
  Q      += gain * u on every query token of the affected query heads
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_PLANT, TENSOR_LENGTHS = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: shape, routing settings and input recipe."""

    name: str
    dtype: str                  # "f32" | "bf16"
    mode: str                   # "prefill" | "decode"
    batch: int                  # sequences
    heads_q: int
    heads_kv: int
    head_dim: int
    block: int = 64
    seqlen: int = 0             # fixed n (prefill) or cached L (decode); 0 => varlen
    varlen_min: int = 0         # varlen: lengths 64*U{varlen_min/64 .. varlen_max/64}
    varlen_max: int = 0
    qpool: str = "mean"         # "mean" | "max"
    share_gqa: bool = False     # route per KV head (mean over its query heads)
    select: str = "topk"        # "topk" | "threshold"
    k_b: int = 16               # J width: total budget (top-k) or k_max (threshold)
    k_min: int = 4
    tau_rel: float = 2.0
    forced_first: bool = False  # force block 0 in addition to the current block
    window: int = 1             # forced local window in blocks, the current block included
    kpool: str = "mean"         # key summaries: block mean (Eq 6) or per-dimension max
    plant_scope: str = "none"   # "none" | "head" | "kv" | "seq"
    plant_blocks: int = 0
    plant_alpha: float = 0.0
    plant_gain: float = 1.0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def route_heads(self) -> int:
        return self.heads_kv if self.share_gqa else self.heads_q

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def varlen(self) -> bool:
        return self.mode == "prefill" and self.seqlen == 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five problem settings the method is evaluated on.
TINY_F32 = Workload(
    name="tiny_f32_b1_h2_n512_d64_kb3", dtype="f32", mode="prefill", batch=1,
    heads_q=2, heads_kv=2, head_dim=64, seqlen=512, qpool="max", k_b=3, seed=1)
TINY_F32_DENSE = TINY_F32.replace(name="tiny_f32_b1_h2_n512_d64_kb8_dense", k_b=8)
PREFILL_MHA = Workload(
    name="prefill_mha_b1_h16_n8192_d128_kb16", dtype="bf16", mode="prefill", batch=1,
    heads_q=16, heads_kv=16, head_dim=128, seqlen=8192, qpool="mean", k_b=16,
    plant_scope="head", plant_blocks=8, plant_alpha=2.0, seed=2)
PREFILL_GQA = Workload(
    name="prefill_gqa_b2_hq32_hkv8_n32768_d128_kb32", dtype="bf16", mode="prefill",
    batch=2, heads_q=32, heads_kv=8, head_dim=128, seqlen=32768, qpool="mean",
    share_gqa=True, k_b=32, forced_first=True,
    plant_scope="kv", plant_blocks=4, plant_alpha=3.0, seed=3)
VARLEN = Workload(
    name="varlen_8seq_2k_64k_hq32_hkv8_d128_thresh", dtype="bf16", mode="prefill",
    batch=8, heads_q=32, heads_kv=8, head_dim=128, seqlen=0, varlen_min=2048,
    varlen_max=65536, qpool="mean", share_gqa=True, select="threshold", k_b=64,
    k_min=4, tau_rel=2.0, plant_scope="seq", plant_blocks=8, plant_alpha=2.0, seed=4)
DECODE = Workload(
    name="decode_64seq_L131072_hq32_hkv8_d128_kb64", dtype="bf16", mode="decode",
    batch=64, heads_q=32, heads_kv=8, head_dim=128, seqlen=131072, qpool="mean",
    share_gqa=True, k_b=64, plant_scope="kv", plant_blocks=16, plant_alpha=2.0, seed=5)

ALL = [TINY_F32, TINY_F32_DENSE, PREFILL_MHA, PREFILL_GQA, VARLEN, DECODE]
BY_NAME = {w.name: w for w in ALL}


def _key(*parts: int) -> int:
    h = hashlib.blake2b(b"|".join(str(int(p)).encode() for p in parts), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _normal(shape, key: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(key)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit(d: int, key: int) -> np.ndarray:
    rng = np.random.Generator(np.random.Philox(key=key))
    u = rng.standard_normal(d)
    return u / np.linalg.norm(u)


def _plant_blocks(n_blocks: int, count: int, key: int) -> np.ndarray:
    """Distinct block ids, uniform over [0, n_blocks-1) (never the last block)."""
    rng = np.random.Generator(np.random.Philox(key=key))
    pool = max(n_blocks - 1, 0)
    count = min(count, pool)
    return np.sort(rng.choice(pool, size=count, replace=False)) if count else np.zeros(0, np.int64)


def seq_lengths(w: Workload) -> list[int]:
    """Sequence lengths: fixed n, decode L, or 64*U{a..b} drawn from the seed."""
    if not w.varlen:
        return [w.seqlen] * w.batch
    rng = np.random.Generator(np.random.Philox(key=_key(w.seed, TENSOR_LENGTHS)))
    lo, hi = w.varlen_min // w.block, w.varlen_max // w.block
    return [int(x) * w.block for x in rng.integers(lo, hi + 1, size=w.batch)]


@dataclasses.dataclass
class Inputs:
    w: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lengths: list
    cu_seqlens: Optional[torch.Tensor]   # int32 [B+1] on the device (varlen only)
    planted: dict                        # (scope key) -> planted block ids


def _plant_units(w: Workload, lengths):
    """Yield (seq, kv_head, q_heads, block ids, unit vector) planting records."""
    d, G = w.head_dim, w.group
    if w.plant_scope == "none":
        return
    for s, L in enumerate(lengths):
        nb = -(-L // w.block)
        for hk in range(w.heads_kv):
            if w.plant_scope == "head":          # MHA: one u per head
                assert G == 1
                u = _unit(d, _key(w.seed, TENSOR_PLANT, 0, hk, 1))
            elif w.plant_scope == "kv":          # one u per (sequence, kv head)
                u = _unit(d, _key(w.seed, TENSOR_PLANT, s, hk, 1))
            else:                                # "seq": one u per sequence
                u = _unit(d, _key(w.seed, TENSOR_PLANT, s, 0, 1))
            blocks = _plant_blocks(nb, w.plant_blocks, _key(w.seed, TENSOR_PLANT, s, hk, 2))
            qh = list(range(hk * G, (hk + 1) * G))
            yield s, hk, qh, blocks, u


def make_inputs(w: Workload, device="cpu", lengths=None) -> Inputs:
    """Draw Q, K, V for workload `w` on `device` (fp32 draws, one rounding to dtype)."""
    dev = torch.device(device)
    d, b = w.head_dim, w.block
    if lengths is not None:
        lengths = list(lengths)
        w = w.replace(batch=len(lengths))
    else:
        lengths = seq_lengths(w)
    dt = w.torch_dtype
    units = list(_plant_units(w, lengths))
    kplant = {}   # (s, hk) -> (blocks, u)
    qplant = {}   # (s, hq) -> u
    for s, hk, qh, blocks, u in units:
        kplant[(s, hk)] = (blocks, u)
        for h in qh:
            qplant[(s, h)] = u

    def fill_chunk(dst, tid, s, h, ntok, u_add=None, blocks=None, alpha=0.0):
        x = _normal((ntok, d), _key(w.seed, tid, s, h), dev)
        if u_add is not None:
            ut = torch.as_tensor(u_add, dtype=torch.float32, device=dev)
            if blocks is None:
                x += w.plant_gain * ut
            else:
                for j in blocks:
                    x[j * b:min((j + 1) * b, ntok)] += alpha * ut
        dst.copy_(x.to(dt))

    cu = None
    if w.mode == "decode":
        S, L = w.batch, w.seqlen
        q = torch.empty((S, w.heads_q, d), dtype=dt, device=dev)
        k = torch.empty((S, w.heads_kv, L, d), dtype=dt, device=dev)
        v = torch.empty_like(k)
        for s in range(S):
            for h in range(w.heads_q):
                fill_chunk(q[s, h:h + 1], TENSOR_Q, s, h, 1, qplant.get((s, h)))
            for h in range(w.heads_kv):
                bl, u = kplant.get((s, h), (None, None))
                fill_chunk(k[s, h], TENSOR_K, s, h, L, u, bl, w.plant_alpha)
                fill_chunk(v[s, h], TENSOR_V, s, h, L)
    elif w.varlen:
        T = sum(lengths)
        offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        q = torch.empty((w.heads_q, T, d), dtype=dt, device=dev)
        k = torch.empty((w.heads_kv, T, d), dtype=dt, device=dev)
        v = torch.empty_like(k)
        for s, L in enumerate(lengths):
            a, e = int(offs[s]), int(offs[s + 1])
            for h in range(w.heads_q):
                fill_chunk(q[h, a:e], TENSOR_Q, s, h, L, qplant.get((s, h)))
            for h in range(w.heads_kv):
                bl, u = kplant.get((s, h), (None, None))
                fill_chunk(k[h, a:e], TENSOR_K, s, h, L, u, bl, w.plant_alpha)
                fill_chunk(v[h, a:e], TENSOR_V, s, h, L)
        cu = torch.as_tensor(offs, dtype=torch.int32, device=dev)
    else:
        B, n = w.batch, w.seqlen
        q = torch.empty((B, w.heads_q, n, d), dtype=dt, device=dev)
        k = torch.empty((B, w.heads_kv, n, d), dtype=dt, device=dev)
        v = torch.empty_like(k)
        for s in range(B):
            for h in range(w.heads_q):
                fill_chunk(q[s, h], TENSOR_Q, s, h, n, qplant.get((s, h)))
            for h in range(w.heads_kv):
                bl, u = kplant.get((s, h), (None, None))
                fill_chunk(k[s, h], TENSOR_K, s, h, n, u, bl, w.plant_alpha)
                fill_chunk(v[s, h], TENSOR_V, s, h, n)
    planted = {key: val[0].tolist() for key, val in kplant.items()}
    return Inputs(w, q, k, v, lengths, cu, planted)


def per_sequence(inp: Inputs):
    """Split tensors into per-sequence CPU float64 numpy views (for the oracle side).

    Returns lists over sequences of q [Hq, len_q, d], k [Hkv, len_k, d], v [Hkv, len_k, d].
    Pure layout plumbing: slicing and dtype widening, no arithmetic of the method.
    """
    w = inp.w
    qs, ks, vs = [], [], []
    if w.mode == "decode":
        for s in range(w.batch):
            qs.append(inp.q[s].unsqueeze(1).double().cpu().numpy())
            ks.append(inp.k[s].double().cpu().numpy())
            vs.append(inp.v[s].double().cpu().numpy())
    elif w.varlen:
        offs = np.concatenate([[0], np.cumsum(inp.lengths)])
        for s in range(w.batch):
            a, e = int(offs[s]), int(offs[s + 1])
            qs.append(inp.q[:, a:e].double().cpu().numpy())
            ks.append(inp.k[:, a:e].double().cpu().numpy())
            vs.append(inp.v[:, a:e].double().cpu().numpy())
    else:
        for s in range(w.batch):
            qs.append(inp.q[s].double().cpu().numpy())
            ks.append(inp.k[s].double().cpu().numpy())
            vs.append(inp.v[s].double().cpu().numpy())
    return qs, ks, vs


def per_sequence_subset(inp: Inputs, seqs):
    """Like per_sequence, for the listed sequences only (lists aligned with `seqs`)."""
    w = inp.w
    offs = np.concatenate([[0], np.cumsum(inp.lengths)])
    qs, ks, vs = [], [], []
    for s in seqs:
        if w.mode == "decode":
            qs.append(inp.q[s].unsqueeze(1).double().cpu().numpy())
            ks.append(inp.k[s].double().cpu().numpy())
            vs.append(inp.v[s].double().cpu().numpy())
        elif w.varlen:
            a, e = int(offs[s]), int(offs[s + 1])
            qs.append(inp.q[:, a:e].double().cpu().numpy())
            ks.append(inp.k[:, a:e].double().cpu().numpy())
            vs.append(inp.v[:, a:e].double().cpu().numpy())
        else:
            qs.append(inp.q[s].double().cpu().numpy())
            ks.append(inp.k[s].double().cpu().numpy())
            vs.append(inp.v[s].double().cpu().numpy())
    return qs, ks, vs
