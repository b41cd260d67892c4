// Shared device-side definitions for the block-sparse attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

constexpr int kBlock = 64;      // b: tokens per block (query and key)
constexpr int kWave = 64;       // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Geometry resolved on the host and passed by value to every kernel.
// Token (s, h, t) of Q lives at q + s*q_seq + h*q_head + (tok0(s) + t)*d;
// K/V likewise with the kv strides.  Summary (s, h, j) lives at
// summaries + (s*sum_seq + h*sum_head + blk0(s) + j)*d.
struct Geom {
  int batch, hq, hkv, group;   // group = hq / hkv
  int hr;                      // routing heads (hkv when shared, else hq)
  int hpr;                     // query heads served by one row (group when shared, else 1)
  int share;                   // 1 when the routing head is the KV head
  int d;                       // head_dim
  int mode;                    // SA_PREFILL / SA_DECODE
  int n;                       // fixed length n / decode cached L; 0 when varlen
  int varlen;
  const int32_t* cu_seqlens;   // device [batch+1] (varlen)
  const int32_t* cu_blocks;    // device [batch+1] block offsets (varlen; in workspace)
  int total_blocks;            // summary slots per kv head plane (varlen) / per (s, h) N (fixed)
  int max_blocks;              // largest per-sequence block count
  int64_t rows;                // worklist rows
  int64_t q_seq, q_head;       // element strides of Q/O (varlen: q_seq = 0)
  int64_t kv_seq, kv_head;     // element strides of K/V
  int64_t sum_seq, sum_head;   // summary strides in blocks (varlen: sum_seq = 0)
  int64_t lse_seq, lse_head;   // strides of the lse array in tokens
  // paged decode cache: K/V are a pool [pool_blocks, hkv, b, d] and logical
  // block j of sequence s lives in page block_table[s * table_stride + j]
  const int32_t* block_table;  // device, or null for a contiguous cache
  int table_stride, pool_blocks;
  // chunked prefill: the queries are tokens [q_tok_off, n) of each sequence
  // (Q, O and lse hold only those), their rows query blocks qblk0 .. N - 1
  int qblk0, q_tok_off;
  // decode with a cached length per sequence (device [batch]); n bounds them all
  const int32_t* seq_lens;
};

struct RowInfo {
  int s, h, r;        // sequence, routing head, query block (decode: last block)
  int len;            // valid tokens (decode: cached length)
  int nblk;           // key blocks of the sequence
  int tok0;           // first token of the sequence in the packed layout (0 if fixed)
  int blk0;           // first block slot of the sequence (varlen), 0 if fixed
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Cached length of decode sequence s: its seq_lens entry clamped into [1, n]
// (the worklist builder reports entries outside), else n.
__device__ __forceinline__ int decode_len(const Geom& g, int s) {
  return g.seq_lens ? min(max(g.seq_lens[s], 1), g.n) : g.n;
}

// Map a worklist row id to (sequence, routing head, query block).
__device__ __forceinline__ RowInfo decode_row(const Geom& g, int64_t row) {
  RowInfo ri;
  if (g.mode == SA_DECODE) {
    ri.s = (int)(row / g.hr);
    ri.h = (int)(row % g.hr);
    ri.len = decode_len(g, ri.s);
    ri.nblk = ceil_div(ri.len, kBlock);
    ri.r = ri.nblk - 1;
    ri.tok0 = 0;
    ri.blk0 = 0;
    return ri;
  }
  if (!g.varlen) {
    int nb = ceil_div(g.n, kBlock);
    const int nrows = nb - g.qblk0;   // query blocks with rows (all but a cached prefix)
    int64_t per_seq = (int64_t)g.hr * nrows;
    ri.s = (int)(row / per_seq);
    int64_t rem = row - (int64_t)ri.s * per_seq;
    ri.h = (int)(rem / nrows);
    ri.r = g.qblk0 + (int)(rem % nrows);
    ri.len = g.n;
    ri.nblk = nb;
    ri.tok0 = 0;
    ri.blk0 = 0;
    return ri;
  }
  // varlen: row = hr * cu_blocks[s] + h * N_s + r; find s by binary search
  int lo = 0, hi = g.batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)g.hr * g.cu_blocks[mid] <= row) lo = mid; else hi = mid - 1;
  }
  ri.s = lo;
  int b0 = g.cu_blocks[lo];
  int nb = g.cu_blocks[lo + 1] - b0;
  int64_t rem = row - (int64_t)g.hr * b0;
  ri.h = (int)(rem / nb);
  ri.r = (int)(rem % nb);
  ri.tok0 = g.cu_seqlens[lo];
  ri.len = g.cu_seqlens[lo + 1] - ri.tok0;
  ri.nblk = nb;
  ri.blk0 = b0;
  return ri;
}

// Q / O element offset of query token t (an absolute position in the sequence).
__device__ __forceinline__ int64_t q_offset(const Geom& g, int s, int h, int tok0, int t) {
  return (int64_t)s * g.q_seq + (int64_t)h * g.q_head + (int64_t)(tok0 + t - g.q_tok_off) * g.d;
}
__device__ __forceinline__ int64_t kv_offset(const Geom& g, int s, int h, int tok0, int t) {
  return (int64_t)s * g.kv_seq + (int64_t)h * g.kv_head + (int64_t)(tok0 + t) * g.d;
}
// Element offset of the first token of logical block j of (sequence s, KV
// head h).  A paged decode cache looks the page up in the block table; a page
// id outside the pool is clamped into it, so nothing reads or writes outside
// the pool (the worklist builder reports such ids, SA_WL_ERR_PAGE).
__device__ __forceinline__ int64_t page_offset(const Geom& g, int page, int h) {
  page = min(max(page, 0), g.pool_blocks - 1);
  return ((int64_t)page * g.hkv + h) * kBlock * g.d;
}
__device__ __forceinline__ int64_t kv_block_offset(const Geom& g, int s, int h, int tok0, int j) {
  if (g.block_table) return page_offset(g, g.block_table[(int64_t)s * g.table_stride + j], h);
  return kv_offset(g, s, h, tok0, j * kBlock);
}
__device__ __forceinline__ int64_t sum_offset(const Geom& g, int s, int h, int blk0, int j) {
  return ((int64_t)s * g.sum_seq + (int64_t)h * g.sum_head + blk0 + j) * g.d;
}
__device__ __forceinline__ int64_t lse_offset(const Geom& g, int s, int h, int tok0, int t) {
  return (int64_t)s * g.lse_seq + (int64_t)h * g.lse_head + tok0 + t - g.q_tok_off;
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Wave-level reductions (64 lanes; all lanes active, every lane gets the
// result).  Within each 16-lane row: DPP quad_perm [1,0,3,2] and [2,3,0,1]
// (partners lane ^ 1, lane ^ 2), then row_half_mirror (lane i <- 7 - i of its
// 8-lane half) and row_mirror (lane i <- 15 - i), after which every lane holds
// its row's result; v_permlane16_swap / v_permlane32_swap then combine rows
// (partners lane ^ 16, lane ^ 32).  All of it stays in the VALU, no LDS.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t row16_reduce(uint32_t x, Op op) {
  x = op(x, dpp_u<0xB1>(x));
  x = op(x, dpp_u<0x4E>(x));
  x = op(x, dpp_u<0x141>(x));
  x = op(x, dpp_u<0x140>(x));
  return x;
}
template <typename Op>
__device__ __forceinline__ uint32_t pair16(uint32_t x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op(r[0], r[1]);
}
template <typename Op>
__device__ __forceinline__ uint32_t pair32(uint32_t x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r[0], r[1]);
}
struct OpAddF { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); } };
struct OpMaxF { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); } };
struct OpAddI { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMinU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  return pair32(pair16(row16_reduce(x, op), op), op);
}
__device__ __forceinline__ float wave_max(float v) { return __uint_as_float(wave_reduce(__float_as_uint(v), OpMaxF{})); }
__device__ __forceinline__ float wave_sum(float v) { return __uint_as_float(wave_reduce(__float_as_uint(v), OpAddF{})); }
__device__ __forceinline__ int wave_sum_i(int v) { return (int)wave_reduce((uint32_t)v, OpAddI{}); }
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) { return wave_reduce(v, OpMinU{}); }
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) { return wave_reduce(v, OpMaxU{}); }
// sum over each 32-lane half of the wave
__device__ __forceinline__ float half_sum(float v) {
  return __uint_as_float(pair16(row16_reduce(__float_as_uint(v), OpAddF{}), OpAddF{}));
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan across an NT-thread workgroup.  `sh` holds NT/64 ints.  All
// threads must call it; *total receives the workgroup sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int inc = wave_incl_scan_i(v);
  __syncthreads();
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = sh[w];
    before += (w < wave) ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

// Cross-lane pair exchanges (gfx950 v_permlane16_swap / v_permlane32_swap).
// With the same value in both operands, the two results of a swap hold, in
// every lane, that lane's value and the value of its partner lane (lane ^ 16,
// resp. lane ^ 32), in some order; combining them with a commutative op gives
// the pairwise reduction.
__device__ __forceinline__ float max_xor16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane mask of lanes below the current one (for ballot-based compaction).
__device__ __forceinline__ uint64_t lanes_below() {
  unsigned lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace sa
