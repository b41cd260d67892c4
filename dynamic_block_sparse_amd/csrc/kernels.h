// Internal launcher declarations (host side) for libsparse_attn.
#pragma once

#include "common.h"

namespace sa {

// Block offsets of a packed batch: cu_blocks[s] = sum_{s' < s} ceil(len_s' / b).
int launch_cu_blocks(const int32_t* cu_seqlens, int32_t* cu_blocks, int batch, hipStream_t st);

// Block summaries of k; with qbar (prefill, mean pooling) the same pass also
// writes each route row's pooled query, [rows, d] fp32.
int launch_summary(const Geom& g, int dtype, const void* k, float* summ, int slots, const void* q,
                   float* qbar, int kpool, hipStream_t st);
size_t route_smem_bytes(const Geom& g, int qpool);
// Candidate scores of every row: [rows, max_blocks] fp32 (workspace).
size_t route_scores_bytes(const Geom& g);
// Pooled queries written by the summary pass: [rows, d] fp32 (workspace;
// prefill with mean pooling only, else 0).
size_t route_qbar_bytes(const Geom& g, int qpool);
// qbar: pooled queries from launch_summary (prefill rows are then scored in
// tiles), or null to pool inside the per-row score kernel.
int launch_route(const Geom& g, const sa_route_cfg& rc, int dtype, const void* q,
                 const float* summ, const float* qbar, float* scores, int32_t* J, hipStream_t st);

struct WorklistBufs {
  const int32_t* J;
  int32_t *row_ptr, *col_idx, *row_perm, *bucket_ptr, *err;
  int32_t *tmp_cols, *tmp_len;   // workspace: [rows * width_pad], [rows]
  int32_t* chunk;                 // workspace: per 256 rows, 10 totals (used above 16384 rows)
};
// Worklist workspace bytes after the rows' slots and lengths: chunk totals.
size_t worklist_chunk_bytes(int64_t rows);
int launch_worklist(const Geom& g, const sa_route_cfg& rc, int width_max, int n_buckets,
                    const WorklistBufs& b, hipStream_t st);

struct FwdBufs {
  const int32_t *row_ptr, *col_idx, *row_perm;
  const void *q, *k, *v;
  void* o;
  float* lse;
  float* part;     // decode partials (workspace)
};
// dense: every row r visits tiles 0 .. r in order (no worklist; rows taken in
// reverse order); else the worklist in b
int launch_prefill(const Geom& g, int dtype, const FwdBufs& b, hipStream_t st, bool dense = false);
int launch_decode(const Geom& g, int dtype, const FwdBufs& b, int splits, hipStream_t st);
size_t decode_partials_bytes(const Geom& g, int splits);

// Backward pass over a forward worklist (prefill): dQ, dK, dV.  delta holds
// D_i per query (lse layout, workspace); dk_acc / dv_acc are the fp32 path's
// accumulators in the K / V layout (workspace), zeroed by the launch.
// kv_tail: K/V hold keys past the sequence end (a cache's capacity), whose
// gradients are zero.
struct BwdBufs {
  const int32_t *row_ptr, *col_idx;
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  // delta: D_i = dO_i . O_i; nlse2: -lse_i log2(e) (both in the lse layout,
  // written by the dQ kernels for the dK/dV kernel)
  float *delta, *nlse2, *dk_acc, *dv_acc;
  // bf16: (row, head) pairs listing each key block and finished workgroups per
  // key block, [key block slot][KV head]; key blocks with more pairs than
  // split_target are shared by several workgroups that add into dk_acc / dv_acc
  int *kcount, *kdone;
  // key-major lists: the rows listing each (key block slot, KV head), as
  // r * (routing heads per KV head) + head, at klist[kptr[i] .. kptr[i + 1])
  int *kptr, *klist;
  // dK/dV workgroups: (slot x KV head) << 4 | chunk, -1 past the last; witems
  // bounds their number (the launch's grid)
  int* witem;
  int witems;
  int split_target, max_chunks;
};
int launch_bwd(const Geom& g, int dtype, const BwdBufs& b, int64_t kv_elems, int kv_tail, hipStream_t st);

// Decode-cache append: rows [len0, len0 + n_new) of every (sequence, KV head)
// and the Eq 11 update of the summaries of the blocks they land in.
struct AppendGeom {
  int hkv, d, len0, n_new;
  int kmax;                        // max-pooled summaries (else block means)
  int64_t cache_seq, cache_head;   // element strides of the K/V cache
  int64_t new_seq, new_head;       // element strides of the new rows
  int64_t sum_seq, sum_head;       // summary strides in blocks
  const int32_t* block_table;      // paged cache: [S, table_stride] pages of a [pool, hkv, b, d] pool
  int table_stride, pool_blocks;
  const int32_t* seq_lens;         // per-sequence len0 (device [S], clamped into [0, len0]), or null
};
int launch_append_kv(const AppendGeom& g, int dtype, int n_seq, int touched, const void* k_new,
                     const void* v_new, void* k_cache, void* v_cache, float* summ, hipStream_t st);

}  // namespace sa
