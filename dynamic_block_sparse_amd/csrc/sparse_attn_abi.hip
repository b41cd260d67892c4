// C-ABI entry points: host-side validation, geometry, workspace carving, launches.
// Nothing here allocates or synchronises.  The only state kept between calls
// is the per-device address of the static scratch that the no-allocation
// worklist entry point uses in place of a workspace argument.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kMaxWidth = 128;        // k_b + forced blocks per row
constexpr int kMaxRouteBlocks = 32768;   // per sequence; decode rows keep their scores in 128 KB of LDS
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  Geom g;
  int qpool = SA_POOL_MEAN;
  int width_max = 0;
  int n_buckets = 0;
  int64_t kv_slots = 0;   // summary slots allocated (a decode cache's capacity)
  int64_t sum_valid = 0;  // summary slots of valid blocks: the summary pass's grid
  int64_t nnz_cap = 0;
  int dtype = SA_BF16;
};

int validate(const sa_problem* p, const sa_route_cfg* rc, Plan* out) {
  if (!p || !rc || !out) return SA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->heads_q % p->heads_kv != 0)
    return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  out->dtype = p->dtype;
  if (p->mode != SA_PREFILL && p->mode != SA_DECODE) return SA_ERR_INVALID_ARG;
  if (p->block != kBlock) return SA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (rc->qpool != SA_POOL_MEAN && rc->qpool != SA_POOL_MAX) return SA_ERR_INVALID_ARG;
  if (rc->kpool != SA_POOL_MEAN && rc->kpool != SA_POOL_MAX) return SA_ERR_INVALID_ARG;
  if (rc->share_gqa != 0 && rc->share_gqa != 1) return SA_ERR_INVALID_ARG;
  if (rc->select != SA_SELECT_TOPK && rc->select != SA_SELECT_THRESHOLD) return SA_ERR_INVALID_ARG;
  if (!(rc->forced & SA_FORCE_CURRENT) || (rc->forced & ~3u)) return SA_ERR_INVALID_ARG;
  if (rc->window < 0 || rc->window > kMaxWidth) return SA_ERR_INVALID_ARG;
  // forced ids a row can add: the local window (current block included) and the sink
  const int nforced = (rc->window > 1 ? rc->window : 1) + ((rc->forced & SA_FORCE_FIRST) ? 1 : 0);
  if (rc->k_b < nforced || rc->k_b + nforced > kMaxWidth) return SA_ERR_INVALID_ARG;
  if (rc->select == SA_SELECT_THRESHOLD &&
      (rc->k_min < 0 || !isfinite(rc->tau_rel) || rc->tau_rel < 0.f))
    return SA_ERR_INVALID_ARG;

  Geom& g = out->g;
  memset(&g, 0, sizeof(g));
  g.batch = p->batch;
  g.hq = p->heads_q;
  g.hkv = p->heads_kv;
  g.group = p->heads_q / p->heads_kv;
  g.share = rc->share_gqa;
  g.hr = g.share ? g.hkv : g.hq;
  g.hpr = g.share ? g.group : 1;
  g.d = p->head_dim;
  g.mode = p->mode;
  const int64_t d = g.d;
  if (p->mode == SA_DECODE) {
    if (p->cu_seqlens || p->seqlen < 1 || p->q_start != 0) return SA_ERR_INVALID_ARG;
    g.n = p->seqlen;
    g.seq_lens = p->seq_lens;   // per-sequence lengths, each <= n (clamped on the device)
    // the cache may hold room beyond the valid length: strides follow the capacity
    const int cap = p->kv_capacity > 0 ? p->kv_capacity : p->seqlen;
    if (p->kv_capacity < 0 || cap < g.n) return SA_ERR_INVALID_ARG;
    const int nb = (g.n + kBlock - 1) / kBlock;
    const int nbc = (cap + kBlock - 1) / kBlock;
    g.max_blocks = nb;
    g.total_blocks = nb;
    g.rows = (int64_t)g.batch * g.hr;
    g.q_seq = (int64_t)g.hq * d;
    g.q_head = d;
    g.kv_seq = (int64_t)g.hkv * cap * d;
    g.kv_head = (int64_t)cap * d;
    g.sum_seq = (int64_t)g.hkv * nbc;
    g.sum_head = nbc;
    g.lse_seq = g.hq;
    g.lse_head = 1;
    out->kv_slots = (int64_t)g.batch * nbc;
    out->sum_valid = (int64_t)g.batch * nb;
    if (p->block_table) {   // paged cache: every logical block of the capacity has a table entry
      if (p->table_stride < nbc || p->pool_blocks < 1) return SA_ERR_INVALID_ARG;
      g.block_table = p->block_table;
      g.table_stride = p->table_stride;
      g.pool_blocks = p->pool_blocks;
    }
  } else if (p->block_table || p->seq_lens) {
    return SA_ERR_INVALID_ARG;   // a block table pages, and seq_lens sizes, only a decode cache
  } else if (p->cu_seqlens) {
    if (p->kv_capacity != 0 || p->q_start != 0) return SA_ERR_INVALID_ARG;   // packed: no cache, no chunk
    // sequences may be empty (no blocks, no rows); at least one block overall
    if (p->seqlen != 0 || p->total_tokens < 1 || p->total_blocks < 1 ||
        p->max_blocks < 1 || p->max_blocks > p->total_blocks)
      return SA_ERR_INVALID_ARG;
    g.varlen = 1;
    g.cu_seqlens = p->cu_seqlens;
    g.n = 0;
    g.max_blocks = p->max_blocks;
    g.total_blocks = p->total_blocks;
    g.rows = (int64_t)g.hr * p->total_blocks;
    g.q_seq = 0;
    g.q_head = (int64_t)p->total_tokens * d;
    g.kv_seq = 0;
    g.kv_head = (int64_t)p->total_tokens * d;
    g.sum_seq = 0;
    g.sum_head = p->total_blocks;
    g.lse_seq = 0;
    g.lse_head = p->total_tokens;
    out->kv_slots = p->total_blocks;
    out->sum_valid = p->total_blocks;
  } else {
    if (p->seqlen < 1) return SA_ERR_INVALID_ARG;
    g.n = p->seqlen;
    // chunked prefill: queries are tokens [q_start, n) (a whole number of blocks
    // in), K/V the whole sequence in a cache of kv_capacity tokens
    const int cap = p->kv_capacity > 0 ? p->kv_capacity : p->seqlen;
    if (p->kv_capacity < 0 || cap < g.n) return SA_ERR_INVALID_ARG;
    if (p->q_start < 0 || p->q_start % kBlock != 0 || p->q_start >= g.n) return SA_ERR_INVALID_ARG;
    const int nb = (g.n + kBlock - 1) / kBlock;
    const int nbc = (cap + kBlock - 1) / kBlock;
    const int nq = g.n - p->q_start;   // query tokens per sequence
    g.qblk0 = p->q_start / kBlock;
    g.q_tok_off = p->q_start;
    g.max_blocks = nb;
    g.total_blocks = nb;
    g.rows = (int64_t)g.batch * g.hr * (nb - g.qblk0);
    g.q_seq = (int64_t)g.hq * nq * d;
    g.q_head = (int64_t)nq * d;
    g.kv_seq = (int64_t)g.hkv * cap * d;
    g.kv_head = (int64_t)cap * d;
    g.sum_seq = (int64_t)g.hkv * nbc;
    g.sum_head = nbc;
    g.lse_seq = (int64_t)g.hq * nq;
    g.lse_head = nq;
    out->kv_slots = (int64_t)g.batch * nbc;
    out->sum_valid = (int64_t)g.batch * nb;
  }
  out->width_max = rc->k_b + nforced;
  int nbk = 1;
  while ((4 << (nbk - 1)) < out->width_max) ++nbk;
  out->n_buckets = nbk;
  out->nnz_cap = g.rows * out->width_max;
  if (out->nnz_cap > INT32_MAX || g.rows > INT32_MAX) return SA_ERR_UNSUPPORTED;
  out->qpool = rc->qpool;
  return SA_OK;
}

size_t ws_cu_blocks(const Plan& pl) {
  return pl.g.varlen ? align_up((size_t)(pl.g.batch + 1) * sizeof(int32_t)) : 0;
}

// Decode split count.  A split holds at most 64 tiles (one per lane of the
// wavefront that streams it), so at least ceil(width / 64) splits are used.
// By default enough splits are made for ~8 wavefronts per CU, each streaming
// >= 4 tiles (measured on MI355X: 8 per CU beats the LDS-bound maximum of 10).
int min_splits(const Plan& pl) { return (pl.width_max + 63) / 64; }

int auto_splits(const Plan& pl) {
  const int64_t target = 2048;
  int64_t s = (target + pl.g.rows - 1) / pl.g.rows;
  int64_t cap = pl.width_max / 4;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < min_splits(pl)) s = min_splits(pl);
  return s < 1 ? 1 : (int)s;
}

int resolve_splits(const Plan& pl, int requested) {
  if (requested <= 0) return auto_splits(pl);
  return requested < min_splits(pl) ? min_splits(pl) : requested;
}

// Elements of one K (or V) tensor in the problem's layout.
int64_t kv_elems(const Plan& pl) {
  return pl.g.varlen ? (int64_t)pl.g.hkv * pl.g.kv_head : (int64_t)pl.g.batch * pl.g.kv_seq;
}

// Key block slots of one KV head (every sequence's blocks).
int64_t key_slots(const Plan& pl) {
  return pl.g.varlen ? (int64_t)pl.g.total_blocks : (int64_t)pl.g.batch * ((pl.g.n + kBlock - 1) / kBlock);
}

// Elements of the lse array (one per query token and head).
int64_t lse_elems(const Plan& pl) {
  return pl.g.varlen ? (int64_t)pl.g.hq * pl.g.lse_head : (int64_t)pl.g.batch * pl.g.lse_seq;
}

// Backward dK/dV split: a key block listed by more than split_target (row,
// head) pairs is shared by up to max_chunks (<= 9) workgroups; split_target
// is an eighth of the most a block can have, at least 64.  A chunk pays for
// its own K/V tile loads, a cleared fp32 accumulator and atomic adds, so
// fewer than ~64 pairs do not amortise it: MHA n 8192 (at most 128 pairs a
// block) ran its backward in 0.66 ms with a floor of 64 or 96 against 0.75 ms
// with 32, 1.24 ms with 16 and 0.675 ms unsplit; at GQA 2 x 32768 (256) and
// the packed 8-sequence batch up to 65536 tokens (512) a quarter or a
// sixteenth of the maximum were 0.5-7 % slower than an eighth.
// Work items: one per (key block slot, KV head) plus at most one more per
// split_target pairs.
void bwd_split(const Plan& pl, int* split_target, int* max_chunks) {
  const int max_units = pl.g.max_blocks * pl.g.group;
  *split_target = std::max(64, max_units / 8);
  *max_chunks = (max_units + *split_target - 1) / *split_target;
}
int64_t bwd_work_items(const Plan& pl) {
  int st, mc;
  bwd_split(pl, &st, &mc);
  const int ngh = pl.g.share ? pl.g.group : 1;
  return key_slots(pl) * pl.g.hkv + pl.nnz_cap * ngh / st + 1;
}

size_t ws_size(const Plan& pl, int which, int splits) {
  size_t sz = ws_cu_blocks(pl);
  if (which == 0) {
    sz += align_up(route_scores_bytes(pl.g));
    sz += align_up(route_qbar_bytes(pl.g, pl.qpool));
  } else if (which == 1) {
    sz += align_up((size_t)pl.g.rows * kMaxWidth * sizeof(int32_t));
    sz += align_up((size_t)pl.g.rows * sizeof(int32_t));
    sz += align_up(worklist_chunk_bytes(pl.g.rows));
  } else if (which == 2 && pl.g.mode == SA_DECODE) {
    sz += align_up(decode_partials_bytes(pl.g, splits));
  } else if (which == 3) {   // backward: D_i and -lse_i log2(e) per query (lse layout), dK and dV fp32
                             // accumulators, per key block pair counts and finished-workgroup counts
    sz += 2 * align_up((size_t)lse_elems(pl) * sizeof(float));
    sz += 2 * align_up((size_t)kv_elems(pl) * sizeof(float));
    sz += align_up((size_t)2 * key_slots(pl) * pl.g.hkv * sizeof(int));
    // key-major pair lists: offsets per (key block slot, KV head) and one entry per listed tile
    sz += align_up((size_t)(key_slots(pl) * pl.g.hkv + 1) * sizeof(int));
    sz += align_up((size_t)pl.nnz_cap * sizeof(int));
    sz += align_up((size_t)bwd_work_items(pl) * sizeof(int));
  }
  return sz;
}

int prep_cu_blocks(Plan& pl, void* ws, hipStream_t st) {
  if (!pl.g.varlen) return SA_OK;
  int32_t* cb = reinterpret_cast<int32_t*>(ws);
  pl.g.cu_blocks = cb;
  return launch_cu_blocks(pl.g.cu_seqlens, cb, pl.g.batch, st);
}

}  // namespace
}  // namespace sa

// Scratch of the no-allocation worklist build: one copy per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address; kernels get the device address that hipGetSymbolAddress
// returns for the current device (noalloc_scratch below), never the name.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace sa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of the scratch: looked up once per device (with
// that device current) and kept.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

// Worklist build into a given workspace (the caller's, or the static scratch).
int build_worklist_impl(const sa_problem* p, const sa_route_cfg* rc, const int32_t* J, int32_t* row_ptr,
                        int32_t* col_idx, int64_t nnz_cap, int32_t* row_perm, int32_t* bucket_ptr,
                        int32_t* err, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (!J || !row_ptr || !col_idx || !row_perm || !bucket_ptr || !err || !ws)
    return SA_ERR_INVALID_ARG;
  if (nnz_cap < pl.nnz_cap) return SA_ERR_WORKSPACE;
  if (ws_bytes < ws_size(pl, 1, 1)) return SA_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if ((st = prep_cu_blocks(pl, ws, hs)) != SA_OK) return st;
  unsigned char* w = reinterpret_cast<unsigned char*>(ws) + ws_cu_blocks(pl);
  WorklistBufs b;
  b.J = J;
  b.row_ptr = row_ptr;
  b.col_idx = col_idx;
  b.row_perm = row_perm;
  b.bucket_ptr = bucket_ptr;
  b.err = err;
  b.tmp_cols = reinterpret_cast<int32_t*>(w);
  b.tmp_len = reinterpret_cast<int32_t*>(w + align_up((size_t)pl.g.rows * kMaxWidth * sizeof(int32_t)));
  b.chunk = reinterpret_cast<int32_t*>(w + align_up((size_t)pl.g.rows * kMaxWidth * sizeof(int32_t)) +
                                       align_up((size_t)pl.g.rows * sizeof(int32_t)));
  return launch_worklist(pl.g, *rc, pl.width_max, pl.n_buckets, b, hs);
}

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" {

int sparse_attn_bwd(const sa_problem* p, const sa_route_cfg* rc, const int32_t* row_ptr,
                    const int32_t* col_idx, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                    size_t ws_bytes, void* stream) {
  using namespace sa;
  Plan pl;
  int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (p->mode != SA_PREFILL) return SA_ERR_UNSUPPORTED;
  if (!row_ptr || !col_idx || !q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return SA_ERR_INVALID_ARG;
  if ((p->dtype == SA_BF16 && p->head_dim != 128) || (p->dtype == SA_F32 && p->head_dim != 64))
    return SA_ERR_UNSUPPORTED;
  if (pl.g.rows > 65535LL * 65535LL) return SA_ERR_UNSUPPORTED;
  const size_t need = ws_size(pl, 3, 0);
  if (ws_bytes < need || !ws) return SA_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if ((st = prep_cu_blocks(pl, ws, hs)) != SA_OK) return st;
  unsigned char* w = reinterpret_cast<unsigned char*>(ws) + ws_cu_blocks(pl);
  const int64_t n = kv_elems(pl);
  BwdBufs b;
  b.row_ptr = row_ptr;
  b.col_idx = col_idx;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.dout = dout;
  b.lse = lse;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.delta = reinterpret_cast<float*>(w);
  w += align_up((size_t)lse_elems(pl) * sizeof(float));
  b.nlse2 = reinterpret_cast<float*>(w);
  w += align_up((size_t)lse_elems(pl) * sizeof(float));
  b.dk_acc = reinterpret_cast<float*>(w);
  w += align_up((size_t)n * sizeof(float));
  b.dv_acc = reinterpret_cast<float*>(w);
  w += align_up((size_t)n * sizeof(float));
  b.kcount = reinterpret_cast<int*>(w);
  b.kdone = b.kcount + key_slots(pl) * pl.g.hkv;
  w += align_up((size_t)2 * key_slots(pl) * pl.g.hkv * sizeof(int));
  b.kptr = reinterpret_cast<int*>(w);
  w += align_up((size_t)(key_slots(pl) * pl.g.hkv + 1) * sizeof(int));
  b.klist = reinterpret_cast<int*>(w);
  w += align_up((size_t)pl.nnz_cap * sizeof(int));
  b.witem = reinterpret_cast<int*>(w);
  bwd_split(pl, &b.split_target, &b.max_chunks);
  const int64_t witems = bwd_work_items(pl);
  if (witems > INT32_MAX) return SA_ERR_UNSUPPORTED;
  b.witems = (int)witems;
  const int kv_tail = !pl.g.varlen && p->kv_capacity > p->seqlen;   // keys no query can attend
  return launch_bwd(pl.g, p->dtype, b, n, kv_tail, hs);
}

int sparse_attn_append_kv(const sa_problem* p, int32_t n_new, const void* k_new, const void* v_new,
                          void* k_cache, void* v_cache, float* summaries, int32_t kpool, void* stream) {
  using namespace sa;
  if (!p || p->mode != SA_DECODE || p->cu_seqlens || p->q_start != 0) return SA_ERR_INVALID_ARG;
  if (kpool != SA_POOL_MEAN && kpool != SA_POOL_MAX) return SA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->heads_q % p->heads_kv != 0)
    return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  if (p->block != kBlock) return SA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (n_new < 0 || p->seqlen < 0 || p->kv_capacity < 1) return SA_ERR_INVALID_ARG;
  if ((int64_t)p->seqlen + n_new > p->kv_capacity) return SA_ERR_INVALID_ARG;
  if (n_new == 0) return SA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !summaries) return SA_ERR_INVALID_ARG;
  // blocks one launch row covers: those of [L0, L0 + n_new), or with per-sequence
  // starts the most that n_new consecutive tokens can straddle
  int touched = (p->seqlen + n_new - 1) / kBlock - p->seqlen / kBlock + 1;
  if (p->seq_lens) touched = std::min((n_new - 1) / kBlock + 2, (p->kv_capacity + kBlock - 1) / kBlock);
  if (touched > 65535 || (int64_t)p->batch * p->heads_kv > INT32_MAX) return SA_ERR_UNSUPPORTED;
  const int64_t d = p->head_dim, cap = p->kv_capacity, nbc = (cap + kBlock - 1) / kBlock;
  AppendGeom g;
  g.hkv = p->heads_kv;
  g.d = p->head_dim;
  g.len0 = p->seqlen;
  g.n_new = n_new;
  g.cache_head = cap * d;
  g.cache_seq = (int64_t)p->heads_kv * cap * d;
  g.new_head = (int64_t)n_new * d;
  g.new_seq = (int64_t)p->heads_kv * n_new * d;
  g.sum_head = nbc;
  g.sum_seq = (int64_t)p->heads_kv * nbc;
  g.block_table = p->block_table;
  g.table_stride = p->table_stride;
  g.pool_blocks = p->pool_blocks;
  g.seq_lens = p->seq_lens;
  g.kmax = kpool == SA_POOL_MAX;
  if (p->block_table && (p->table_stride < nbc || p->pool_blocks < 1)) return SA_ERR_INVALID_ARG;
  return launch_append_kv(g, p->dtype, p->batch, touched, k_new, v_new, k_cache, v_cache, summaries,
                          reinterpret_cast<hipStream_t>(stream));
}

const char* sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_WORKSPACE: return "workspace or capacity too small";
    case SA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int sparse_attn_sizes(const sa_problem* p, const sa_route_cfg* rc, int64_t* rows,
                      int32_t* width_max, int64_t* nnz_cap, int32_t* n_buckets,
                      int64_t* kv_blocks) {
  Plan pl;
  const int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (rows) *rows = pl.g.rows;
  if (width_max) *width_max = pl.width_max;
  if (nnz_cap) *nnz_cap = pl.nnz_cap;
  if (n_buckets) *n_buckets = pl.n_buckets;
  if (kv_blocks) *kv_blocks = pl.kv_slots;
  return SA_OK;
}

size_t sparse_attn_workspace_size(const sa_problem* p, const sa_route_cfg* rc, int32_t which,
                                  int32_t num_splits) {
  Plan pl;
  if (validate(p, rc, &pl) != SA_OK || which < 0 || which > 3) return 0;
  return ws_size(pl, which, resolve_splits(pl, num_splits));
}

int sparse_attn_route(const sa_problem* p, const sa_route_cfg* rc, const void* q, const void* k,
                      float* summaries, int32_t summaries_in, int32_t* J, void* ws,
                      size_t ws_bytes, void* stream) {
  Plan pl;
  int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (!q || !summaries || !J || (!summaries_in && !k)) return SA_ERR_INVALID_ARG;
  if (summaries_in != 0 && summaries_in != 1) return SA_ERR_INVALID_ARG;
  if (pl.g.max_blocks > kMaxRouteBlocks) return SA_ERR_UNSUPPORTED;
  if (ws_bytes < ws_size(pl, 0, 1) || (ws_size(pl, 0, 1) && !ws)) return SA_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if ((st = prep_cu_blocks(pl, ws, hs)) != SA_OK) return st;
  unsigned char* w = reinterpret_cast<unsigned char*>(ws) + ws_cu_blocks(pl);
  float* scores = reinterpret_cast<float*>(w);
  // pooled queries come out of the summary pass when it runs here
  float* qbar = nullptr;
  if (!summaries_in && route_qbar_bytes(pl.g, pl.qpool) > 0)
    qbar = reinterpret_cast<float*>(w + align_up(route_scores_bytes(pl.g)));
  if (!summaries_in) {
    // one wavefront per valid block: the summary kernel maps slot -> (sequence, block)
    // over the valid blocks (slots of a cache's spare capacity are never written)
    if ((st = launch_summary(pl.g, p->dtype, k, summaries, (int)pl.sum_valid, q, qbar, rc->kpool, hs)) != SA_OK)
      return st;
  }
  return launch_route(pl.g, *rc, p->dtype, q, summaries, qbar, scores, J, hs);
}

int sparse_attn_build_worklist(const sa_problem* p, const sa_route_cfg* rc, const int32_t* J,
                               int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                               int32_t* row_perm, int32_t* bucket_ptr, int32_t* err, void* ws,
                               size_t ws_bytes, void* stream) {
  return build_worklist_impl(p, rc, J, row_ptr, col_idx, nnz_cap, row_perm, bucket_ptr, err, ws, ws_bytes,
                             stream);
}

int sparse_attn_build_worklist_noalloc(const sa_problem* p, const sa_route_cfg* rc, const int32_t* J,
                                       int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                                       int32_t* row_perm, int32_t* bucket_ptr, int32_t* err,
                                       void* stream) {
  Plan pl;
  const int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  const size_t need = ws_size(pl, 1, 1);
  if (need > SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_WORKSPACE;   // more rows than the scratch holds
  void* ws = nullptr;
  const int sst = noalloc_scratch(&ws);
  if (sst != SA_OK) return sst;
  return build_worklist_impl(p, rc, J, row_ptr, col_idx, nnz_cap, row_perm, bucket_ptr, err, ws,
                             SA_NOALLOC_SCRATCH_BYTES, stream);
}

int sparse_attn_fwd(const sa_problem* p, const sa_route_cfg* rc, const int32_t* row_ptr,
                    const int32_t* col_idx, const int32_t* row_perm, const void* q,
                    const void* k, const void* v, void* o, float* lse, int32_t num_splits,
                    void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (!row_ptr || !col_idx || !row_perm || !q || !k || !v || !o) return SA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 256) return SA_ERR_INVALID_ARG;
  if (p->dtype == SA_BF16 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  // bf16 prefill serves any number of query heads per row (2 wavefronts per
  // head, rows of 3 or more heads as workgroups of 4); decode up to 16 (the
  // N slots of its matrix instruction)
  if (p->dtype == SA_BF16 && p->mode == SA_DECODE && pl.g.hpr > 16) return SA_ERR_UNSUPPORTED;
  const int splits = resolve_splits(pl, num_splits);
  const size_t need = ws_size(pl, 2, splits);
  if (ws_bytes < need || (need && !ws)) return SA_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if ((st = prep_cu_blocks(pl, ws, hs)) != SA_OK) return st;
  FwdBufs b;
  b.row_ptr = row_ptr;
  b.col_idx = col_idx;
  b.row_perm = row_perm;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.lse = lse;
  b.part = nullptr;
  if (p->mode == SA_DECODE) {
    b.part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) + ws_cu_blocks(pl));
    return launch_decode(pl.g, p->dtype, b, splits, hs);
  }
  return launch_prefill(pl.g, p->dtype, b, hs);
}

int sparse_attn_fwd_dense(const sa_problem* p, const sa_route_cfg* rc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = validate(p, rc, &pl);
  if (st != SA_OK) return st;
  if (p->mode != SA_PREFILL) return SA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return SA_ERR_INVALID_ARG;
  if (p->dtype == SA_BF16 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  const size_t need = ws_size(pl, 2, 1);
  if (ws_bytes < need || (need && !ws)) return SA_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if ((st = prep_cu_blocks(pl, ws, hs)) != SA_OK) return st;
  FwdBufs b;
  b.row_ptr = nullptr;
  b.col_idx = nullptr;
  b.row_perm = nullptr;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.lse = lse;
  b.part = nullptr;
  return launch_prefill(pl.g, p->dtype, b, hs, /*dense=*/true);
}

}  // extern "C"
