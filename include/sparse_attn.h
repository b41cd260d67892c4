/*
 * sparse_attn.h -- dynamic coarse-grained block-sparse attention on AMD gfx950.
 *
 * C ABI of libsparse_attn.so.  Three calls carry the method:
 *
 *   sparse_attn_route            Q, K            -> block index table J
 *   sparse_attn_build_worklist   J               -> sorted, deduplicated CSR worklist
 *   sparse_attn_fwd              Q, K, V, worklist -> O (and log-sum-exp)
 *
 * with a dense causal variant for the fallback and the comparison:
 *
 *   sparse_attn_fwd_dense        Q, K, V -> O (every earlier block)
 *
 * and one for the decode cache that routing reads:
 *
 *   sparse_attn_append_kv        new K/V rows -> cache rows and block summaries
 *
 * and one for training:
 *
 *   sparse_attn_bwd              dO and the forward's worklist and lse -> dQ, dK, dV
 *
 * The method ([P2] "2.1 Coarse-grained selection: from content grouping to
 * dynamic sparse blocks", PaperTrace sparse-attention 2-1; [P3] "From index to
 * kernel", PaperTrace sparse-attention 5-1):
 *   - tokens are cut into blocks of b = 64; each query block r is routed to at
 *     most k_b key blocks, giving J of shape [B, H, N_q, k_b]  ([P2] opening
 *     paragraph, [P2] §1.2 Eq 1);
 *   - routing scores mean-pooled key-block summaries against a pooled query
 *     ([P2] §2.1 Eq 6), selects top-k or a clipped threshold count ([P2] Eq 7),
 *     scores only complete history blocks and always adds the current block
 *     ([P2] §2.1 "causal boundary", §4.1);
 *   - the worklist sorts each row by address, drops duplicates and builds CSR
 *     row pointers / column indices grouped by length bucket ([P2] §1.2,
 *     §3.1 "index-to-kernel acceptance table"; [P3] "from index output to
 *     worklist");
 *   - the attention kernel loads only the listed K/V tiles, computes exact
 *     Q K^T / sqrt(d) ([P2] Eq 2) with causal and padding masks, and merges
 *     tiles with the online softmax of [P2] Eq 3-5; decode splits a row's tiles
 *     into groups whose partial (m, l, u) states are merged by the same rule
 *     ([P2] §2.2; [P3] "sparse softmax numerics").
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are device memory owned by the caller; pointers
 *     marked (host) are host memory read during the call only.  The library
 *     allocates nothing, never synchronises the stream, and enqueues all work
 *     on `stream` (a hipStream_t; NULL is the null stream).  It keeps no
 *     global state except the static scratch of the no-allocation worklist
 *     build (below); every other call is reentrant.
 *   - Host-detectable problems (bad sizes, unsupported shapes, null pointers,
 *     workspace too small) return a nonzero status before anything is
 *     enqueued.  Data-dependent problems found on the device (block ids out of
 *     range or acausal) set bits in the caller's device word `err`; the
 *     offending entries are dropped.  Nothing falls back silently to another
 *     path ([P2] §3.1 "dense fallback": failures are not hidden).
 *   - Block ids are sequence-local logical ids ([P2] §2.1 variable-length
 *     paragraph; [P2] §3.1 "summaries are cache state"); all index data are
 *     int32 ([P2] §3.1 index dtype paragraph).
 *
 * Layouts (contiguous, row-major; d = head_dim; elements of `dtype`)
 *   fixed-length prefill   Q, O [B, Hq, n, d]      K, V [B, Hkv, n, d]
 *   packed varlen prefill  Q, O [Hq, T, d]         K, V [Hkv, T, d]
 *                          cu_seqlens [B + 1] int32 token offsets
 *   decode                 Q, O [S, Hq, d]         K, V [S, Hkv, C, d] (C = kv_capacity,
 *                                                  of which the first L = seqlen are valid)
 *   log-sum-exp            same as Q without d, fp32
 *   summaries (fp32)       fixed [B, Hkv, N, d]; decode [S, Hkv, ceil(C / b), d];
 *                          varlen [Hkv, sum_s N_s, d]
 *   J (int32)              rows x k_b, rows in (sequence, routing head, query
 *                          block) row-major order; decode has one row per
 *                          (sequence, routing head)
 *   Query head h uses KV head h / (Hq / Hkv).  With share_gqa the routing
 *   head is the KV head and one row serves its Hq / Hkv query heads;
 *   otherwise the routing head is the query head.
 */
#ifndef SPARSE_ATTN_H_
#define SPARSE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
#define SA_OK 0
#define SA_ERR_INVALID_ARG 1   /* null pointer, inconsistent sizes, bad enum */
#define SA_ERR_UNSUPPORTED 2   /* valid but not implemented (head_dim, block, dtype combo) */
#define SA_ERR_WORKSPACE 3     /* workspace or output capacity too small */
#define SA_ERR_HIP 4           /* a HIP launch failed */

/* Device error bits of the worklist's `err` word (their OR over all rows). */
#define SA_WL_ERR_RANGE 1      /* an id < -1 or >= the sequence's block count */
#define SA_WL_ERR_ACAUSAL 2    /* prefill: an id after the row's query block */
#define SA_WL_ERR_PAGE 4       /* paged decode cache: the block's page lies outside the pool */
#define SA_WL_ERR_LENGTH 8     /* decode: a seq_lens entry outside [1, seqlen] (clamped) */

#define SA_F32 0
#define SA_BF16 1
#define SA_PREFILL 0
#define SA_DECODE 1
#define SA_POOL_MEAN 0
#define SA_POOL_MAX 1
#define SA_SELECT_TOPK 0
#define SA_SELECT_THRESHOLD 1
#define SA_FORCE_CURRENT 1u    /* the query's own block (prefill: r; decode: last); required */
#define SA_FORCE_FIRST 2u      /* block 0 (a global sink branch, [P2] §3.2 union) */

/* Problem geometry (host struct, read during the call). */
typedef struct sa_problem {
  int32_t batch;          /* B sequences (decode: S) */
  int32_t heads_q;        /* Hq */
  int32_t heads_kv;       /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t block;          /* b: 64 */
  int32_t seqlen;         /* fixed-length n, or decode cached length L; 0 for packed varlen */
  int32_t dtype;          /* SA_F32 or SA_BF16 (Q, K, V, O) */
  int32_t mode;           /* SA_PREFILL or SA_DECODE */
  const int32_t* cu_seqlens; /* (device) [batch + 1] packed varlen offsets, else NULL; a
                             sequence may be empty (no blocks, no rows), the batch not */
  int32_t total_tokens;   /* varlen: cu_seqlens[batch] (host-known); else ignored */
  int32_t total_blocks;   /* varlen: sum_s ceil(len_s / b) (host-known); else ignored */
  int32_t max_blocks;     /* varlen: max_s ceil(len_s / b) (host-known); else ignored */
  int32_t kv_capacity;    /* decode: tokens allocated per (sequence, KV head) in the K/V
                             cache, >= seqlen; 0 = seqlen.  K/V are [S, Hkv, kv_capacity, d]
                             and summaries [S, Hkv, ceil(kv_capacity / b), d], of which the
                             first seqlen tokens / ceil(seqlen / b) blocks are valid.
                             Fixed-length prefill may use it the same way (chunked prefill
                             over a cache); must be 0 for packed varlen. */
  const int32_t* block_table; /* decode, optional (device): paged cache.  [batch, table_stride]
                             int32: logical block j of sequence s lives in page
                             block_table[s * table_stride + j] of a K/V pool
                             [pool_blocks, heads_kv, b, d] (each (page, head) tile is one
                             contiguous chunk).  Summaries stay per logical block.  NULL:
                             the contiguous layout above.  Must be NULL for prefill. */
  int32_t table_stride;   /* paged: entries per sequence, >= ceil(kv_capacity / b) */
  int32_t pool_blocks;    /* paged: pages in the pool; a page id outside [0, pool_blocks)
                             is reported by the worklist builder (SA_WL_ERR_PAGE, entry
                             dropped) and clamped by every kernel that reads or writes
                             the pool, so nothing touches memory outside it */
  int32_t q_start;        /* fixed-length prefill, optional: chunked prefill.  The queries are
                             tokens [q_start, seqlen) of each sequence (a multiple of b, < seqlen);
                             Q, O and lse hold only those ([B, Hq, seqlen - q_start, d]) while
                             K/V hold the whole sequence (kv_capacity may exceed seqlen, as for
                             a decode cache).  Rows are query blocks q_start / b .. N - 1, routed
                             against every earlier block with the usual causal rules.  0 = the
                             whole sequence; must be 0 for packed varlen and decode. */
  const int32_t* seq_lens; /* decode, optional (device): [batch] int32, the cached length of
                             each sequence when they differ (requests of a decode batch
                             have different histories, [P3] "From index output to
                             worklist").  seqlen is then an upper bound on every entry and
                             sizes the problem.  Routing, the worklist and the attention
                             take length L_s for sequence s: its blocks 0 .. ceil(L_s / b)
                             - 1, the last one forced and masked to its valid keys.  An
                             entry outside [1, seqlen] is clamped into that range by every
                             kernel (nothing reads outside the cache) and reported by the
                             worklist builder (SA_WL_ERR_LENGTH).  sparse_attn_append_kv
                             takes it as each sequence's length before the append (there
                             [0, seqlen]).  NULL: every sequence holds seqlen tokens.  Must
                             be NULL for prefill. */
} sa_problem;

/* Routing settings (host struct). */
typedef struct sa_route_cfg {
  int32_t qpool;          /* SA_POOL_MEAN or SA_POOL_MAX (max over per-query scores) */
  int32_t share_gqa;      /* 1: one routing head per KV head, scores averaged over its query heads */
  int32_t select;         /* SA_SELECT_TOPK or SA_SELECT_THRESHOLD */
  int32_t k_b;            /* J width: top-k budget incl. forced blocks, or k_max; k_b + forced <= 128 */
  int32_t k_min;          /* threshold: lower clip of Eq 7 */
  float tau_rel;          /* threshold: tau_r = max_j g_rj - tau_rel */
  uint32_t forced;        /* SA_FORCE_* bits; SA_FORCE_CURRENT must be set */
  int32_t window;         /* local branch: the current block and the window - 1 blocks before
                             it are forced and never scored ([P2] §3.2 union of a local, a
                             global and a dynamic branch); 0 or 1 = the current block only */
  int32_t kpool;          /* key summaries: SA_POOL_MEAN (the block mean of [P2] Eq 6) or
                             SA_POOL_MAX (per-dimension maximum over the block's valid keys,
                             [P2] §2.1 and §4); stored summaries must have been built the
                             same way */
} sa_route_cfg;

/* Host-side sizes derived from the geometry (no device work).
 *   rows       worklist rows R (prefill: H_r * total blocks, or H_r * B * (N - q_start / b)
 *              for chunked prefill; decode: S * H_r)
 *   width_max  widest possible worklist row: k_b + max(window, 1) + (SA_FORCE_FIRST ? 1 : 0)
 *   nnz_cap    R * width_max: a col_idx capacity that can never overflow
 *   n_buckets  NB: buckets 4, 8, ..., 4 * 2^(NB-1) cover width_max
 *   kv_blocks  summary slots (B * N; decode S * ceil(kv_capacity / b); varlen
 *              total_blocks)
 * Returns SA_OK or SA_ERR_INVALID_ARG / SA_ERR_UNSUPPORTED. */
int sparse_attn_sizes(const sa_problem* p, const sa_route_cfg* rc, int64_t* rows,
                      int32_t* width_max, int64_t* nnz_cap, int32_t* n_buckets,
                      int64_t* kv_blocks);

/* Bytes of device workspace needed by call `which` (0 route, 1 worklist,
 * 2 fwd, 3 bwd).  For fwd in decode mode `num_splits` is the split-KV group count
 * (0 = the library's choice, the same one sparse_attn_fwd makes).  Returns 0
 * for an invalid problem. */
size_t sparse_attn_workspace_size(const sa_problem* p, const sa_route_cfg* rc, int32_t which,
                                  int32_t num_splits);

/* Routing ([P2] §2.1 Eq 6 and Eq 7; causal protocol of [P2] §2.1 and §4.1).
 *   q, k        (device) inputs in the layouts above
 *   summaries   (device, fp32) block summaries c_j = mean of the block's valid
 *               keys.  summaries_in = 0: computed from k and written here (this
 *               is the cache state of [P2] §3.1); summaries_in = 1: read from
 *               here (decode keeps them with the KV cache) and k is not read.
 *   J           (device, int32) [rows, k_b]: forced blocks ascending, then the
 *               selected history blocks ascending, then -1 padding.
 *   Per row: forced F = the window blocks max(r - W + 1, 0) .. r (W = max(window, 1);
 *   decode: r = N - 1) plus block 0 with SA_FORCE_FIRST; candidates are the
 *   complete history blocks j < r (decode: j < N-1) that are not forced; score g_j = pool over the block's valid queries of
 *   q . c_j (no 1/sqrt(d)), averaged over the row's query heads; keep the top
 *   D = min(max(K_r - |F|, 0), |C|) by (score desc, id asc), where K_r = k_b
 *   (top-k) or min(k_b, max(k_min, |F| + #{g_j >= max g - tau_rel})).
 *   Scores are fp32; ties closer than fp32 rounding may order differently from
 *   an exact evaluation.
 *   ws          (device) sparse_attn_workspace_size(p, rc, 0, 0) bytes: the
 *               candidate scores of every row ([rows, max_blocks] fp32); for
 *               prefill with mean pooling, the pooled query of every row
 *               ([rows, d] fp32, written by the summary pass when
 *               summaries_in = 0); for a packed batch, the per-sequence block
 *               offsets.
 *   A sequence may hold up to 32768 blocks (2,097,152 tokens at block 64);
 *   beyond that SA_ERR_UNSUPPORTED.  Rows with more than 8192 candidates are
 *   selected from their scores in memory rather than in registers (same picks). */
int sparse_attn_route(const sa_problem* p, const sa_route_cfg* rc, const void* q, const void* k,
                      float* summaries, int32_t summaries_in, int32_t* J, void* ws,
                      size_t ws_bytes, void* stream);

/* Worklist ([P2] §1.2, §3.1 CSR form; [P3] "from index output to worklist").
 *   J           (device) [rows, k_b] block ids; -1 = empty slot
 *   row_ptr     (device) [rows + 1] exclusive scan of row lengths
 *   col_idx     (device) [nnz_cap]; row i holds its ascending unique ids at
 *               col_idx[row_ptr[i] .. row_ptr[i+1])
 *   row_perm    (device) [rows] rows sorted by (bucket asc, row asc)
 *   bucket_ptr  (device) [n_buckets + 1] row_perm ranges per bucket; bucket of
 *               a row = smallest power of two >= max(length, 4)
 *   err         (device) one int32, set to the OR of the SA_WL_ERR_* bits of
 *               every row (0: no entry was dropped); no need to clear it first
 *   Each row = ascending unique({valid J entries} U forced blocks). */
int sparse_attn_build_worklist(const sa_problem* p, const sa_route_cfg* rc, const int32_t* J,
                               int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                               int32_t* row_perm, int32_t* bucket_ptr, int32_t* err, void* ws,
                               size_t ws_bytes, void* stream);

/* Bytes of the static device scratch behind sparse_attn_build_worklist_noalloc
 * (one copy per GPU the library runs on, held until the process ends). */
#define SA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* The worklist build of sparse_attn_build_worklist without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * calls no allocating routine: the workspace the build needs
 * (sparse_attn_workspace_size(p, rc, 1, 0) bytes: per row its sorted ids and
 * length, for a packed batch the block offsets) is carved from a static
 * device array of SA_NOALLOC_SCRATCH_BYTES bytes, the one of the device that
 * is current when the call is made (stream must belong to that device; the
 * array's address is looked up once per device, on its first call there).
 * Arguments, outputs and results are those of sparse_attn_build_worklist,
 * bit for bit.  Returns SA_ERR_WORKSPACE when the problem needs more than
 * SA_NOALLOC_SCRATCH_BYTES (about 64K worklist rows), SA_ERR_HIP when the
 * scratch cannot be located.  Every call on one GPU shares that GPU's
 * scratch and overwrites it (nothing in it needs to start at zero): calls
 * that can overlap on one GPU (different streams, or host threads) race and
 * must be ordered by the caller. */
int sparse_attn_build_worklist_noalloc(const sa_problem* p, const sa_route_cfg* rc, const int32_t* J,
                                       int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                                       int32_t* row_perm, int32_t* bucket_ptr, int32_t* err,
                                       void* stream);

/* Attention over the worklist ([P2] Eq 2-5; [P3] "sparse softmax numerics").
 *   q, k, v     (device) inputs; o (device) output, same layout and dtype as q
 *   lse         (device, fp32, nullable) m + ln(l) of the scaled logits per query
 *   row_ptr, col_idx, row_perm  (device) a worklist from sparse_attn_build_worklist
 *   Prefill: query i of block r attends key p iff block(p) is in the row,
 *   p <= i and p < the sequence length.  Decode: the single query attends every
 *   cached position of the listed blocks; the row's tiles are cut into
 *   num_splits groups (0 = library's choice; raised to at least
 *   ceil((k_b + forced) / 64)) whose partial (m, l, u) states are merged with
 *   Eq 3-5: inside one workgroup for up to 8 groups (no workspace), through
 *   fp32 states in the workspace and a second kernel for more.  Accumulation
 *   and softmax are fp32; bf16 inputs use bf16 matrix-core products with P
 *   rounded to bf16 before P V.  bf16 needs head_dim 128, and in decode at
 *   most 16 query heads per row (else SA_ERR_UNSUPPORTED); prefill takes any
 *   number. */
int sparse_attn_fwd(const sa_problem* p, const sa_route_cfg* rc, const int32_t* row_ptr,
                    const int32_t* col_idx, const int32_t* row_perm, const void* q,
                    const void* k, const void* v, void* o, float* lse, int32_t num_splits,
                    void* ws, size_t ws_bytes, void* stream);

/* Dense causal attention with the same kernels, layouts, dtypes and masks as
 * sparse_attn_fwd: the dense fallback of [P2] §3.1 (a router that keeps
 * nearly every block is better served densely; failures are not hidden by
 * it) and the dense side of the sparse / dense comparison.  Every query
 * block r attends every key block 0 .. r of its sequence, as if its worklist
 * row listed them all in ascending order, with no worklist and no limit on
 * the row length; query i attends key p iff p <= i and p < the sequence
 * length.  Prefill only (fixed-length, chunked or packed varlen).
 *   rc      only share_gqa is used (one row serves a KV head's query heads,
 *           else one query head); the other fields must be valid as for the
 *           sparse calls
 *   q, k, v, o, lse  as for sparse_attn_fwd (lse nullable)
 *   ws      (device) sparse_attn_workspace_size(p, rc, 2, 0) bytes (the block
 *           offsets of a packed batch; 0 otherwise)
 * bf16 needs head_dim 128 (any number of query heads per row); fp32 takes
 * head_dim 64 or 128.  Returns SA_ERR_UNSUPPORTED for decode problems. */
int sparse_attn_fwd_dense(const sa_problem* p, const sa_route_cfg* rc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward pass of the prefill attention over the forward's worklist ([P2] §4
 * training paragraph and [P3]: gradients reuse the forward's block selection).
 *   row_ptr, col_idx  (device) the worklist the forward used (same problem and config)
 *   q, k, v, o        (device) the forward's inputs and output
 *   lse               (device, fp32) the forward's log-sum-exp (natural log)
 *   dout              (device) dL/dO, layout and dtype of o
 *   dq                (device, out) layout and dtype of q
 *   dk, dv            (device, out) layout and dtype of k: every element is
 *                     written (0 for keys no query attends)
 *   With P_ip = exp(q_i . k_p / sqrt(d) - lse_i) over the keys query i attended,
 *   D_i = dO_i . O_i and dS_ip = P_ip (dO_i . v_p - D_i):
 *   dQ_i = sum_p dS_ip k_p / sqrt(d), dK_p = sum_i dS_ip q_i / sqrt(d),
 *   dV_p = sum_i P_ip dO_i.  bf16: fp32 accumulation on the matrix cores with P
 *   and dS rounded to bf16 as operands; dQ is repeatable bit for bit, and so
 *   are dK, dV except for key blocks listed by many (row, head) pairs, whose
 *   work is shared by several workgroups that add in atomic order.  fp32:
 *   fp32 arithmetic, dK and dV accumulated in fp32 workspace with atomics, so
 *   their summation order is not fixed.
 *   Prefill only (fixed, packed varlen or chunked); bf16 with head_dim 128 or
 *   fp32 with head_dim 64.
 *   ws                (device) sparse_attn_workspace_size(p, rc, 3, 0) bytes. */
int sparse_attn_bwd(const sa_problem* p, const sa_route_cfg* rc, const int32_t* row_ptr,
                    const int32_t* col_idx, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                    size_t ws_bytes, void* stream);

/* Decode-cache append ([P2] §3.1 "summaries are cache state" and Eq 11: the
 * summaries are kept with the KV cache and updated as keys arrive, not
 * rebuilt by a scan over the history).
 *   p           decode geometry (mode SA_DECODE): batch = S, heads_kv, head_dim,
 *               dtype; seqlen = L0, the cached length of every sequence before
 *               the call (0 allowed); kv_capacity >= L0 + n_new (required).
 *               heads_q is not used but must be a valid multiple of heads_kv.
 *               With seq_lens set, sequence s starts from its own L0_s =
 *               seq_lens[s] (clamped into [0, seqlen]; seqlen bounds them all)
 *               and every L0_s below stands for it.
 *   n_new       tokens appended to every sequence (0: nothing is enqueued)
 *   k_new, v_new (device) [S, Hkv, n_new, d] rows to append, in order
 *   k_cache, v_cache (device) [S, Hkv, kv_capacity, d]: rows [L0, L0 + n_new)
 *               receive k_new / v_new; no other row is touched
 *   summaries   (device, fp32) [S, Hkv, ceil(kv_capacity / b), d]: every block j
 *               that receives a new token is updated in place to
 *               (r_j * c_j + sum of its new keys) / (r_j + its new count), r_j =
 *               valid keys of block j before the call (a block with r_j = 0
 *               starts from its new keys); other blocks are not touched.
 *               Summaries of blocks below ceil(L0 / b) must hold the means of
 *               the cached keys (sparse_attn_route with summaries_in = 0 writes
 *               them; this call keeps them).
 *   kpool       SA_POOL_MEAN: the update above.  SA_POOL_MAX (max-pooled
 *               summaries): c_j <- max(c_j, per-dimension max of its new keys),
 *               or that max alone when r_j = 0.
 *   Arithmetic is fp32 (sums of the new keys in token order).  Calls on one
 *   stream apply in order; the caller advances seqlen (and each seq_lens
 *   entry) by n_new afterwards.
 *   Returns SA_ERR_INVALID_ARG for a non-decode problem, a negative n_new,
 *   L0 + n_new > kv_capacity, an unknown kpool or a null pointer (when
 *   n_new > 0). */
int sparse_attn_append_kv(const sa_problem* p, int32_t n_new, const void* k_new, const void* v_new,
                          void* k_cache, void* v_cache, float* summaries, int32_t kpool, void* stream);

/* Human-readable text for a status code (static string). */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H_ */
