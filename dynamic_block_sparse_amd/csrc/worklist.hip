// Worklist builder: J -> sorted, deduplicated, forced CSR rows with length buckets.
//
// [P2] §1.2: a row's block ids are sorted by address (neighbouring tiles can
// then coalesce and L2 behaves) and a block entering twice must be removed
// before the softmax.  [P2] §3.1 "index-to-kernel acceptance table": fixed
// width J in, CSR row_ptr / col_idx out, built on the device so the GPU never
// waits on a host-side dedup; int32 ids.  [P2] Eq 7 and [P3] "from index
// output to worklist": rows are grouped into capacity buckets 4, 8, 16, ...
//
// Two launches, no atomics on the output (bit-exact, run-to-run stable):
//   1. rows:    one wavefront per row: validate, add forced ids, LSD radix
//               sort with 1-bit ballot splits through LDS, drop duplicates,
//               write the row's unique ids and its length to workspace
//   2. finish:  one workgroup per 64 or 256 rows: row_ptr (exclusive scan of the
//               lengths), per-bucket counts -> bucket_ptr, the stable
//               (bucket, row) order -> row_perm, and the copy of each row's
//               ids to col_idx[row_ptr[row] ..].  Every workgroup reads all
//               row lengths (4 bytes a row) for the totals and for what
//               precedes its chunk, so none waits for another; a thread's
//               own row (length and ids) is loaded in the same round trip.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kWidthPad = 128;   // slots per row in workspace (k_b + forced <= 128)
constexpr int kMaxBuckets = 8;
constexpr int64_t kChunkedRows = 16384;   // above this many rows the finishing pass reads chunk totals

__device__ __forceinline__ int bucket_of(int len) {
  return len <= 4 ? 0 : (32 - __clz(len - 1)) - 2;
}

__global__ void __launch_bounds__(64) wl_rows_kernel(Geom g, sa_route_cfg rc, int nbits,
                                                     const int32_t* __restrict__ J,
                                                     int32_t* __restrict__ tmp_cols,
                                                     int32_t* __restrict__ tmp_len) {
  __shared__ uint32_t keys[2 * kWave];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const uint32_t sentinel = 1u << nbits;   // sorts after every valid id
  const bool ff = (rc.forced & SA_FORCE_FIRST) != 0;
  int ebits = 0;
  if (g.seq_lens) {   // decode: a length outside [1, n] was clamped by decode_row
    const int L = g.seq_lens[ri.s];
    if (L < 1 || L > g.n) ebits |= SA_WL_ERR_LENGTH;
  }

  const int win = max(rc.window, 1);
  auto load_slot = [&](int p) -> uint32_t {
    int v;
    if (p < rc.k_b) v = J[row * rc.k_b + p];
    else if (p < rc.k_b + win) v = max(ri.r - (p - rc.k_b), -1);   // forced window: r, r-1, ..
    else if (p == rc.k_b + win && ff) v = 0;                         // forced first block
    else v = -1;
    if (v == -1) return sentinel;
    if (v < -1 || v >= ri.nblk) {
      ebits |= SA_WL_ERR_RANGE;
      return sentinel;
    }
    if (g.mode == SA_PREFILL && v > ri.r) {
      ebits |= SA_WL_ERR_ACAUSAL;
      return sentinel;
    }
    if (g.block_table) {   // paged decode cache: the block's page must lie in the pool
      const int page = g.block_table[(int64_t)ri.s * g.table_stride + v];
      if (page < 0 || page >= g.pool_blocks) {
        ebits |= SA_WL_ERR_PAGE;
        return sentinel;
      }
    }
    return (uint32_t)v;
  };
  uint32_t k0 = load_slot(lane);
  uint32_t k1 = load_slot(kWave + lane);

  const uint64_t below = lanes_below();
  for (int b = 0; b <= nbits; ++b) {
    const uint32_t b0 = (k0 >> b) & 1u, b1 = (k1 >> b) & 1u;
    const uint64_t z0 = __ballot(b0 == 0), z1 = __ballot(b1 == 0);
    const int nz0 = __popcll(z0);
    const int nz = nz0 + __popcll(z1);
    const int zb0 = __popcll(z0 & below);
    const int zb1 = __popcll(z1 & below);
    const int p0 = b0 ? nz + (lane - zb0) : zb0;
    const int p1 = b1 ? nz + (kWave - nz0) + (lane - zb1) : nz0 + zb1;
    keys[p0] = k0;
    keys[p1] = k1;
    __syncthreads();
    k0 = keys[lane];
    k1 = keys[kWave + lane];
    __syncthreads();
  }
  // keys[] now holds the sorted slots; keep the first of each run of equal ids
  const uint32_t prev0 = lane > 0 ? keys[lane - 1] : 0xffffffffu;
  const uint32_t prev1 = keys[kWave + lane - 1];
  const bool u0 = k0 != sentinel && k0 != prev0;
  const bool u1 = k1 != sentinel && k1 != prev1;
  const uint64_t m0 = __ballot(u0), m1 = __ballot(u1);
  const int n0 = __popcll(m0);
  int32_t* out = tmp_cols + row * kWidthPad;
  if (u0) out[__popcll(m0 & below)] = (int32_t)k0;
  if (u1) out[n0 + __popcll(m1 & below)] = (int32_t)k1;
  // the row's length, and above it the OR of its lanes' error bits (the
  // finishing pass ORs them over all rows into the caller's word)
  const uint64_t er = __ballot(ebits & SA_WL_ERR_RANGE);
  const uint64_t ea = __ballot(ebits & SA_WL_ERR_ACAUSAL);
  const uint64_t ep = __ballot(ebits & SA_WL_ERR_PAGE);
  const uint64_t el = __ballot(ebits & SA_WL_ERR_LENGTH);
  const int rowbits = (er ? SA_WL_ERR_RANGE : 0) | (ea ? SA_WL_ERR_ACAUSAL : 0) | (ep ? SA_WL_ERR_PAGE : 0) |
                      (el ? SA_WL_ERR_LENGTH : 0);
  if (lane == 0) tmp_len[row] = (n0 + __popcll(m1)) | (rowbits << 16);
}

// Step 2 for rows c0 .. c0 + NT - 1 (c0 = NT * block).  Thread t first sums,
// over every row and over the rows before c0, the length and one count per
// bucket; then owns row c0 + t: its row pointer and its slot in the bucket
// order come from those prefixes plus an exclusive scan inside the chunk.
// NT = 64 for up to 1024 rows (more, smaller workgroups: decode's 512 rows
// 18 us vs 27 us in two 256-thread ones), else 256 (fewer passes over the row
// lengths per workgroup).  Above kChunkedRows rows the totals come from the
// chunk totals of wl_chunk_kernel (CHUNKED) instead of every row length.
// Large problems: chunk totals.  Workgroup c sums, over rows 256 c .. + 255,
// the lengths, the rows per bucket and the OR of the error bits, into
// chunk[c][0 .. kChunkK), so the finishing pass reads one total per chunk
// instead of every row length (rows x chunks loads would grow as the square
// of the rows).
constexpr int kChunkRows = 256;
constexpr int kChunkK = kMaxBuckets + 2;   // [0] length sum, [1 + b] rows in bucket b, [K - 1] error bits

__global__ void __launch_bounds__(kChunkRows) wl_chunk_kernel(int64_t rows, const int32_t* __restrict__ tmp_len,
                                                             int32_t* __restrict__ chunk) {
  constexpr int NW = kChunkRows / kWave;
  __shared__ int red[NW][kChunkK];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t r = (int64_t)blockIdx.x * kChunkRows + tid;
  const int x = r < rows ? tmp_len[r] : 0;
  const int len = x & 0xffff, bk = r < rows ? bucket_of(len) : -1;
  int v[kChunkK];
  v[0] = len;
#pragma unroll
  for (int b = 0; b < kMaxBuckets; ++b) v[1 + b] = b == bk ? 1 : 0;
#pragma unroll
  for (int k = 0; k < kChunkK - 1; ++k) v[k] = wave_sum_i(v[k]);
  // error bits: one bit per ballot
  int eb = 0;
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) eb |= __ballot((x >> (16 + bit)) & 1) ? (1 << bit) : 0;
  v[kChunkK - 1] = eb;
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < kChunkK; ++k) red[wave][k] = v[k];
  __syncthreads();
  if (tid < kChunkK) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t = tid == kChunkK - 1 ? (t | red[w][tid]) : t + red[w][tid];
    chunk[(int64_t)blockIdx.x * kChunkK + tid] = t;
  }
}

template <int NT, bool CHUNKED, int PRE>
__global__ void __launch_bounds__(NT) wl_finish_kernel(int64_t rows, int n_buckets,
                                                        const int32_t* __restrict__ tmp_cols,
                                                        const int32_t* __restrict__ tmp_len,
                                                        const int32_t* __restrict__ chunk,
                                                        int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int32_t* __restrict__ row_perm,
                                                        int32_t* __restrict__ bucket_ptr,
                                                        int32_t* __restrict__ err) {
  constexpr int K = kMaxBuckets + 1;   // [0] length sum, [1 + b] rows in bucket b
  constexpr int NW = NT / kWave;
  static_assert(!CHUNKED || NT == kChunkRows, "a chunk is one workgroup's rows");
  __shared__ int red[NW][2 * K];
  __shared__ int wtot[NW][K];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t c0 = (int64_t)blockIdx.x * NT;
  // this thread's row: its length word and its first 4 PRE slots (every id
  // it can hold), loaded before the totals so that all of the kernel's
  // loads take one memory round trip (rows past the end load row 0's)
  const int64_t r = c0 + tid;
  const bool valid = r < rows;
  const int own = valid ? tmp_len[r] : 0;
  const int32_t* const src = tmp_cols + (valid ? r : 0) * kWidthPad;
  u32x4 ids[PRE];
#pragma unroll
  for (int u = 0; u < PRE; ++u) ids[u] = *reinterpret_cast<const u32x4*>(src + 4 * u);
  // ---- totals over all rows and over the rows before this chunk
  int all[K], pre[K];
  int ebits = 0;   // error bits of every row (workgroup 0 writes their OR to err)
#pragma unroll
  for (int k = 0; k < K; ++k) all[k] = pre[k] = 0;
  if constexpr (CHUNKED) {
    // from the chunk totals: chunk c holds rows c NT .. (c + 1) NT - 1
    const int64_t nch = (rows + NT - 1) / NT;
    for (int64_t c = tid; c < nch; c += NT) {
      const int32_t* t = chunk + c * kChunkK;
      const int in_pre = c < (int64_t)blockIdx.x ? 1 : 0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int x = t[k];
        all[k] += x;
        pre[k] += in_pre * x;
      }
      ebits |= t[kChunkK - 1];
    }
  } else {
  // UP lengths per thread are loaded before any is used (clamped to the last
  // row, weight 0 past the end): one memory round trip per UP rows
  constexpr int UP = 8;
  for (int64_t r0 = tid; r0 < rows; r0 += (int64_t)NT * UP) {
    int lens[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) lens[u] = tmp_len[min(r0 + (int64_t)u * NT, rows - 1)];
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      ebits |= lens[u] >> 16;   // a clamped repeat of the last row adds nothing new
      lens[u] &= 0xffff;
    }
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int64_t r = r0 + (int64_t)u * NT;
      const int in_all = r < rows ? 1 : 0, in_pre = r < c0 ? 1 : 0;
      const int len = lens[u] * in_all;
      const int bk = bucket_of(lens[u]);
      all[0] += len;
      pre[0] += in_pre * len;
#pragma unroll
      for (int b = 0; b < kMaxBuckets; ++b) {
        const int one = (b == bk ? 1 : 0) * in_all;
        all[1 + b] += one;
        pre[1 + b] += in_pre * one;
      }
    }
  }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    all[k] = wave_sum_i(all[k]);
    pre[k] = wave_sum_i(pre[k]);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      red[wave][k] = all[k];
      red[wave][K + k] = pre[k];
    }
  }
  if (blockIdx.x == 0) {   // the OR of every row's error bits
    __shared__ int eor;
    if (tid == 0) eor = 0;
    __syncthreads();
    const uint64_t any = __ballot(ebits != 0);
    if (any) atomicOr(&eor, ebits);
    __syncthreads();
    if (tid == 0) *err = eor;
  }
  // ---- this thread's row and the exclusive scan of the chunk
  const int len = own & 0xffff;
  const int bk = valid ? bucket_of(len) : -1;
  int v[K], inc[K];
  v[0] = len;
#pragma unroll
  for (int b = 0; b < kMaxBuckets; ++b) v[1 + b] = b == bk ? 1 : 0;
#pragma unroll
  for (int k = 0; k < K; ++k) inc[k] = wave_incl_scan_i(v[k]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) wtot[wave][k] = inc[k];
  }
  __syncthreads();
  int tot[K], before[K], excl[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    int t = 0, p = 0, w0 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      t += red[w][k];
      p += red[w][K + k];
      w0 += w < wave ? wtot[w][k] : 0;
    }
    tot[k] = t;
    before[k] = p;
    excl[k] = w0 + inc[k] - v[k];
  }
  // bucket b starts after all rows of buckets < b
  int base_acc = 0, pos = 0;
#pragma unroll
  for (int b = 0; b < kMaxBuckets; ++b) {
    if (b == bk) pos = base_acc + before[1 + b] + excl[1 + b];
    if (blockIdx.x == 0 && tid == 0 && b < n_buckets) bucket_ptr[b] = base_acc;
    base_acc += b < n_buckets ? tot[1 + b] : 0;
  }
  if (blockIdx.x == 0 && tid == 0) {
    bucket_ptr[n_buckets] = base_acc;
    row_ptr[rows] = tot[0];
  }
  if (valid) {
    row_ptr[r] = before[0] + excl[0];
    row_perm[pos] = (int32_t)r;
  }
  // ---- copy this row's ids (loaded at the start) to col_idx[row_ptr[r] ..]
  // with 4-byte stores (row_ptr is not aligned)
  if (valid) {
    int32_t* dst = col_idx + before[0] + excl[0];
#pragma unroll
    for (int u = 0; u < PRE; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * u + e < len) dst[4 * u + e] = (int32_t)ids[u][e];
  }
}

__global__ void __launch_bounds__(1024) cu_blocks_kernel(const int32_t* __restrict__ cu_seqlens,
                                                         int32_t* __restrict__ cu_blocks,
                                                         int batch) {
  __shared__ int sh[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 1024) {
    const int s = base + threadIdx.x;
    int nb = 0;
    if (s < batch) nb = (cu_seqlens[s + 1] - cu_seqlens[s] + kBlock - 1) / kBlock;
    int total;
    const int ex = block_excl_scan<1024>(nb, sh, &total);
    if (s < batch) cu_blocks[s] = carry + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) cu_blocks[batch] = carry;
}

int launch_cu_blocks(const int32_t* cu_seqlens, int32_t* cu_blocks, int batch, hipStream_t st) {
  cu_blocks_kernel<<<1, 1024, 0, st>>>(cu_seqlens, cu_blocks, batch);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

size_t worklist_chunk_bytes(int64_t rows) {
  return (size_t)((rows + kChunkRows - 1) / kChunkRows) * kChunkK * sizeof(int32_t);
}

template <int PRE>
int launch_finish(const Geom& g, int n_buckets, const WorklistBufs& b, hipStream_t st) {
  const unsigned nch = (unsigned)((g.rows + kChunkRows - 1) / kChunkRows);
  if (g.rows <= 1024) {
    wl_finish_kernel<64, false, PRE><<<(unsigned)((g.rows + 63) / 64), 64, 0, st>>>(
        g.rows, n_buckets, b.tmp_cols, b.tmp_len, nullptr, b.row_ptr, b.col_idx, b.row_perm, b.bucket_ptr, b.err);
  } else if (g.rows <= kChunkedRows) {
    wl_finish_kernel<256, false, PRE><<<nch, 256, 0, st>>>(g.rows, n_buckets, b.tmp_cols, b.tmp_len, nullptr,
                                                           b.row_ptr, b.col_idx, b.row_perm, b.bucket_ptr, b.err);
  } else {   // many rows: chunk totals first, so no workgroup reads every row length
    wl_chunk_kernel<<<nch, kChunkRows, 0, st>>>(g.rows, b.tmp_len, b.chunk);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    wl_finish_kernel<256, true, PRE><<<nch, 256, 0, st>>>(g.rows, n_buckets, b.tmp_cols, b.tmp_len, b.chunk,
                                                          b.row_ptr, b.col_idx, b.row_perm, b.bucket_ptr, b.err);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int launch_worklist(const Geom& g, const sa_route_cfg& rc, int width_max, int n_buckets,
                    const WorklistBufs& b, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (width_max > kWidthPad || n_buckets > kMaxBuckets) return SA_ERR_UNSUPPORTED;
  int nbits = 1;
  while ((1 << nbits) < g.max_blocks) ++nbits;
  wl_rows_kernel<<<(unsigned)g.rows, 64, 0, st>>>(g, rc, nbits, b.J, b.tmp_cols, b.tmp_len);
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  // 16-byte chunks of a row's slots that the finishing pass loads: every id
  // the row can hold (8, 17 or 32 chunks)
  if (width_max <= 32) return launch_finish<8>(g, n_buckets, b, st);
  if (width_max <= 68) return launch_finish<17>(g, n_buckets, b, st);
  return launch_finish<32>(g, n_buckets, b, st);
}

}  // namespace sa
