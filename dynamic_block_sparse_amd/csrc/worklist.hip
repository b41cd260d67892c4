// Worklist builder: J -> sorted, deduplicated, forced CSR rows with length buckets.
//
// [P2] §1.2: a row's block ids are sorted by address (neighbouring tiles can
// then coalesce and L2 behaves) and a block entering twice must be removed
// before the softmax.  [P2] §3.1 "index-to-kernel acceptance table": fixed
// width J in, CSR row_ptr / col_idx out, built on the device so the GPU never
// waits on a host-side dedup; int32 ids.  [P2] Eq 7 and [P3] "from index
// output to worklist": rows are grouped into capacity buckets 4, 8, 16, ...
//
// Three launches, no atomics on the output (bit-exact, run-to-run stable):
//   1. rows:    one wavefront per row: validate, add forced ids, LSD radix
//               sort with 1-bit ballot splits through LDS, drop duplicates,
//               write the row's unique ids and its length to workspace
//   2. scan:    one 1024-thread workgroup: row_ptr (exclusive scan of the
//               lengths), per-bucket counts -> bucket_ptr, and the stable
//               (bucket, row) order -> row_perm
//   3. scatter: copy each row's ids to col_idx[row_ptr[row] ..]
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kWidthPad = 128;   // slots per row in workspace (k_b + forced <= 128)
constexpr int kMaxBuckets = 8;

__device__ __forceinline__ int bucket_of(int len) {
  return len <= 4 ? 0 : (32 - __clz(len - 1)) - 2;
}

__global__ void __launch_bounds__(64) wl_rows_kernel(Geom g, sa_route_cfg rc, int nbits,
                                                     const int32_t* __restrict__ J,
                                                     int32_t* __restrict__ tmp_cols,
                                                     int32_t* __restrict__ tmp_len,
                                                     int32_t* __restrict__ err) {
  __shared__ uint32_t keys[2 * kWave];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const uint32_t sentinel = 1u << nbits;   // sorts after every valid id
  const bool ff = (rc.forced & SA_FORCE_FIRST) != 0;
  int ebits = 0;

  auto load_slot = [&](int p) -> uint32_t {
    int v;
    if (p < rc.k_b) v = J[row * rc.k_b + p];
    else if (p == rc.k_b) v = ri.r;                 // forced current block
    else if (p == rc.k_b + 1 && ff) v = 0;          // forced first block
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
  if (lane == 0) tmp_len[row] = n0 + __popcll(m1);
  // OR the row's error bits into the caller's word (one atomic per bad row)
  const uint64_t er = __ballot(ebits & SA_WL_ERR_RANGE);
  const uint64_t ea = __ballot(ebits & SA_WL_ERR_ACAUSAL);
  if (lane == 0 && (er | ea))
    atomicOr(err, (er ? SA_WL_ERR_RANGE : 0) | (ea ? SA_WL_ERR_ACAUSAL : 0));
}

// Row pointers and the bucket order in one 1024-thread workgroup.  Thread t
// owns a contiguous chunk of rows; the row-length sum and the per-bucket row
// counts of every chunk are scanned together (wave scans, then a scan of the
// 16 wave totals in LDS), so the whole scan costs two barriers.
__global__ void __launch_bounds__(1024) wl_scan_kernel(int64_t rows, int n_buckets,
                                                       const int32_t* __restrict__ tmp_len,
                                                       int32_t* __restrict__ row_ptr,
                                                       int32_t* __restrict__ row_perm,
                                                       int32_t* __restrict__ bucket_ptr) {
  constexpr int K = kMaxBuckets + 1;   // [0] length sum, [1 + b] rows in bucket b
  constexpr int NW = 1024 / kWave;
  __shared__ int wtot[NW][K];
  __shared__ int total[K];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t chunk = (rows + 1023) / 1024;
  const int64_t r0 = min((int64_t)tid * chunk, rows), r1 = min(r0 + chunk, rows);
  int v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = 0;
  for (int64_t r = r0; r < r1; ++r) {
    const int len = tmp_len[r];
    v[0] += len;
    const int bk = bucket_of(len);
#pragma unroll
    for (int b = 0; b < kMaxBuckets; ++b) v[1 + b] += (b == bk) ? 1 : 0;
  }
  // inclusive wave scans of all K values
  int inc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) inc[k] = v[k];
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int t = __shfl_up(inc[k], o, kWave);
      if (lane >= o) inc[k] += t;
    }
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) wtot[wave][k] = inc[k];
  }
  __syncthreads();
  // thread k turns column k of the wave totals into exclusive wave prefixes
  if (tid < K) {
    int acc = 0;
    for (int w = 0; w < NW; ++w) {
      const int x = wtot[w][tid];
      wtot[w][tid] = acc;
      acc += x;
    }
    total[tid] = acc;
  }
  __syncthreads();
  int excl[K], tot[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    excl[k] = wtot[wave][k] + inc[k] - v[k];
    tot[k] = total[k];
  }
  // bucket b starts after all rows of buckets < b
  int base[kMaxBuckets];
  {
    int acc = 0;
#pragma unroll
    for (int b = 0; b < kMaxBuckets; ++b) {
      base[b] = acc;
      acc += (b < n_buckets) ? tot[1 + b] : 0;
    }
    if (tid == 0) {
#pragma unroll
      for (int b = 0; b < kMaxBuckets; ++b)
        if (b < n_buckets) bucket_ptr[b] = base[b];
      bucket_ptr[n_buckets] = acc;
      row_ptr[rows] = tot[0];
    }
  }
  int run = excl[0];
  int rank[kMaxBuckets];
#pragma unroll
  for (int b = 0; b < kMaxBuckets; ++b) rank[b] = base[b] + excl[1 + b];
  for (int64_t r = r0; r < r1; ++r) {
    const int len = tmp_len[r];
    row_ptr[r] = run;
    run += len;
    const int bk = bucket_of(len);
    int pos = 0;
#pragma unroll
    for (int b = 0; b < kMaxBuckets; ++b) {
      if (b == bk) {
        pos = rank[b];
        rank[b] += 1;
      }
    }
    row_perm[pos] = (int32_t)r;
  }
}

__global__ void __launch_bounds__(256) wl_scatter_kernel(int64_t rows,
                                                         const int32_t* __restrict__ tmp_cols,
                                                         const int32_t* __restrict__ tmp_len,
                                                         const int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col_idx) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const int n = tmp_len[row];
  const int32_t* src = tmp_cols + row * kWidthPad;
  int32_t* dst = col_idx + row_ptr[row];
  for (int i = lane; i < n; i += kWave) dst[i] = src[i];
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

int launch_worklist(const Geom& g, const sa_route_cfg& rc, int width_max, int n_buckets,
                    const WorklistBufs& b, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (width_max > kWidthPad || n_buckets > kMaxBuckets) return SA_ERR_UNSUPPORTED;
  int nbits = 1;
  while ((1 << nbits) < g.max_blocks) ++nbits;
  wl_rows_kernel<<<(unsigned)g.rows, 64, 0, st>>>(g, rc, nbits, b.J, b.tmp_cols, b.tmp_len, b.err);
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  wl_scan_kernel<<<1, 1024, 0, st>>>(g.rows, n_buckets, b.tmp_len, b.row_ptr, b.row_perm,
                                     b.bucket_ptr);
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  wl_scatter_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, st>>>(g.rows, b.tmp_cols, b.tmp_len,
                                                                  b.row_ptr, b.col_idx);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
