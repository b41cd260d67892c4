// Decode-cache append: new K/V rows go into the cache, and the summaries of
// the blocks they land in are updated in place.
//
// [P2] §3.1 (summaries are cache state) and Eq 11: block j's summary is the
// running mean of its r_j valid keys, kept with the KV cache and updated as
// keys arrive instead of being rebuilt by a scan over the history.  A chunk of
// n new keys of block j turns c_j into (r_j c_j + sum of the new keys) /
// (r_j + n); a block that had no valid key (r_j = 0) starts from the new keys.
// Max-pooled summaries ([P2] §2.1, §4) take the per-dimension maximum with the
// new keys instead.
//
// A paged cache (a block table into a [pool, Hkv, b, d] pool) writes each
// block's rows into its page.
//
// One wavefront per (sequence, KV head, touched block).  Each lane owns E =
// d / 64 adjacent columns: it copies those columns of the block's new K and V
// rows (so a row moves as one coalesced 128- or 256-byte burst per tensor),
// sums the new keys of its columns in fp32 in token order, and writes the
// updated summary.  Rows are handled four at a time so their loads are in
// flight together.
#include "common.h"
#include "kernels.h"

namespace sa {

template <typename T, int E>
__global__ void __launch_bounds__(64) append_kv_kernel(AppendGeom g, const T* __restrict__ k_new,
                                                       const T* __restrict__ v_new, T* __restrict__ k_cache,
                                                       T* __restrict__ v_cache, float* __restrict__ summ) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x;
  const int s = (int)blockIdx.x / g.hkv, h = (int)blockIdx.x % g.hkv;
  // this sequence's length before the append (its own, or the common one)
  const int len0 = g.seq_lens ? min(max(g.seq_lens[s], 0), g.len0) : g.len0;
  const int j = len0 / kBlock + (int)blockIdx.y;   // block that receives tokens [t0, t1)
  const int lo = j * kBlock;
  const int t0 = max(lo, len0), t1 = min(lo + kBlock, len0 + g.n_new);
  if (t0 >= t1) return;   // the grid covers the most blocks any start can touch
  const int r_old = max(0, min(lo + kBlock, len0) - lo);   // valid keys before the append
  const int col = lane * E;
  const T* kn = k_new + (int64_t)s * g.new_seq + (int64_t)h * g.new_head + col;
  const T* vn = v_new + (int64_t)s * g.new_seq + (int64_t)h * g.new_head + col;
  // destination rows: token t of the block sits at row t - lo of its page (paged
  // cache, page id clamped into the pool) or at row t of the sequence's plane
  int64_t dst0;
  if (g.block_table) {
    const int page = min(max(g.block_table[(int64_t)s * g.table_stride + j], 0), g.pool_blocks - 1);
    dst0 = ((int64_t)page * g.hkv + h) * kBlock * D - (int64_t)lo * D;
  } else {
    dst0 = (int64_t)s * g.cache_seq + (int64_t)h * g.cache_head;
  }
  T* kd = k_cache + dst0 + col;
  T* vd = v_cache + dst0 + col;

  // block sums of the new keys, or their per-dimension maxima (max-pooled summaries)
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = g.kmax ? -INFINITY : 0.f;
  constexpr int U = 4;
  int t = t0;
  for (; t + U <= t1; t += U) {
    T kx[U][E], vx[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kx[u][e] = kn[(int64_t)(t + u - len0) * D + e];
        vx[u][e] = vn[(int64_t)(t + u - len0) * D + e];
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kd[(int64_t)(t + u) * D + e] = kx[u][e];
        vd[(int64_t)(t + u) * D + e] = vx[u][e];
        acc[e] = g.kmax ? fmaxf(acc[e], (float)kx[u][e]) : acc[e] + (float)kx[u][e];
      }
  }
  for (; t < t1; ++t) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const T kx = kn[(int64_t)(t - len0) * D + e];
      const T vx = vn[(int64_t)(t - len0) * D + e];
      kd[(int64_t)t * D + e] = kx;
      vd[(int64_t)t * D + e] = vx;
      acc[e] = g.kmax ? fmaxf(acc[e], (float)kx) : acc[e] + (float)kx;
    }
  }
  float* c = summ + ((int64_t)s * g.sum_seq + (int64_t)h * g.sum_head + j) * D + col;
  const float inv = 1.f / (float)(r_old + t1 - t0);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (g.kmax) {
      c[e] = r_old > 0 ? fmaxf(c[e], acc[e]) : acc[e];
    } else {
      const float sum = r_old > 0 ? fmaf((float)r_old, c[e], acc[e]) : acc[e];
      c[e] = sum * inv;
    }
  }
}

int launch_append_kv(const AppendGeom& g, int dtype, int n_seq, int touched, const void* k_new,
                     const void* v_new, void* k_cache, void* v_cache, float* summ, hipStream_t st) {
  const dim3 grid((unsigned)(n_seq * g.hkv), (unsigned)touched);
  if (dtype == SA_BF16) {
    if (g.d == 128)
      append_kv_kernel<__bf16, 2><<<grid, 64, 0, st>>>(g, (const __bf16*)k_new, (const __bf16*)v_new,
                                                       (__bf16*)k_cache, (__bf16*)v_cache, summ);
    else
      append_kv_kernel<__bf16, 1><<<grid, 64, 0, st>>>(g, (const __bf16*)k_new, (const __bf16*)v_new,
                                                       (__bf16*)k_cache, (__bf16*)v_cache, summ);
  } else {
    if (g.d == 128)
      append_kv_kernel<float, 2><<<grid, 64, 0, st>>>(g, (const float*)k_new, (const float*)v_new,
                                                      (float*)k_cache, (float*)v_cache, summ);
    else
      append_kv_kernel<float, 1><<<grid, 64, 0, st>>>(g, (const float*)k_new, (const float*)v_new,
                                                      (float*)k_cache, (float*)v_cache, summ);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
