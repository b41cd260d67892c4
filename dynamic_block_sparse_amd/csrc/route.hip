// Routing kernels: block summaries, pooled query scores and per-row selection.
//
// [P2] §2.1 Eq 6: c_j = mean of block j's keys, g_rj = pool over the queries of
// block r of q . c_j.  [P2] Eq 7: clipped threshold count.  [P2] §2.1 "causal
// boundary" / §4.1: only complete history blocks are scored; the current block
// is a fixed branch.  [P2] §4: shared GQA routing averages over the head group.
// [P1] (top-k of long candidate lists): select without materialising a sort,
// with a stable rule for equal scores (lower block id first).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace sa {

// Route row of (sequence s, routing head h, query block r): the inverse of
// decode_row for prefill rows.
__device__ __forceinline__ int64_t prefill_row_index(const Geom& g, int s, int h, int r, int blk0, int nblk) {
  if (g.varlen) return (int64_t)g.hr * blk0 + (int64_t)h * nblk + r;
  return ((int64_t)s * g.hr + h) * (nblk - g.qblk0) + (r - g.qblk0);   // rows from query block qblk0
}

// ---------------------------------------------------------------------------
// Block summaries.  One wavefront per (sequence, kv head, key block): lanes own
// an 8-element column chunk and a key phase, so every load is a 16-byte (bf16)
// or 32-byte (fp32) piece of a contiguous 64 x d tile; phases are summed with
// cross-lane shuffles.  Padding tokens past the sequence end never enter the
// sum, and a partial block divides by its own count.
// With `qbar`, grid rows hkv .. hkv + hr - 1 pool the queries the same way in
// the same pass ([P2] Eq 6 mean pooling): the wavefront of (sequence, routing
// head h, query block r) averages the block's valid queries over the row's
// query heads (the KV head's group when routing is shared) and writes the
// route row's pooled vector to qbar[row][0 .. d).
template <typename T, int D>
__global__ void __launch_bounds__(256) summary_kernel(Geom g, const T* __restrict__ k,
                                                      float* __restrict__ summ, int slots,
                                                      const T* __restrict__ q, float* __restrict__ qbar,
                                                      int kpool) {
  constexpr int CH = D / 8;        // column chunks per row
  constexpr int PH = kWave / CH;   // key phases per wave
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int slot = blockIdx.x * 4 + wave;
  const bool pool_q = (int)blockIdx.y >= g.hkv;
  const int h = pool_q ? (int)blockIdx.y - g.hkv : (int)blockIdx.y;
  if (slot >= slots) return;
  int s, j, tok0 = 0, blk0 = 0, len;
  if (g.varlen) {
    int lo = 0, hi = g.batch - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (g.cu_blocks[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    s = lo;
    blk0 = g.cu_blocks[s];
    j = slot - blk0;
    tok0 = g.cu_seqlens[s];
    len = g.cu_seqlens[s + 1] - tok0;
  } else {
    const int nb = ceil_div(g.n, kBlock);
    s = slot / nb;
    j = slot % nb;
    len = g.mode == SA_DECODE ? decode_len(g, s) : g.n;
    if (j * kBlock >= len) return;   // past a shorter decode sequence's last block
  }
  if (pool_q && j < g.qblk0) return;   // a cached prefix block has no queries (chunked prefill)
  const int cnt = min(kBlock, len - j * kBlock);
  const int c = lane % CH, ph = lane / CH;
  // max-pooled key summaries keep each dimension's maximum over the block's
  // valid keys; block means (and pooled queries) sum and divide
  const bool kmax = !pool_q && kpool == SA_POOL_MAX;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = kmax ? -INFINITY : 0.f;
  const int nh = pool_q ? g.hpr : 1;   // query heads pooled into the row
  const int h0 = g.share ? h * g.group : h;
  const T* base = pool_q ? q + q_offset(g, s, h0, tok0, j * kBlock) + c * 8
                         : k + kv_block_offset(g, s, h, tok0, j) + c * 8;
  auto add_row = [&](int t) {
    const T* p = base + (int64_t)t * D;
    float x[8];
    if constexpr (sizeof(T) == 2) {
      u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(u[i]);
        x[2 * i + 1] = bf16_hi(u[i]);
      }
    } else {
      f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
      f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = x0[i];
        x[4 + i] = x1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = kmax ? fmaxf(acc[i], x[i]) : acc[i] + x[i];
  };
  for (int hh = 0; hh < nh; ++hh) {
    if (cnt == kBlock) {
      // full block: every row's load is issued before the sums need them
#pragma unroll
      for (int t = 0; t < kBlock / PH; ++t) add_row(ph + t * PH);
    } else {
      for (int t = ph; t < cnt; t += PH) add_row(t);
    }
    base += g.q_head;   // next query head of the group (only read when pooling queries)
  }
  // combine the key phases: partners lane ^ 8 (D = 64 only), ^ 16, ^ 32
  auto combine = [&](auto op) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t u = __float_as_uint(acc[i]);
      if constexpr (CH <= 8) u = op(u, dpp_u<0x128>(u));   // row_ror:8 = lane ^ 8 in a 16-lane row
      u = pair32(pair16(u, op), op);
      acc[i] = __uint_as_float(u);
    }
  };
  if (kmax)
    combine(OpMaxF{});
  else
    combine(OpAddF{});
  if (ph == 0) {
    const float inv = kmax ? 1.f : 1.f / (float)(cnt * nh);
    const int nblk = g.varlen ? g.cu_blocks[s + 1] - blk0 : ceil_div(g.n, kBlock);
    float* out = pool_q ? qbar + prefill_row_index(g, s, h, j, blk0, nblk) * D + c * 8
                        : summ + sum_offset(g, s, h, blk0, j) + c * 8;
    f32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o0[i] = acc[i] * inv;
      o1[i] = acc[4 + i] * inv;
    }
    *reinterpret_cast<f32x4*>(out) = o0;
    *reinterpret_cast<f32x4*>(out + 4) = o1;
  }
}

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);   // -0 -> +0 so equal values share a key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Per-row routing context: candidates are the complete history blocks j < r
// (decode: j < N-1) other than the forced ones; candidate i is block start + i.
// Forced: the local window lo .. cur (lo = max(cur - W + 1, 0)) and, with
// SA_FORCE_FIRST, block 0; the candidates are then the contiguous range
// [start, lo) with start = 1 when block 0 is forced outside the window.
struct RouteRow {
  RowInfo ri;
  int kvh, h0, qt0, nq, cur, lo, start, nc, nforced;
  bool ff;
};

__device__ __forceinline__ RouteRow route_row(const Geom& g, const sa_route_cfg& rc, int64_t row) {
  RouteRow w;
  w.ri = decode_row(g, row);
  w.kvh = g.share ? w.ri.h : w.ri.h / g.group;
  w.h0 = g.share ? w.ri.h * g.group : w.ri.h;
  if (g.mode == SA_DECODE) {
    w.qt0 = 0;
    w.nq = 1;
  } else {
    w.qt0 = w.ri.r * kBlock;
    w.nq = min(kBlock, w.ri.len - w.qt0);
  }
  w.cur = w.ri.r;   // decode: the last cached block
  w.ff = (rc.forced & SA_FORCE_FIRST) != 0;
  w.lo = max(w.cur - max(rc.window, 1) + 1, 0);   // first block of the local window
  w.start = (w.ff && w.lo > 0) ? 1 : 0;
  w.nc = max(w.lo - w.start, 0);
  w.nforced = (w.cur - w.lo + 1) + ((w.ff && w.lo > 0) ? 1 : 0);
  return w;
}

// ---------------------------------------------------------------------------
// Prefill scores under mean pooling, as tiles of the product Qbar C^T of one
// (sequence, routing head) ([P2] Eq 6: g_rj = qbar_r . c_j for j < r): a
// workgroup takes kScoreRows query blocks x kScoreCols key blocks, stages
// the pooled queries (from the summary pass) and the summaries in LDS (every
// load issued before the first store), and each thread accumulates 2-8 dot
// products in fp32.  Scored per row instead, every summary is read once per
// later query block (O(N^2 d) reads from L2); here once per tile row.  (Up to
// 256 key blocks per sequence, route_tile_select_kernel scores and selects
// in one pass instead.)
// Scores land in scores[row * max_blocks + (j - start_r)] for the row's
// candidates j (start_r = 1 when block 0 is forced and r > 0).
template <int D, int kScoreRows, int kScoreCols>
__global__ void __launch_bounds__(256) route_score_tile_kernel(Geom g, sa_route_cfg rc,
                                                               const float* __restrict__ qbar,
                                                               const float* __restrict__ summ,
                                                               float* __restrict__ scores) {
  constexpr int LD = D + 4;   // row pitch in floats
  constexpr int QV = kScoreRows * D / 4 / 256, CV = kScoreCols * D / 4 / 256;   // float4 per thread
  __shared__ __attribute__((aligned(16))) float qs[kScoreRows * LD];
  __shared__ __attribute__((aligned(16))) float cs[kScoreCols * LD];
  const int s = blockIdx.z / g.hr, h = blockIdx.z % g.hr;
  int blk0 = 0, nblk;
  if (g.varlen) {
    blk0 = g.cu_blocks[s];
    nblk = g.cu_blocks[s + 1] - blk0;
  } else {
    nblk = ceil_div(g.n, kBlock);
  }
  const int r0 = g.qblk0 + blockIdx.x * kScoreRows, j0 = blockIdx.y * kScoreCols;
  // candidates satisfy j < r <= r0 + kScoreRows - 1: tiles above the diagonal have none
  if (r0 >= nblk || j0 > r0 + kScoreRows - 2) return;   // uniform
  const int kvh = g.share ? h : h / g.group;
  // rows of (s, h) are row0 + r for its query blocks r >= qblk0
  const int64_t row0 = prefill_row_index(g, s, h, g.qblk0, blk0, nblk) - g.qblk0;
  const float* cbase = summ + sum_offset(g, s, kvh, blk0, 0);
  const int tid = threadIdx.x;
  // stage (rows past the end: clamped copies, never written out)
  f32x4 qv4[QV], cv4[CV];
#pragma unroll
  for (int u = 0; u < QV; ++u) {
    const int e = tid + 256 * u, rr = e / (D / 4), k4 = e % (D / 4);
    qv4[u] = *reinterpret_cast<const f32x4*>(qbar + (row0 + min(r0 + rr, nblk - 1)) * D + 4 * k4);
  }
#pragma unroll
  for (int u = 0; u < CV; ++u) {
    const int e = tid + 256 * u, jj = e / (D / 4), k4 = e % (D / 4);
    cv4[u] = *reinterpret_cast<const f32x4*>(cbase + (int64_t)min(j0 + jj, nblk - 1) * D + 4 * k4);
  }
#pragma unroll
  for (int u = 0; u < QV; ++u) {
    const int e = tid + 256 * u;
    *reinterpret_cast<f32x4*>(qs + (e / (D / 4)) * LD + 4 * (e % (D / 4))) = qv4[u];
  }
#pragma unroll
  for (int u = 0; u < CV; ++u) {
    const int e = tid + 256 * u;
    *reinterpret_cast<f32x4*>(cs + (e / (D / 4)) * LD + 4 * (e % (D / 4))) = cv4[u];
  }
  __syncthreads();
  constexpr int RA = kScoreRows * kScoreCols / 256 >= 2 && kScoreRows >= 32 ? 2 : 1;   // rows per thread
  constexpr int CB = kScoreRows * kScoreCols / 256 / RA;                              // columns per thread
  constexpr int CG = kScoreCols / CB;                                                 // column groups
  // rows RA rg ..; columns cg, cg + CG, ...: the 16 lanes of a column group
  // set read 16 consecutive summary rows, whose 16-byte slices fall in
  // distinct LDS banks at the 132-float pitch (contiguous columns per thread
  // put rows 4 apart on the same banks)
  const int rg = tid / CG, cg = tid % CG;
  float acc[RA][CB];
#pragma unroll
  for (int a = 0; a < RA; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b) acc[a][b] = 0.f;
#pragma unroll 4
  for (int k = 0; k < D; k += 4) {
    f32x4 qv[RA], cv[CB];
#pragma unroll
    for (int a = 0; a < RA; ++a) qv[a] = *reinterpret_cast<const f32x4*>(qs + (RA * rg + a) * LD + k);
#pragma unroll
    for (int b = 0; b < CB; ++b) cv[b] = *reinterpret_cast<const f32x4*>(cs + (cg + CG * b) * LD + k);
#pragma unroll
    for (int a = 0; a < RA; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][b] = __builtin_fmaf(qv[a][i], cv[b][i], acc[a][b]);
  }
  const bool ff = (rc.forced & SA_FORCE_FIRST) != 0;
#pragma unroll
  for (int a = 0; a < RA; ++a) {
    const int r = r0 + RA * rg + a;
    if (r >= nblk) continue;
    const int start = (ff && r > 0) ? 1 : 0;
    float* srow = scores + (row0 + r) * (int64_t)g.max_blocks;
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int j = j0 + cg + CG * b;
      if (j >= start && j < r) srow[j - start] = acc[a][b];
    }
  }
}

// Decode rows (few, with long histories) split their candidates into chunks
// of kDecodeChunk, one workgroup each; prefill rows are many and take one.
constexpr int kDecodeChunk = 512;

// ---------------------------------------------------------------------------
// Routing scores: one 256-thread workgroup per (worklist row, chunk of
// `chunk` candidates).
//   mean pool: one pooled vector over the row's query heads and valid
//     queries, dotted with every candidate summary;
//   max pool: per-query scores, max over the block's queries, mean over heads.
// Scores land in scores[row * max_blocks + i] for candidate i.
template <typename T, int D, int U>
__global__ void __launch_bounds__(256) route_score_kernel(Geom g, sa_route_cfg rc, const T* __restrict__ q,
                                                          const float* __restrict__ summ,
                                                          float* __restrict__ scores, int chunk) {
  extern __shared__ float smem[];
  float* qbar = smem;          // [D]
  float* red = qbar + D;       // [16 * D] phase partials / max-pool rows

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.x;
  const RouteRow w = route_row(g, rc, row);
  const int c0 = blockIdx.y * chunk, c1 = min(w.nc, c0 + chunk);
  if (c0 >= c1) return;   // uniform: the whole workgroup leaves
  const int nh = g.hpr;
  const float* cbase = summ + sum_offset(g, w.ri.s, w.kvh, w.ri.blk0, 0);
  float* srow = scores + row * (int64_t)g.max_blocks;

  if (rc.qpool == SA_POOL_MEAN) {
    // ---- mean pool over (head, query) pairs
    constexpr int CH = D / 8, PH = 256 / CH;
    const int c = tid % CH, ph = tid / CH;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    const int items = nh * w.nq;
    // UP items per thread are loaded before any is added (clamped to a
    // valid item, weight 0 past the end), so a row's pooled query costs one
    // memory round trip per UP items rather than one per item
    constexpr int UP = 8;
    for (int it0 = ph; it0 < items; it0 += PH * UP) {
      if constexpr (sizeof(T) == 2) {
        u32x4 x[UP];
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int it = min(it0 + u * PH, items - 1);
          const int hh = w.h0 + it / w.nq, t = it % w.nq;
          x[u] = *reinterpret_cast<const u32x4*>(q + q_offset(g, w.ri.s, hh, w.ri.tok0, w.qt0 + t) + c * 8);
        }
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const float wgt = it0 + u * PH < items ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wgt * bf16_lo(x[u][i]);
            acc[2 * i + 1] += wgt * bf16_hi(x[u][i]);
          }
        }
      } else {
        f32x4 x0[UP], x1[UP];
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int it = min(it0 + u * PH, items - 1);
          const int hh = w.h0 + it / w.nq, t = it % w.nq;
          const T* p = q + q_offset(g, w.ri.s, hh, w.ri.tok0, w.qt0 + t) + c * 8;
          x0[u] = *reinterpret_cast<const f32x4*>(p);
          x1[u] = *reinterpret_cast<const f32x4*>(p + 4);
        }
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const float wgt = it0 + u * PH < items ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i] += wgt * x0[u][i];
            acc[4 + i] += wgt * x1[u][i];
          }
        }
      }
    }
    // two 16-byte stores per lane (eight 4-byte ones at a 32-byte lane stride
    // conflicted ~12 cycles per LDS instruction)
    *reinterpret_cast<f32x4*>(red + ph * D + c * 8) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(red + ph * D + c * 8 + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    if (tid < D) {
      float sacc = 0.f;
      for (int p2 = 0; p2 < PH; ++p2) sacc += red[p2 * D + tid];
      qbar[tid] = sacc / (float)items;
    }
    __syncthreads();
    // ---- scores: LPC lanes cooperate on one candidate (4 floats each).
    // U candidates per lane group are loaded before any is reduced, so a
    // wavefront keeps U x 1 KB of summary reads in flight (U = 16 for the
    // long, HBM-resident decode histories; 8 for prefill rows, whose
    // summaries are shared through L2 and whose candidate lists are short).
    constexpr int LPC = D / 4, CPS = kWave / LPC;
    const int cl = lane % LPC, cw = lane / LPC;
    const f32x4 qv = *reinterpret_cast<const f32x4*>(qbar + cl * 4);
    for (int base = c0 + wave * CPS; base < c1; base += 4 * CPS * U) {
      float part[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // unconditional load of a clamped candidate: a guarded load would be
        // waited for before the next one is issued
        const int ci = base + u * 4 * CPS + cw;
        const int cc = min(ci, c1 - 1);
        const f32x4 cv = *reinterpret_cast<const f32x4*>(cbase + (int64_t)(w.start + cc) * D + cl * 4);
        part[u] = (qv[0] * cv[0] + qv[1] * cv[1] + qv[2] * cv[2] + qv[3] * cv[3]) * (ci < c1 ? 1.f : 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ci = base + u * 4 * CPS + cw;
        static_assert(LPC == 32 || LPC == 16, "lanes per candidate");
        float x = part[u];
        x = LPC == 32 ? half_sum(x) : __uint_as_float(row16_reduce(__float_as_uint(x), OpAddF{}));
        if (cl == 0 && ci < c1) srow[ci] = x;
      }
    }
  } else {
    // ---- max pool: per-query scores, max over the block's queries, mean over
    // heads.  Each wavefront owns candidates c0 + wave, +4, ..., accumulated
    // over heads in registers (lane 0).
    constexpr int LD = D + 1;
    const int nmine = (c1 - c0 - wave + 3) / 4;
    for (int hh = 0; hh < nh; ++hh) {
      __syncthreads();
      for (int e = tid; e < w.nq * D; e += 256) {
        const int t = e / D, dd = e % D;
        red[t * LD + dd] = to_f32<T>(q[q_offset(g, w.ri.s, w.h0 + hh, w.ri.tok0, w.qt0 + t) + dd]);
      }
      __syncthreads();
      for (int k = 0; k < nmine; ++k) {
        const int ci = c0 + wave + 4 * k;
        const float* cj = cbase + (int64_t)(w.start + ci) * D;
        float dot = 0.f;
        if (lane < w.nq) {
          for (int dd = 0; dd < D; ++dd) dot += red[lane * LD + dd] * cj[dd];
        } else {
          dot = -INFINITY;
        }
        dot = wave_max(dot);
        if (lane == 0) srow[ci] = (hh == 0 ? 0.f : srow[ci]) + dot / (float)nh;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection: one wavefront per worklist row; the row's candidate scores sit
// in registers as order-preserving keys (E per lane, candidate lane + 64 e).
//   1. budget: top-k, or Eq 7's clipped count of scores >= max - tau_rel;
//   2. the D-th largest key T, built bit by bit from the MSB as the largest
//      value with #(key >= T) >= D (ballot counts, no LDS, no barriers);
//   3. picks = keys > T plus the lowest-id keys == T, written in ascending id
//      order from ballot prefix counts; forced blocks first, -1 padding last.
// Empty key slots hold 0, which no threshold with a set bit counts.
// The J row of a selection: forced ids first (the sink when outside the
// window, then the window ascending), then the picks in ascending id order
// (keys above thr, and the take_eq lowest-id keys equal to it; every valid
// key when take_all), then -1.  key[e] is candidate lane + 64 e's
// order-preserving key.
template <int E>
__device__ __forceinline__ void emit_row(const sa_route_cfg& rc, const RouteRow& w, int64_t row, const uint32_t (&key)[E],
                                         int dsel, bool take_all, uint32_t thr, int take_eq,
                                         int32_t* __restrict__ J, int lane) {
  int32_t* jrow = J + row * rc.k_b;
  if (lane <= w.cur - w.lo) {
    const int k0 = (w.ff && w.lo > 0) ? 1 : 0;
    if (lane == 0 && k0) jrow[0] = 0;
    jrow[k0 + lane] = w.lo + lane;
  }
  if (dsel > 0) {
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane + 64 * e;
      const bool valid = i < w.nc;
      const bool eq = !take_all && valid && key[e] == thr;
      const uint64_t beq = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(beq & below);
      const bool take = valid && (take_all || key[e] > thr || (eq && eq_rank < take_eq));
      const uint64_t bt = __ballot(take);
      if (take) jrow[w.nforced + pos + __popcll(bt & below)] = w.start + i;
      pos += __popcll(bt);
      eq_seen += __popcll(beq);
    }
  }
  for (int i = w.nforced + dsel + lane; i < rc.k_b; i += 64) jrow[i] = -1;
}

// The selection of one row by one wavefront (lane = its lane id); srow holds
// the row's candidate scores (global memory or LDS).
template <int E, typename Scores>
__device__ __forceinline__ void select_row(const sa_route_cfg& rc, const RouteRow& w, int64_t row, Scores srow,
                                           int32_t* __restrict__ J, int lane) {
  // Every load is issued unconditionally (clamped to a valid slot) and the
  // guard applies to the value: a load under a per-slot branch is waited for
  // before the next branch, which serialises E memory round trips.
  uint32_t key[E];
  float mx = -INFINITY;
  const int last = max(w.nc - 1, 0);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;
    const float x = srow[min(i, last)];
    const bool ok = i < w.nc;
    key[e] = order_key(x) & (ok ? 0xffffffffu : 0u);   // masks, not a branch
    mx = fmaxf(mx, ok ? x : -INFINITY);
  }
  // #(key >= x) over the row: lane counts in four independent chains, then
  // one wave sum
  auto count_ge = [&](uint32_t x) {
    int c[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < E; ++e) c[e & 3] += key[e] >= x ? 1 : 0;
    return wave_sum_i((c[0] + c[1]) + (c[2] + c[3]));
  };

  int kr = rc.k_b;
  uint32_t k0 = 0u;   // Eq 7's threshold as a key, and the candidates at or above it
  int above = -1;
  if (rc.select == SA_SELECT_THRESHOLD) {
    mx = wave_max(mx);
    k0 = order_key(mx - rc.tau_rel);
    above = w.nc > 0 ? count_ge(k0) : 0;
    kr = min(rc.k_b, max(rc.k_min, w.nforced + above));
  }
  const int dsel = min(max(kr - w.nforced, 0), w.nc);
  const bool take_all = (dsel == w.nc);
  uint32_t thr = 0u;
  int take_eq = 0;
  if (!take_all && dsel > 0 && dsel == above && k0 > 0u) {
    // neither k_b nor k_min binds: the picks are exactly the candidates at or
    // above Eq 7's threshold (the dsel-th largest key T is >= k0 and exactly
    // dsel keys are >= T), so no search: keys > k0 - 1, none taken by equality
    thr = k0 - 1u;
    take_eq = 0;
  } else if (!take_all && dsel > 0) {
    // T lies in [kmin, kmax]: the bits above their highest difference are
    // common to every candidate key and need no search
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (lane + 64 * e < w.nc) {
        kmin = min(kmin, key[e]);
        kmax = max(kmax, key[e]);
      }
    }
    kmin = wave_min_u(kmin);
    kmax = wave_max_u(kmax);
    const uint32_t diff = kmin ^ kmax;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    uint32_t t = top < 0 ? kmax : top >= 31 ? 0u : (kmax & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (count_ge(cand) >= dsel) t = cand;
    }
    thr = t;
    take_eq = dsel - (t == 0xffffffffu ? 0 : count_ge(t + 1u));
  }

  emit_row<E>(rc, w, row, key, dsel, take_all, thr, take_eq, J, lane);
}

// The selection of one row by one wavefront over scores in memory (global
// memory or LDS), for rows longer than select_row holds in registers (more
// than 8192 candidates).  Same budget, same rule and the same picks as
// select_row: Eq 7's count from the row maximum; then the budget-th largest
// order-preserving key T, found one 8-bit digit at a time from the top with
// a 256-bin histogram in LDS (`hist`, this wavefront's own); then the picks
// in ascending id order, 64 candidates at a time.
template <typename Scores>
__device__ __forceinline__ void select_row_mem(const sa_route_cfg& rc, const RouteRow& w, int64_t row, Scores srow,
                                            int32_t* __restrict__ J, int lane, uint32_t* hist) {
  const int nc = w.nc;
  auto key_at = [&](int i) { return order_key(srow[i]); };
  auto count_ge = [&](uint32_t x) {
    int c = 0;
    for (int i = lane; i < nc; i += kWave) c += key_at(i) >= x ? 1 : 0;
    return wave_sum_i(c);
  };
  int kr = rc.k_b;
  uint32_t k0 = 0u;
  int above = -1;
  if (rc.select == SA_SELECT_THRESHOLD) {
    float mx = -INFINITY;
    for (int i = lane; i < nc; i += kWave) mx = fmaxf(mx, srow[i]);
    mx = wave_max(mx);
    k0 = order_key(mx - rc.tau_rel);
    above = nc > 0 ? count_ge(k0) : 0;
    kr = min(rc.k_b, max(rc.k_min, w.nforced + above));
  }
  const int dsel = min(max(kr - w.nforced, 0), nc);
  const bool take_all = dsel == nc;
  uint32_t thr = 0u;
  int need = dsel;
  if (!take_all && dsel > 0 && dsel == above && k0 > 0u) {
    thr = k0 - 1u;   // the candidates at or above Eq 7's threshold (see select_row)
    need = 0;
  } else if (!take_all && dsel > 0) {
    uint32_t pmask = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = lane; b < 256; b += kWave) hist[b] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < nc; i += kWave) {
        const uint32_t k = key_at(i);
        if ((k & pmask) == thr) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      // lane l holds bins 255 - 4l .. 252 - 4l (the largest digits first)
      int c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = (int)hist[255 - 4 * lane - j];
        tot += c[j];
      }
      const int incl = wave_incl_scan_i(tot), excl = incl - tot;
      const uint64_t reach = __ballot(incl >= need);   // some lane reaches need: need <= matching keys
      const int owner = __ffsll((unsigned long long)reach) - 1;
      int run = excl, bin = 255 - 4 * lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run + c[j] >= need) {
          bin = 255 - 4 * lane - j;
          break;
        }
        run += c[j];
      }
      const int bin_o = __builtin_amdgcn_readlane(bin, owner);
      const int run_o = __builtin_amdgcn_readlane(run, owner);
      thr |= (uint32_t)bin_o << shift;
      need -= run_o;
      pmask |= 255u << shift;
      __builtin_amdgcn_wave_barrier();   // every lane has read the histogram before the next clear
    }
  }
  int32_t* jrow = J + row * rc.k_b;
  if (lane <= w.cur - w.lo) {   // forced blocks first: the sink outside the window, then the window
    const int kf = (w.ff && w.lo > 0) ? 1 : 0;
    if (lane == 0 && kf) jrow[0] = 0;
    jrow[kf + lane] = w.lo + lane;
  }
  if (dsel > 0) {
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = w.nforced, eq_seen = 0;
    for (int base = 0; base < nc; base += kWave) {
      const int i = base + lane;
      const bool valid = i < nc;
      const uint32_t k = valid ? key_at(i) : 0u;
      const bool eq = valid && !take_all && k == thr;
      const uint64_t beq = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(beq & below);
      const bool take = valid && (take_all || k > thr || (eq && eq_rank < need));
      const uint64_t bt = __ballot(take);
      if (take) jrow[pos + __popcll(bt & below)] = w.start + i;
      pos += __popcll(bt);
      eq_seen += __popcll(beq);
    }
  }
  for (int i = w.nforced + dsel + lane; i < rc.k_b; i += kWave) jrow[i] = -1;
}

// Rows with more than 8192 candidates: one wavefront per row over its scores
// in the route workspace.
__global__ void __launch_bounds__(64) route_select_mem_kernel(Geom g, sa_route_cfg rc,
                                                              const float* __restrict__ scores,
                                                              int32_t* __restrict__ J) {
  __shared__ uint32_t hist[256];
  const int64_t row = blockIdx.x;
  const RouteRow w = route_row(g, rc, row);
  select_row_mem(rc, w, row, scores + row * (int64_t)g.max_blocks, J, (int)threadIdx.x, hist);
}

template <int E>
__global__ void __launch_bounds__(64) route_select_kernel(Geom g, sa_route_cfg rc, const float* __restrict__ scores,
                                                          int32_t* __restrict__ J) {
  const int64_t row = blockIdx.x;
  const RouteRow w = route_row(g, rc, row);
  select_row<E>(rc, w, row, scores + row * (int64_t)g.max_blocks, J, (int)threadIdx.x);
}

// ---------------------------------------------------------------------------
// Prefill routing under mean pooling when every sequence has at most NC key
// blocks: scores and selection in one pass.  A workgroup of R wavefronts
// takes R query blocks of one (sequence, routing head) and all NC key
// blocks: it stages their pooled queries and the summaries in LDS, and
// wavefront w then scores query block r0 + w against every key block (lane l
// takes blocks l + 64 b: consecutive lanes read consecutive summary rows,
// disjoint banks at the 132-float pitch), parks the scores in its own LDS
// row and selects that row with select_row.  The same scores ([P2] Eq 6, fp32
// dot products of the same operands in the same order as the tile kernel)
// and the same picks as the score and select launches, without the scores'
// round trip through memory and the second launch.
template <int D, int NC, int R>
__global__ void __launch_bounds__(R * 64) route_tile_select_kernel(Geom g, sa_route_cfg rc,
                                                                 const float* __restrict__ qbar,
                                                                 const float* __restrict__ summ,
                                                                 int32_t* __restrict__ J) {
  constexpr int NT = R * kWave, LD = D + 4, E = NC / kWave;
  constexpr int QV = (R * D / 4 + NT - 1) / NT, CV = NC * D / 4 / NT;   // float4 per thread
  __shared__ __attribute__((aligned(16))) float qs[R * LD];
  __shared__ __attribute__((aligned(16))) float cs[NC * LD];
  __shared__ float sc[R][NC];
  const int s = blockIdx.z / g.hr, h = blockIdx.z % g.hr;
  int blk0 = 0, nblk;
  if (g.varlen) {
    blk0 = g.cu_blocks[s];
    nblk = g.cu_blocks[s + 1] - blk0;
  } else {
    nblk = ceil_div(g.n, kBlock);
  }
  const int r0 = g.qblk0 + (int)blockIdx.x * R;
  if (r0 >= nblk) return;   // uniform
  const int kvh = g.share ? h : h / g.group;
  const int64_t row0 = prefill_row_index(g, s, h, g.qblk0, blk0, nblk) - g.qblk0;
  const float* cbase = summ + sum_offset(g, s, kvh, blk0, 0);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  // stage (rows past the end: clamped copies, never selected)
  f32x4 qv4[QV], cv4[CV];
#pragma unroll
  for (int u = 0; u < QV; ++u) {
    const int e = min(tid + NT * u, R * D / 4 - 1), rr = e / (D / 4), k4 = e % (D / 4);
    qv4[u] = *reinterpret_cast<const f32x4*>(qbar + (row0 + min(r0 + rr, nblk - 1)) * D + 4 * k4);
  }
#pragma unroll
  for (int u = 0; u < CV; ++u) {
    const int e = tid + NT * u, jj = e / (D / 4), k4 = e % (D / 4);
    cv4[u] = *reinterpret_cast<const f32x4*>(cbase + (int64_t)min(jj, nblk - 1) * D + 4 * k4);
  }
#pragma unroll
  for (int u = 0; u < QV; ++u) {
    const int e = tid + NT * u;
    if (e < R * D / 4) *reinterpret_cast<f32x4*>(qs + (e / (D / 4)) * LD + 4 * (e % (D / 4))) = qv4[u];
  }
#pragma unroll
  for (int u = 0; u < CV; ++u) {
    const int e = tid + NT * u;
    *reinterpret_cast<f32x4*>(cs + (e / (D / 4)) * LD + 4 * (e % (D / 4))) = cv4[u];
  }
  __syncthreads();
  const int r = r0 + wave;
  if (r >= nblk) return;   // no barrier follows
  float acc[E];
#pragma unroll
  for (int b = 0; b < E; ++b) acc[b] = 0.f;
#pragma unroll 4
  for (int k = 0; k < D; k += 4) {
    const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + wave * LD + k);
#pragma unroll
    for (int b = 0; b < E; ++b) {
      const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + (lane + kWave * b) * LD + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b] = __builtin_fmaf(qv[i], cv[i], acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < E; ++b) sc[wave][lane + kWave * b] = acc[b];
  const int64_t row = row0 + r;
  const RouteRow w = route_row(g, rc, row);
  select_row<E>(rc, w, row, (const float*)&sc[wave][w.start], J, lane);
}

// ---------------------------------------------------------------------------
// Decode routing in one pass per row ([P2] §3.1: the summaries are cache
// state, and a decode step's router scans each stored summary of the row once;
// [P2] §2.2: decode cost is reading history).  One workgroup of 256 threads per
// (sequence, routing head), so that the rows of a decode batch (512 at 64
// sequences x 8 KV heads, ~130 registers a lane) are resident at once: the mean of the row's query heads' queries (one
// each), then every candidate summary dotted with it, LPC lanes per summary
// with 16-byte loads, each wavefront keeping U loads in flight (every slot is
// refilled as soon as it is consumed); the scores stay in LDS.  Top-k rows
// are selected by the whole workgroup (a radix select over the scores'
// order-preserving keys), threshold rows by select_row; both emit the same
// picks as route_select_kernel.
template <typename T, int D, int E>
__global__ void __launch_bounds__(256) route_decode_kernel(Geom g, sa_route_cfg rc, const T* __restrict__ q,
                                                           const float* __restrict__ summ,
                                                           int32_t* __restrict__ J) {
  constexpr int NWV = 4, U = 16;
  constexpr int LPC = D / 4, CPL = kWave / LPC;   // lanes per candidate, candidates per wave load
  extern __shared__ float smem[];
  float* const qbar = smem;                        // [D]
  float* const sc = smem + D;                      // [max_blocks] candidate scores
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.x;
  const RouteRow w = route_row(g, rc, row);
  const int cl = lane % LPC, cw = lane / LPC;
  const float* cbase = summ + sum_offset(g, w.ri.s, w.kvh, w.ri.blk0, w.start) + cl * 4;
  const int nc = w.nc, last = max(nc - 1, 0);
  constexpr int kPerIter = NWV * U * CPL;          // candidates per workgroup iteration
  // candidate of load u in iteration it for this lane
  auto cand = [&](int it, int u) { return it * kPerIter + (u * NWV + wave) * CPL + cw; };
  // U loads in flight per wavefront: slot u is consumed and at once refilled
  // with its candidate of the next iteration (unconditional, clamped loads);
  // the first ones go out before the query pooling
  auto load = [&](int it, int u) {
    return *reinterpret_cast<const f32x4*>(cbase + (int64_t)min(cand(it, u), last) * D);
  };
  const int iters = (nc + kPerIter - 1) / kPerIter;
  f32x4 buf[U];
  if (iters > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) buf[u] = load(0, u);
  }
  if (tid < D) {   // mean over the row's query heads, summed in head order
    float acc = 0.f;
    for (int hh = 0; hh < g.hpr; ++hh) acc += to_f32<T>(q[q_offset(g, w.ri.s, w.h0 + hh, 0, 0) + tid]);
    qbar[tid] = acc / (float)g.hpr;
  }
  __syncthreads();
  const f32x4 qv = *reinterpret_cast<const f32x4*>(qbar + cl * 4);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f32x4 cv = buf[u];
      buf[u] = load(it + 1 < iters ? it + 1 : it, u);
      float x = qv[0] * cv[0] + qv[1] * cv[1] + qv[2] * cv[2] + qv[3] * cv[3];
      static_assert(LPC == 32 || LPC == 16, "lanes per candidate");
      x = LPC == 32 ? half_sum(x) : __uint_as_float(row16_reduce(__float_as_uint(x), OpAddF{}));
      const int c = cand(it, u);
      if (cl == 0 && c < nc) sc[c] = x;
    }
  }
  __syncthreads();
  if constexpr (E > 128) {   // more than 8192 candidates: one wavefront over the scores in LDS
    __shared__ uint32_t hm[256];
    if (wave == 0) select_row_mem(rc, w, row, (const float*)sc, J, lane, hm);
  } else {
    if (rc.select != SA_SELECT_TOPK) {   // Eq 7's threshold count: the one-wavefront selection
      if (wave == 0) select_row<E>(rc, w, row, (const float*)sc, J, lane);
      return;
    }
    // Top-k: the D-th largest order-preserving key T found by the whole
    // workgroup, one 8-bit digit at a time from the top: each pass histograms
    // the digit over the keys that match the digits found so far, and
    // wavefront 0 finds the bin holding the need-th largest of them.  Then
    // need = the number of keys equal to T to take (the lowest ids).
    __shared__ uint32_t hist[2][4][256];   // per pass parity, one per wavefront (fewer same-address atomics)
    __shared__ int pick[2];
    __shared__ int wcnt[4][2];
    const int dsel = min(max(rc.k_b - w.nforced, 0), nc);
    const bool take_all = dsel == nc;
    uint32_t thr = 0u;
    int need = dsel;
    // this thread's keys, candidates tid + 256 k
    constexpr int KPT = (kWave * E + 255) / 256;
    uint32_t kt[KPT];
  #pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int i = tid + 256 * k;
      kt[k] = i < nc ? order_key(sc[i]) : 0u;
    }
    if (!take_all && dsel > 0) {   // uniform over the workgroup
      uint32_t pmask = 0u;
  #pragma unroll
      for (int b = 0; b < 8; ++b) (&hist[0][0][0])[256 * b + tid] = 0u;
      __syncthreads();
      for (int shift = 24, par = 0; shift >= 0; shift -= 8, par ^= 1) {
        uint32_t (&h)[4][256] = hist[par];
  #pragma unroll
        for (int k = 0; k < KPT; ++k)
          if (tid + 256 * k < nc && (kt[k] & pmask) == thr) atomicAdd(&h[wave][(kt[k] >> shift) & 255u], 1u);
        __syncthreads();
        // the other parity's histograms, read in the previous pass, start the next one cleared
  #pragma unroll
        for (int b = 0; b < 4; ++b) hist[par ^ 1][b][tid] = 0u;
        if (wave == 0) {
          // lane l holds bins 255 - 4l .. 252 - 4l (the largest digits first)
          int c[4], tot = 0;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = 255 - 4 * lane - j;
            c[j] = (int)(h[0][b] + h[1][b] + h[2][b] + h[3][b]);
            tot += c[j];
          }
          const int incl = wave_incl_scan_i(tot), excl = incl - tot;
          const uint64_t reach = __ballot(incl >= need);   // some lane reaches need: need <= matching keys
          const int owner = __ffsll((unsigned long long)reach) - 1;
          if (lane == owner) {
            int run = excl, bin = 255 - 4 * lane;
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (run + c[j] >= need) {
                bin = 255 - 4 * lane - j;
                break;
              }
              run += c[j];
            }
            pick[0] = bin;
            pick[1] = need - run;
          }
        }
        __syncthreads();
        thr |= (uint32_t)pick[0] << shift;
        need = pick[1];
        pmask |= 255u << shift;
      }
    }
    if constexpr (E < 4) {
      if (wave == 0) {
        uint32_t key[E];
        const int lastc = max(nc - 1, 0);
  #pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane + 64 * e;
          key[e] = order_key(sc[min(i, lastc)]) & (i < nc ? 0xffffffffu : 0u);
        }
        emit_row<E>(rc, w, row, key, dsel, take_all, thr, need, J, lane);
      }
    } else {
      // the picks in ascending id order, written by all four wavefronts: wave v
      // takes candidates lane + 64 e for e in [EW v, EW v + EW); the picks and
      // the keys equal to T of the waves before it give its first position and
      // the rank of its first key equal to T
      constexpr int EW = E / 4;
      int32_t* jrow = J + row * rc.k_b;
      uint32_t key[EW];
      bool valid[EW];
      int ngt = 0, neq = 0;
  #pragma unroll
      for (int e = 0; e < EW; ++e) {
        const int i = lane + kWave * (EW * wave + e);
        valid[e] = i < nc;
        key[e] = valid[e] ? order_key(sc[i]) : 0u;
        ngt += __popcll(__ballot(valid[e] && (take_all || key[e] > thr)));
        neq += __popcll(__ballot(valid[e] && !take_all && key[e] == thr));
      }
      if (lane == 0) {
        wcnt[wave][0] = ngt;
        wcnt[wave][1] = neq;
      }
      __syncthreads();
      int gtb = 0, eqb = 0;
      for (int v = 0; v < wave; ++v) {
        gtb += wcnt[v][0];
        eqb += wcnt[v][1];
      }
      if (dsel > 0) {
        const uint64_t below = (1ull << lane) - 1ull;
        int pos = w.nforced + gtb + min(eqb, need), eq_seen = eqb;
  #pragma unroll
        for (int e = 0; e < EW; ++e) {
          const int i = lane + kWave * (EW * wave + e);
          const bool eq = valid[e] && !take_all && key[e] == thr;
          const uint64_t beq = __ballot(eq);
          const int eq_rank = eq_seen + __popcll(beq & below);
          const bool take = valid[e] && (take_all || key[e] > thr || (eq && eq_rank < need));
          const uint64_t bt = __ballot(take);
          if (take) jrow[pos + __popcll(bt & below)] = w.start + i;
          pos += __popcll(bt);
          eq_seen += __popcll(beq);
        }
      }
      if (wave == 0) {   // forced blocks first (the sink outside the window, then the window), -1 last
        if (lane <= w.cur - w.lo) {
          const int k0 = (w.ff && w.lo > 0) ? 1 : 0;
          if (lane == 0 && k0) jrow[0] = 0;
          jrow[k0 + lane] = w.lo + lane;
        }
        for (int i = w.nforced + dsel + lane; i < rc.k_b; i += kWave) jrow[i] = -1;
      }
    }
  }
}

size_t route_decode_smem_bytes(const Geom& g) { return (size_t)(g.d + std::max(g.max_blocks, 1)) * sizeof(float); }

// ---------------------------------------------------------------------------
int launch_summary(const Geom& g, int dtype, const void* k, float* summ, int slots, const void* q,
                   float* qbar, int kpool, hipStream_t st) {
  if (slots <= 0) return SA_OK;
  dim3 grid((slots + 3) / 4, g.hkv + (qbar ? g.hr : 0));
  if (dtype == SA_BF16) {
    if (g.d == 128)
      summary_kernel<__bf16, 128><<<grid, 256, 0, st>>>(g, (const __bf16*)k, summ, slots, (const __bf16*)q, qbar,
                                                       kpool);
    else
      summary_kernel<__bf16, 64><<<grid, 256, 0, st>>>(g, (const __bf16*)k, summ, slots, (const __bf16*)q, qbar,
                                                       kpool);
  } else {
    if (g.d == 128)
      summary_kernel<float, 128><<<grid, 256, 0, st>>>(g, (const float*)k, summ, slots, (const float*)q, qbar,
                                                      kpool);
    else
      summary_kernel<float, 64><<<grid, 256, 0, st>>>(g, (const float*)k, summ, slots, (const float*)q, qbar,
                                                      kpool);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

size_t route_smem_bytes(const Geom& g, int qpool) {
  const size_t qb = (size_t)g.d * 4;
  const size_t mean_red = (size_t)(256 / (g.d / 8)) * g.d * 4;   // phase partials
  const size_t max_red = (size_t)kBlock * (g.d + 1) * 4;         // one head's query rows
  return qb + (qpool == SA_POOL_MAX ? max_red : mean_red);
}

size_t route_scores_bytes(const Geom& g) { return (size_t)g.rows * g.max_blocks * sizeof(float); }
size_t route_qbar_bytes(const Geom& g, int qpool) {
  return (g.mode == SA_PREFILL && qpool == SA_POOL_MEAN) ? (size_t)g.rows * g.d * sizeof(float) : 0;
}

int launch_select(const Geom& g, const sa_route_cfg& rc, const float* scores, int32_t* J, hipStream_t st);

template <typename T, int D>
int launch_route_decode_t(const Geom& g, const sa_route_cfg& rc, const T* q, const float* summ, int32_t* J,
                          hipStream_t st) {
  // keys per lane of the selection: the smallest power of two with 64 E >= max_blocks
  const dim3 grid((unsigned)g.rows);
  const size_t smem = route_decode_smem_bytes(g);
  const int mb = std::max(g.max_blocks, 1);
  if (mb > 8192 && smem > 65536 &&   // scores of up to 32768 candidates: more LDS than the default
      hipFuncSetAttribute(reinterpret_cast<const void*>(&route_decode_kernel<T, D, 256>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return SA_ERR_HIP;
  if (mb <= 128) route_decode_kernel<T, D, 2><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 256) route_decode_kernel<T, D, 4><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 512) route_decode_kernel<T, D, 8><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 1024) route_decode_kernel<T, D, 16><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 2048) route_decode_kernel<T, D, 32><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 4096) route_decode_kernel<T, D, 64><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else if (mb <= 8192) route_decode_kernel<T, D, 128><<<grid, 256, smem, st>>>(g, rc, q, summ, J);
  else route_decode_kernel<T, D, 256><<<grid, 256, smem, st>>>(g, rc, q, summ, J);   // selection from LDS
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int launch_route_decode(const Geom& g, const sa_route_cfg& rc, int dtype, const void* q, const float* summ,
                        int32_t* J, hipStream_t st) {
  if (dtype == SA_BF16)
    return g.d == 128 ? launch_route_decode_t<__bf16, 128>(g, rc, (const __bf16*)q, summ, J, st)
                      : launch_route_decode_t<__bf16, 64>(g, rc, (const __bf16*)q, summ, J, st);
  return g.d == 128 ? launch_route_decode_t<float, 128>(g, rc, (const float*)q, summ, J, st)
                    : launch_route_decode_t<float, 64>(g, rc, (const float*)q, summ, J, st);
}

int launch_route(const Geom& g, const sa_route_cfg& rc, int dtype, const void* q,
                 const float* summ, const float* qbar, float* scores, int32_t* J, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  const size_t smem = route_smem_bytes(g, rc.qpool);
  const int mbk = std::max(g.max_blocks, 1);
  if (g.mode == SA_PREFILL && rc.qpool == SA_POOL_MEAN && qbar && (int64_t)g.batch * g.hr <= 65535) {
    if (mbk <= 256) {   // every row's scores fit one workgroup: score and select in one pass
      constexpr int R = 8;   // measured at 128 key blocks: 4 and 8 rows a workgroup alike, 16 slower
      dim3 fgrid((unsigned)((mbk - g.qblk0 + R - 1) / R), 1, (unsigned)(g.batch * g.hr));
#define SA_TS(D, NC) route_tile_select_kernel<D, NC, R><<<fgrid, R * 64, 0, st>>>(g, rc, qbar, summ, J)
      if (g.d == 128) {
        if (mbk <= 64) SA_TS(128, 64);
        else if (mbk <= 128) SA_TS(128, 128);
        else SA_TS(128, 256);
      } else {
        if (mbk <= 64) SA_TS(64, 64);
        else if (mbk <= 128) SA_TS(64, 128);
        else SA_TS(64, 256);
      }
#undef SA_TS
      return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
    }
    // longer histories: 32 x 64 score tiles, then the selection launch
    dim3 tgrid((unsigned)((mbk - g.qblk0 + 31) / 32), (unsigned)((mbk + 63) / 64), (unsigned)(g.batch * g.hr));
    if (g.d == 128) route_score_tile_kernel<128, 32, 64><<<tgrid, 256, 0, st>>>(g, rc, qbar, summ, scores);
    else route_score_tile_kernel<64, 32, 64><<<tgrid, 256, 0, st>>>(g, rc, qbar, summ, scores);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    return launch_select(g, rc, scores, J, st);
  }
  if (g.mode == SA_DECODE && rc.qpool == SA_POOL_MEAN) return launch_route_decode(g, rc, dtype, q, summ, J, st);
  const int chunk = g.mode == SA_DECODE ? kDecodeChunk : std::max(g.max_blocks, 1);
  const int chunks = (std::max(g.max_blocks, 1) + chunk - 1) / chunk;
  dim3 grid((unsigned)g.rows, (unsigned)chunks);
  const bool dec = g.mode == SA_DECODE;
#define SA_SCORE(T, D)                                                                     \
  (dec ? route_score_kernel<T, D, 16><<<grid, 256, smem, st>>>(g, rc, (const T*)q, summ, scores, chunk) \
       : route_score_kernel<T, D, 8><<<grid, 256, smem, st>>>(g, rc, (const T*)q, summ, scores, chunk))
  if (dtype == SA_BF16) {
    if (g.d == 128) SA_SCORE(__bf16, 128);
    else SA_SCORE(__bf16, 64);
  } else {
    if (g.d == 128) SA_SCORE(float, 128);
    else SA_SCORE(float, 64);
  }
#undef SA_SCORE
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  return launch_select(g, rc, scores, J, st);
}

int launch_select(const Geom& g, const sa_route_cfg& rc, const float* scores, int32_t* J, hipStream_t st) {
  // keys per lane: the smallest power of two with 64 E >= max_blocks
  dim3 sgrid((unsigned)g.rows);
  const int mb = std::max(g.max_blocks, 1);
  if (mb <= 128) route_select_kernel<2><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 256) route_select_kernel<4><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 512) route_select_kernel<8><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 1024) route_select_kernel<16><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 2048) route_select_kernel<32><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 4096) route_select_kernel<64><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else if (mb <= 8192) route_select_kernel<128><<<sgrid, 64, 0, st>>>(g, rc, scores, J);
  else route_select_mem_kernel<<<sgrid, 64, 0, st>>>(g, rc, scores, J);   // scores read from memory
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
