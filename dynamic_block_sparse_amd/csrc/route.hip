// Routing kernels: block summaries, pooled query scores and per-row selection.
//
// [P2] §2.1 Eq 6: c_j = mean of block j's keys, g_rj = pool over the queries of
// block r of q . c_j.  [P2] Eq 7: clipped threshold count.  [P2] §2.1 "causal
// boundary" / §4.1: only complete history blocks are scored; the current block
// is a fixed branch.  [P2] §4: shared GQA routing averages over the head group.
// [P1] (top-k of long candidate lists): select without materialising a sort,
// with a stable rule for equal scores (lower block id first).
#include "common.h"
#include "kernels.h"

namespace sa {

// ---------------------------------------------------------------------------
// Block summaries.  One wavefront per (sequence, kv head, key block): lanes own
// an 8-element column chunk and a key phase, so every load is a 16-byte (bf16)
// or 32-byte (fp32) piece of a contiguous 64 x d tile; phases are summed with
// cross-lane shuffles.  Padding tokens past the sequence end never enter the
// sum, and a partial block divides by its own count.
template <typename T, int D>
__global__ void __launch_bounds__(256) summary_kernel(Geom g, const T* __restrict__ k,
                                                      float* __restrict__ summ, int slots) {
  constexpr int CH = D / 8;        // column chunks per row
  constexpr int PH = kWave / CH;   // key phases per wave
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int slot = blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
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
    len = g.n;
  }
  const int cnt = min(kBlock, len - j * kBlock);
  const int c = lane % CH, ph = lane / CH;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const T* base = k + kv_offset(g, s, h, tok0, j * kBlock) + c * 8;
  for (int t = ph; t < cnt; t += PH) {
    const T* p = base + (int64_t)t * D;
    if constexpr (sizeof(T) == 2) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_lo(x[i]);
        acc[2 * i + 1] += bf16_hi(x[i]);
      }
    } else {
      f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
      f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += x0[i];
        acc[4 + i] += x1[i];
      }
    }
  }
#pragma unroll
  for (int o = CH; o < kWave; o <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
  }
  if (ph == 0) {
    const float inv = 1.f / (float)cnt;
    float* out = summ + sum_offset(g, s, h, blk0, j) + c * 8;
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

// ---------------------------------------------------------------------------
// Block-wide helpers for 256-thread workgroups.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan over the 256 threads; returns the prefix, *total = sum.
__device__ __forceinline__ int block_excl_scan256(int v, int* sh /* >= 4 ints */, int* total) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int inc = wave_incl_scan(v);
  __syncthreads();
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int x = sh[w];
    before += (w < wave) ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

__device__ __forceinline__ float block_max256(float v, float* sh) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);   // -0 -> +0 so equal values share a key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Routing: one 256-thread workgroup per worklist row.
//   1. pool the row's queries (mean: one pooled vector over the row's query
//      heads and valid queries; max: per-query scores, max per head, mean
//      over heads)
//   2. score every complete-history candidate block against the summaries
//   3. pick the budget (top-k or Eq 7) and select the top D by
//      (score desc, id asc) with an MSB-first radix select on order-preserving
//      score keys, then emit the picks in ascending id order
template <typename T, int D>
__global__ void __launch_bounds__(256) route_kernel(Geom g, sa_route_cfg rc, const T* __restrict__ q,
                                                    const float* __restrict__ summ,
                                                    int32_t* __restrict__ J) {
  extern __shared__ float smem[];
  float* sc = smem;                                  // [max_blocks] candidate scores
  float* qbar = sc + ((g.max_blocks + 3) & ~3);      // [D]
  float* red = qbar + D;                             // [16 * D] phase partials / max-pool rows
  __shared__ int ishare[8];
  __shared__ float fshare[4];
  __shared__ int hist[256];
  __shared__ uint32_t sel_state[2];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  const int h0 = g.share ? ri.h * g.group : ri.h;
  const int nh = g.hpr;
  int qt0, nq;
  if (g.mode == SA_DECODE) {
    qt0 = 0;
    nq = 1;
  } else {
    qt0 = ri.r * kBlock;
    nq = min(kBlock, ri.len - qt0);
  }
  const int cur = ri.r;
  const bool ff = (rc.forced & SA_FORCE_FIRST) != 0;
  const int n_hist = (g.mode == SA_DECODE) ? ri.nblk - 1 : ri.r;   // blocks j < current
  const int start = (ff && n_hist > 0) ? 1 : 0;
  const int nc = max(n_hist - start, 0);
  const int nforced = 1 + ((ff && cur != 0) ? 1 : 0);
  const float* cbase = summ + sum_offset(g, ri.s, kvh, ri.blk0, 0);

  if (rc.qpool == SA_POOL_MEAN) {
    // ---- 1. mean pool over (head, query) pairs
    constexpr int CH = D / 8, PH = 256 / CH;
    const int c = tid % CH, ph = tid / CH;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    const int items = nh * nq;
    for (int it = ph; it < items; it += PH) {
      const int hh = h0 + it / nq, t = it % nq;
      const T* p = q + q_offset(g, ri.s, hh, ri.tok0, qt0 + t) + c * 8;
      if constexpr (sizeof(T) == 2) {
        u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_lo(x[i]);
          acc[2 * i + 1] += bf16_hi(x[i]);
        }
      } else {
        f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
        f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += x0[i];
          acc[4 + i] += x1[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[ph * D + c * 8 + i] = acc[i];
    __syncthreads();
    if (tid < D) {
      float sacc = 0.f;
      for (int p2 = 0; p2 < PH; ++p2) sacc += red[p2 * D + tid];
      qbar[tid] = sacc / (float)items;
    }
    __syncthreads();
    // ---- 2. scores: LPC lanes cooperate on one candidate (4 floats each)
    constexpr int LPC = D / 4, CPS = kWave / LPC;
    const int cl = lane % LPC, cw = lane / LPC;
    const f32x4 qv = *reinterpret_cast<const f32x4*>(qbar + cl * 4);
    for (int base = wave * CPS; base < nc; base += 4 * CPS) {
      const int j = start + base + cw;
      float part = 0.f;
      if (base + cw < nc) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(cbase + (int64_t)j * D + cl * 4);
        part = qv[0] * cv[0] + qv[1] * cv[1] + qv[2] * cv[2] + qv[3] * cv[3];
      }
#pragma unroll
      for (int o = 1; o < LPC; o <<= 1) part += __shfl_xor(part, o, kWave);
      if (cl == 0 && base + cw < nc) sc[base + cw] = part;
    }
  } else {
    // ---- max pool: per-query scores, max over the block's queries, mean over heads
    for (int i = tid; i < nc; i += 256) sc[i] = 0.f;
    constexpr int LD = D + 1;
    for (int hh = 0; hh < nh; ++hh) {
      __syncthreads();
      for (int e = tid; e < nq * D; e += 256) {
        const int t = e / D, dd = e % D;
        red[t * LD + dd] = to_f32<T>(q[q_offset(g, ri.s, h0 + hh, ri.tok0, qt0 + t) + dd]);
      }
      __syncthreads();
      for (int ci = wave; ci < nc; ci += 4) {
        const float* cj = cbase + (int64_t)(start + ci) * D;
        float dot = 0.f;
        if (lane < nq) {
          for (int dd = 0; dd < D; ++dd) dot += red[lane * LD + dd] * cj[dd];
        } else {
          dot = -INFINITY;
        }
        dot = wave_max(dot);
        if (lane == 0) sc[ci] += dot / (float)nh;
      }
    }
  }
  __syncthreads();

  // ---- 3. budget
  int kr = rc.k_b;
  if (rc.select == SA_SELECT_THRESHOLD) {
    float m = -INFINITY;
    for (int i = tid; i < nc; i += 256) m = fmaxf(m, sc[i]);
    m = block_max256(m, fshare);
    const float tau = m - rc.tau_rel;
    int above = 0;
    for (int i = tid; i < nc; i += 256) above += (sc[i] >= tau) ? 1 : 0;
    int tot;
    (void)block_excl_scan256(above, ishare, &tot);
    const int count = nforced + (nc > 0 ? tot : 0);
    kr = min(rc.k_b, max(rc.k_min, count));
  }
  const int dsel = min(max(kr - nforced, 0), nc);

  // ---- radix select of the dsel-th largest key (all keys valid candidates)
  uint32_t thr = 0u;
  int take_eq = 0;
  const bool take_all = (dsel == nc);
  if (!take_all && dsel > 0) {
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = dsel;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += 256) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += 256) {
        const uint32_t key = order_key(sc[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        int cnt[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cnt[i] = hist[255 - 4 * lane - i];
          local += cnt[i];
        }
        const int incl = wave_incl_scan(local);
        int above = incl - local;     // keys with a larger digit
        if (above < remaining && remaining <= incl) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (above < remaining && remaining <= above + cnt[i]) {
              sel_state[0] = (uint32_t)(255 - 4 * lane - i);
              sel_state[1] = (uint32_t)(remaining - above);
            }
            above += cnt[i];
          }
        }
      }
      __syncthreads();
      prefix |= sel_state[0] << shift;
      pmask |= 255u << shift;
      remaining = (int)sel_state[1];
      __syncthreads();
    }
    thr = prefix;
    take_eq = remaining;
  }

  // ---- emit forced blocks, picks (ascending id) and padding
  int32_t* jrow = J + row * rc.k_b;
  if (tid == 0) {
    int w = 0;
    if (ff && cur != 0) jrow[w++] = 0;
    jrow[w++] = cur;
  }
  if (dsel > 0) {
    const int chunk = (nc + 255) / 256;
    const int c0 = min(tid * chunk, nc), c1 = min(c0 + chunk, nc);
    // rank of this thread's first equal-to-threshold key among all equal keys
    int n_eq = 0;
    if (!take_all)
      for (int i = c0; i < c1; ++i) n_eq += (order_key(sc[i]) == thr) ? 1 : 0;
    int tot;
    const int eq_base = block_excl_scan256(n_eq, ishare, &tot);
    int n_take = 0;
    {
      int e = eq_base;
      for (int i = c0; i < c1; ++i) {
        const uint32_t key = order_key(sc[i]);
        const bool tk = take_all || key > thr || (key == thr && e++ < take_eq);
        n_take += tk ? 1 : 0;
      }
    }
    int pos = block_excl_scan256(n_take, ishare + 4, &tot);
    {
      int e = eq_base;
      for (int i = c0; i < c1; ++i) {
        const uint32_t key = order_key(sc[i]);
        const bool tk = take_all || key > thr || (key == thr && e++ < take_eq);
        if (tk) jrow[nforced + pos++] = start + i;
      }
    }
  }
  for (int i = nforced + dsel + tid; i < rc.k_b; i += 256) jrow[i] = -1;
}

// ---------------------------------------------------------------------------
int launch_summary(const Geom& g, int dtype, const void* k, float* summ, int slots,
                   hipStream_t st) {
  if (slots <= 0) return SA_OK;
  dim3 grid((slots + 3) / 4, g.hkv);
  if (dtype == SA_BF16) {
    if (g.d == 128)
      summary_kernel<__bf16, 128><<<grid, 256, 0, st>>>(g, (const __bf16*)k, summ, slots);
    else
      summary_kernel<__bf16, 64><<<grid, 256, 0, st>>>(g, (const __bf16*)k, summ, slots);
  } else {
    if (g.d == 128)
      summary_kernel<float, 128><<<grid, 256, 0, st>>>(g, (const float*)k, summ, slots);
    else
      summary_kernel<float, 64><<<grid, 256, 0, st>>>(g, (const float*)k, summ, slots);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

size_t route_smem_bytes(const Geom& g, int qpool) {
  const size_t sc = (size_t)((g.max_blocks + 3) & ~3) * 4;
  const size_t qb = (size_t)g.d * 4;
  const size_t mean_red = (size_t)(256 / (g.d / 8)) * g.d * 4;   // phase partials
  const size_t max_red = (size_t)kBlock * (g.d + 1) * 4;         // one head's query rows
  return sc + qb + (qpool == SA_POOL_MAX ? max_red : mean_red);
}

int launch_route(const Geom& g, const sa_route_cfg& rc, int dtype, const void* q,
                 const float* summ, int32_t* J, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  const size_t smem = route_smem_bytes(g, rc.qpool);
  dim3 grid((unsigned)g.rows);
  if (dtype == SA_BF16) {
    if (g.d == 128)
      route_kernel<__bf16, 128><<<grid, 256, smem, st>>>(g, rc, (const __bf16*)q, summ, J);
    else
      route_kernel<__bf16, 64><<<grid, 256, smem, st>>>(g, rc, (const __bf16*)q, summ, J);
  } else {
    if (g.d == 128)
      route_kernel<float, 128><<<grid, 256, smem, st>>>(g, rc, (const float*)q, summ, J);
    else
      route_kernel<float, 64><<<grid, 256, smem, st>>>(g, rc, (const float*)q, summ, J);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
