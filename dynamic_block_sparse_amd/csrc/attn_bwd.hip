// Backward pass of the block-sparse attention over the forward's worklist.
//
// [P2] §4 (training) and [P3]: the backward pass reuses the forward's block
// selection, so every query attends exactly the keys it attended in the
// forward, and the forward's log-sum-exp recovers the probabilities without a
// second softmax.  For query i and attended key p (scale c = 1 / sqrt(d)):
//   P_ip = exp(c q_i . k_p - lse_i),   D_i = sum_d dO_id O_id,
//   dS_ip = P_ip (dO_i . v_p - D_i),
//   dQ_i = c sum_p dS_ip k_p,  dK_p = c sum_i dS_ip q_i,  dV_p = sum_i P_ip dO_i.
//
// bf16 path (d = 128), two kernels on v_mfma_f32_32x32x16_bf16:
//   * dQ, one workgroup per (worklist row, query head), 2 wavefronts of 32
//     query rows: the row's Q and dO are staged in LDS once, each listed K/V
//     tile is loaded into registers while the previous one is multiplied and
//     then staged in LDS, S^T = K Q^T and dP^T = V dO^T give every lane one query
//     row of P and dS, and dQ^T += K^T dS^T reads K^T with LDS transpose
//     reads.  It also writes D_i, which the second kernel reads;
//   * dK and dV, one workgroup per (key block, KV head), 4 wavefronts (2 key
//     halves x 2 query halves): K and V of the block are staged once; the kernel walks every
//     worklist row of the sequence whose list holds the block (binary search
//     of the sorted lists, 64 rows per step, one row per lane), stages the
//     row's Q and dO, forms S = Q K^T and dP = dO V^T with one key per lane,
//     and accumulates dV^T += dO^T P and dK^T += Q^T dS in registers over all
//     of them, so each key is written once.  A key block listed by more
//     (row, head) pairs than a target (a counting pass finds out) is shared
//     by up to 8 workgroups, each taking an equal run of its pairs: they add
//     their sums into fp32 accumulators with atomics and the last one to
//     finish converts them (only such blocks' sums have no fixed order).
//   P and dS enter the second products as bf16 operands (as P does in the
//   forward); everything else is fp32.
// fp32 path (d = 64): a plain SIMT kernel, one lane per query row, with dK
// and dV added into fp32 workspace accumulators by atomics (their summation
// order is therefore not fixed) and converted by a last pass.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sa {

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

__global__ void __launch_bounds__(256) bwd_fill_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

template <typename T>
__global__ void __launch_bounds__(256) bwd_convert_kernel(const float* __restrict__ acc, T* __restrict__ out,
                                                          int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = (T)acc[i];
}

// fp32 SIMT kernel: one wavefront per (worklist row, query head), one lane per
// query row.  Per listed tile the K, V tiles are staged in LDS, each lane forms
// its row of P and dS over the tile's 64 keys, accumulates dQ in registers and
// writes P and dS transposed to LDS; then lane t takes key t and reduces
// dV_t = sum_i P_it dO_i and dK_t = c sum_i dS_it q_i over the row's 64
// queries in chunks of 32 columns, and adds them to the accumulators.
template <typename T, int D>
__global__ void __launch_bounds__(64) attn_bwd_simt_kernel(Geom g, BwdBufs a) {
  // row padding of the per-lane-row tiles (Q, dO): an odd number of dwords per
  // row, so the 64 lanes reading their own rows hit distinct banks
  constexpr int PAD = sizeof(T) == 2 ? 2 : 1;
  constexpr int CH = 32;   // dK / dV columns reduced per pass
  __shared__ T ks[64][D], vs[64][D];
  __shared__ T qs[64][D + PAD], dos[64][D + PAD];
  __shared__ float pst[64][65], dst[64][65];   // P^T and dS^T of the tile: [key][query]

  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const int head = (g.share ? ri.h * g.group : ri.h) + (int)blockIdx.y;
  const int kvh = head / g.group;
  const int qpos = ri.r * kBlock + lane;
  const bool qvalid = qpos < ri.len;
  const float c = rsqrtf((float)D);
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  const T* o = (const T*)a.o;
  const T* dout = (const T*)a.dout;

  // this row's Q and dO rows (zeros past the sequence end), D_i and lse_i
  float delta = 0.f, lse = 0.f;
  {
    const int64_t qo = q_offset(g, ri.s, head, ri.tok0, qvalid ? qpos : ri.r * kBlock);
    for (int e = 0; e < D; ++e) {
      const T qv = qvalid ? q[qo + e] : (T)0.f;
      const T dv = qvalid ? dout[qo + e] : (T)0.f;
      qs[lane][e] = qv;
      dos[lane][e] = dv;
      if (qvalid) delta = fmaf(to_f(dv), to_f(o[qo + e]), delta);
    }
    if (qvalid) lse = a.lse[lse_offset(g, ri.s, head, ri.tok0, qpos)];
  }
  float dq[D];
#pragma unroll
  for (int e = 0; e < D; ++e) dq[e] = 0.f;

  for (int t = a.row_ptr[row]; t < a.row_ptr[row + 1]; ++t) {
    const int j = a.col_idx[t];
    const int cnt = min(kBlock, ri.len - j * kBlock);
    const int64_t kb = kv_block_offset(g, ri.s, kvh, ri.tok0, j);
    __syncthreads();   // the previous tile's LDS is no longer read
    for (int e = lane; e < 64 * D; e += 64) {
      const int key = e / D, dd = e % D;
      ks[key][dd] = key < cnt ? k[kb + e] : (T)0.f;
      vs[key][dd] = key < cnt ? v[kb + e] : (T)0.f;
    }
    __syncthreads();
    // this lane's row of P and dS over the tile's keys; dQ += c dS K
    for (int key = 0; key < 64; ++key) {
      const int kpos = j * kBlock + key;
      const bool ok = qvalid && key < cnt && kpos <= qpos;
      float s = 0.f, dp = 0.f;
      for (int e = 0; e < D; ++e) {
        s = fmaf(to_f(qs[lane][e]), to_f(ks[key][e]), s);
        dp = fmaf(to_f(dos[lane][e]), to_f(vs[key][e]), dp);
      }
      const float p = ok ? expf(s * c - lse) : 0.f;
      const float ds = p * (dp - delta);
#pragma unroll
      for (int e = 0; e < D; ++e) dq[e] = fmaf(ds * c, to_f(ks[key][e]), dq[e]);
      pst[key][lane] = p;
      dst[key][lane] = ds;
    }
    __syncthreads();
    // lane = key: dV_key = sum_i P_i,key dO_i and dK_key = c sum_i dS_i,key q_i
    if (lane < cnt) {
      float* dvp = a.dv_acc + kb + (int64_t)lane * D;
      float* dkp = a.dk_acc + kb + (int64_t)lane * D;
      for (int c0 = 0; c0 < D; c0 += CH) {
        float av[CH], ak[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) av[e] = ak[e] = 0.f;
        for (int i = 0; i < 64; ++i) {
          const float p = pst[lane][i], ds = dst[lane][i];
#pragma unroll
          for (int e = 0; e < CH; ++e) {
            av[e] = fmaf(p, to_f(dos[i][c0 + e]), av[e]);
            ak[e] = fmaf(ds, to_f(qs[i][c0 + e]), ak[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          atomicAdd(dvp + c0 + e, av[e]);
          atomicAdd(dkp + c0 + e, ak[e] * c);
        }
      }
    }
  }
  if (qvalid) {
    T* dqp = (T*)a.dq + q_offset(g, ri.s, head, ri.tok0, qpos);
#pragma unroll
    for (int e = 0; e < D; ++e) dqp[e] = (T)dq[e];
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA kernels (d = 128).  v_mfma_f32_32x32x16_bf16 layouts, lane =
// 32 half + l32:  A operand = A[l32][8 half + e],  B operand = B[8 half +
// e][l32],  accumulator element i = C[8 (i / 4) + 4 half + i % 4][l32].
// A 32-row block of an accumulator converts in place into the B operand of a
// product that contracts over those rows, in the order
//   k-slot (half, e) of step ks = row 16 ks + 8 (e / 4) + 4 half + e % 4,
// and the A operand of that product is read in the same order from a
// row-major LDS tile with ds_read_b64_tr_b16 (tr8 below).
//
// LDS tiles are [64 rows][128 d] bf16 (256 bytes a row) in 16-byte chunks,
// the chunk index XORed with a row swizzle: rsw for tiles read only by rows
// (16-byte reads of one row per lane), tsw for tiles also read transposed.

#define SA_LDS __attribute__((address_space(3)))
typedef short i16x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

// rsw: 16 consecutive rows read at one chunk land on 16 distinct chunk slots.
// tsw keeps that (it is a bijection of row & 15) and also gives the four
// consecutive rows of a transpose read, each touching an aligned chunk pair,
// distinct pair slots whose partners (chunk + 2, read by the neighbouring
// 16 lanes) are distinct too: (row & 3) selects the pair slot's high bits.
__device__ __forceinline__ int rsw(int row) { return row & 15; }
__device__ __forceinline__ int tsw(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// 8 bf16 of tile row `row`, columns 8 c .. 8 c + 7
template <bool TR>
__device__ __forceinline__ bf16x8 row8(const unsigned char* t, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(t + row * 256 + ((c ^ (TR ? tsw(row) : rsw(row))) << 4));
}

// A operand of a product contracting over tile rows: lane (l32, half) gets
// column db * 32 + l32 of the rows rb * 32 + 16 ks + 8 (e / 4) + 4 half + e % 4.
// Each 16-lane group's transpose read returns, to lane i, column i of the
// 4 x 16 block its lanes address row-wise.
__device__ __forceinline__ bf16x8 tr8(const unsigned char* t, int rb, int ks, int db, int lane) {
  const int gi = lane >> 4, li = lane & 15, vh = gi >> 1, vdh = gi & 1;
  const int d = db * 32 + 16 * vdh + 4 * (li & 3);
  const int chunk = d >> 3, h8 = (d >> 2) & 1;
  const int r0 = rb * 32 + 16 * ks + 4 * vh + (li >> 2), r1 = r0 + 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (SA_LDS i16x4*)(t + r0 * 256 + ((chunk ^ tsw(r0)) << 4) + h8 * 8));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (SA_LDS i16x4*)(t + r1 * 256 + ((chunk ^ tsw(r1)) << 4) + h8 * 8));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The lane-dependent parts of the tile reads above, computed once: a read's
// address is then the tile's base + one of these + a constant.
//   row8<TR>(t, 32 b + l32, 2 ks + half) = t + 8192 b + row[ks]
//   tr8(t, rb, ks, db, lane)             = halves at t + 8192 rb + 4096 ks + tr[db][0 / 1]
// (tsw and rsw depend on row & 15 only, which 32 b, 16 ks and 32 rb leave alone.)
struct TileReadOffsets {
  uint32_t row[8], tr[4][2];
};
template <bool TR>
__device__ __forceinline__ TileReadOffsets tile_read_offsets(int lane) {
  TileReadOffsets o;
  const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    o.row[ks] = (uint32_t)(l32 * 256 + (((2 * ks + half) ^ (TR ? tsw(l32) : rsw(l32))) << 4));
  const int gi = lane >> 4, li = lane & 15, vh = gi >> 1, vdh = gi & 1;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + 16 * vdh + 4 * (li & 3);
    const int chunk = d >> 3, h8 = (d >> 2) & 1;
    const int r0 = 4 * vh + (li >> 2), r1 = r0 + 8;
    o.tr[db][0] = (uint32_t)(r0 * 256 + ((chunk ^ tsw(r0)) << 4) + h8 * 8);
    o.tr[db][1] = (uint32_t)(r1 * 256 + ((chunk ^ tsw(r1)) << 4) + h8 * 8);
  }
  return o;
}
typedef SA_LDS const unsigned char* lds_ptr;
__device__ __forceinline__ lds_ptr to_lds(const unsigned char* p) { return (lds_ptr)p; }
__device__ __forceinline__ bf16x8 row8_at(lds_ptr t, uint32_t off) {
  return *reinterpret_cast<SA_LDS const bf16x8*>(t + off);
}
__device__ __forceinline__ bf16x8 tr8_at(lds_ptr t, const uint32_t (&off)[2]) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(t + off[0]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(t + off[1]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kMfma = 0x008, kDsRead = 0x100;   // scheduling-group masks

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Stage `rows` valid rows (the rest zero) of a [64][128] bf16 tile whose row
// i starts at src + i * 128, by the workgroup's NT threads.
template <bool TR, int NT>
__device__ __forceinline__ void stage_tile(unsigned char* t, const __bf16* src, int rows, int tid) {
#pragma unroll
  for (int it = 0; it < 1024 / NT; ++it) {
    const int c = it * NT + tid, row = c >> 4, ch = c & 15;
    const u32x4 x = row < rows ? *reinterpret_cast<const u32x4*>(src + row * 128 + ch * 8) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(t + row * 256 + ((ch ^ (TR ? tsw(row) : rsw(row))) << 4)) = x;
  }
}

// Rows of a 32-column accumulator block scaled and stored as bf16: lane owns
// column l32 (one output row at dst) and writes its 16 elements as four runs
// of 4 consecutive d.
__device__ __forceinline__ void store_acc(const f32x16 (&acc)[4], float scale, __bf16* dst, int half) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[db][4 * gq + e] * scale);
      *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * gq + 4 * half) = v;
    }
}

// The next tile's K and V rows are loaded into registers while the current
// tile is multiplied, and written to LDS after the next barrier.
struct TileRegs {
  u32x4 k[8], v[8];
};
__device__ __forceinline__ void load_tile_regs(TileRegs& t, const __bf16* k, const __bf16* v, int rows, int tid) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = it * 128 + tid, row = c >> 4, ch = c & 15;
    const u32x4 z = {0, 0, 0, 0};
    t.k[it] = row < rows ? *reinterpret_cast<const u32x4*>(k + row * 128 + ch * 8) : z;
    t.v[it] = row < rows ? *reinterpret_cast<const u32x4*>(v + row * 128 + ch * 8) : z;
  }
}
__device__ __forceinline__ void store_tile_regs(const TileRegs& t, unsigned char* kt, unsigned char* vt, int tid) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = it * 128 + tid, row = c >> 4, ch = c & 15;
    *reinterpret_cast<u32x4*>(kt + row * 256 + ((ch ^ tsw(row)) << 4)) = t.k[it];
    *reinterpret_cast<u32x4*>(vt + row * 256 + ((ch ^ rsw(row)) << 4)) = t.v[it];
  }
}

__global__ void __launch_bounds__(128) bwd_dq_bf16_kernel(Geom g, BwdBufs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kt[64 * 256], vt[64 * 256], qs[64 * 256], dos[64 * 256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const int head = (g.share ? ri.h * g.group : ri.h) + (int)blockIdx.y;
  const int kvh = head / g.group;
  const int qpos = ri.r * kBlock + w * 32 + l32;
  const bool qvalid = qpos < ri.len;
  const int qrows = min(kBlock, ri.len - ri.r * kBlock);
  const float c = 0.08838834764831845f, cl2 = c * kLog2e;   // 1 / sqrt(128)
  const __bf16* k = (const __bf16*)a.k;
  const __bf16* v = (const __bf16*)a.v;
  const int t0 = a.row_ptr[row], t1 = a.row_ptr[row + 1];

  // the first tile's loads go out before anything else
  TileRegs nxt;
  if (t0 < t1) {
    const int j = a.col_idx[t0];
    const int64_t kb = kv_block_offset(g, ri.s, kvh, ri.tok0, j);
    load_tile_regs(nxt, k + kb, v + kb, min(kBlock, ri.len - j * kBlock), tid);
  }
  // the row's Q and dO (B operands, read by rows); D_i = dO_i . O_i
  const int64_t qo0 = q_offset(g, ri.s, head, ri.tok0, ri.r * kBlock);
  stage_tile<false, 128>(qs, (const __bf16*)a.q + qo0, qrows, tid);
  stage_tile<false, 128>(dos, (const __bf16*)a.dout + qo0, qrows, tid);
  float delta = 0.f, lse2 = 0.f;
  {
    const int64_t qo = qo0 + (int64_t)(w * 32 + l32) * 128 + half * 8;
    const __bf16* dp = (const __bf16*)a.dout + qo;
    const __bf16* op = (const __bf16*)a.o + qo;
    float part = 0.f;
    if (qvalid)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 dv8 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dp + ks * 16));
        const bf16x8 ov8 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + ks * 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf((float)dv8[e], (float)ov8[e], part);
      }
    delta = part + __shfl_xor(part, 32);
    if (qvalid) {
      const int64_t lo = lse_offset(g, ri.s, head, ri.tok0, qpos);
      lse2 = a.lse[lo] * kLog2e;
      if (half == 0) a.delta[lo] = delta;
      else a.nlse2[lo] = -lse2;
    }
  }
  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

  const int qrow = w * 32 + l32;
  for (int t = t0; t < t1; ++t) {
    const int j = a.col_idx[t];
    __syncthreads();   // the previous tile is no longer read
    store_tile_regs(nxt, kt, vt, tid);
    __syncthreads();
    if (t + 1 < t1) {   // next tile in flight during this one's products
      const int jn = a.col_idx[t + 1];
      const int64_t kbn = kv_block_offset(g, ri.s, kvh, ri.tok0, jn);
      load_tile_regs(nxt, k + kbn, v + kbn, min(kBlock, ri.len - jn * kBlock), tid);
    }
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[b2][i] = dpacc[b2][i] = 0.f;
    // the six LDS operands of step ks + 1 are read while step ks multiplies
    bf16x8 op[2][6];
    auto rd = [&](int ks, bf16x8 (&o)[6]) {
      o[0] = row8<true>(kt, l32, 2 * ks + half);
      o[1] = row8<true>(kt, 32 + l32, 2 * ks + half);
      o[2] = row8<false>(vt, l32, 2 * ks + half);
      o[3] = row8<false>(vt, 32 + l32, 2 * ks + half);
      o[4] = row8<false>(qs, qrow, 2 * ks + half);
      o[5] = row8<false>(dos, qrow, 2 * ks + half);
    };
    rd(0, op[0]);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) rd(ks + 1, op[(ks + 1) & 1]);
      const bf16x8(&o)[6] = op[ks & 1];
      sacc[0] = mfma(o[0], o[4], sacc[0]);
      sacc[1] = mfma(o[1], o[4], sacc[1]);
      dpacc[0] = mfma(o[2], o[5], dpacc[0]);
      dpacc[1] = mfma(o[3], o[5], dpacc[1]);
      if (ks + 1 < 8) __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
      __builtin_amdgcn_sched_group_barrier(kMfma, 4, 0);
    }
    // dS^T of this lane's query over the tile's keys, as B operands
    bf16x8 dsb[2][2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kpos = j * kBlock + b2 * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        const bool ok = qvalid && kpos <= qpos;
        const float p = __builtin_amdgcn_exp2f(ok ? fmaf(sacc[b2][i], cl2, -lse2) : -INFINITY);
        dsb[b2][i / 8][i % 8] = (__bf16)(p * (dpacc[b2][i] - delta));
      }
    // dQ^T += K^T dS^T: the transpose reads run four MFMAs ahead
    bf16x8 ta[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ta[i] = tr8(kt, (i >> 1) & 1, i & 1, i >> 2, lane);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int db = i >> 2, b2 = (i >> 1) & 1, ks = i & 1;
      const bf16x8 av = ta[i & 3];
      if (i + 4 < 16) ta[i & 3] = tr8(kt, ((i + 4) >> 1) & 1, (i + 4) & 1, (i + 4) >> 2, lane);
      dq[db] = mfma(av, dsb[b2][ks], dq[db]);
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (i + 4 < 16) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
  }
  if (qvalid) store_acc(dq, c, (__bf16*)a.dq + q_offset(g, ri.s, head, ri.tok0, qpos), half);
}

// Global -> LDS loads (see the forward kernels): lane l's 16 bytes (4 bytes)
// from base + off land at lds_wave_base + 16 l (+ 4 l).  Issued as inline asm
// so the compiler does not wait for them at unrelated LDS reads; the loop
// waits for them explicitly before the barrier that publishes a pair.
__device__ __forceinline__ void bwd_load_lds16(const unsigned char* base, uint32_t off, const unsigned char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SA_LDS const unsigned char*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void bwd_load_lds4(const unsigned char* base, uint32_t off, const unsigned char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SA_LDS const unsigned char*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ const unsigned char* bwd_uniform(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const unsigned char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void bwd_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `pairs` younger pairs' loads (L per pair) are in flight
template <int L>
__device__ __forceinline__ void bwd_wait_pairs(int pairs) {
  if (pairs >= 2) bwd_wait_vmcnt<2 * L>();
  else if (pairs == 1) bwd_wait_vmcnt<L>();
  else bwd_wait_vmcnt<0>();
}

// dQ for rows serving 2, 4 or 8 query heads (routing shared across a KV head's
// group): one workgroup per (worklist row, pair of its heads), 4 wavefronts,
// wave w taking query head 2 blockIdx.y + w / 2 and query rows 32 (w % 2) ..
// + 32.  The row's listed K and V tiles are read once for both heads: they
// stream global -> LDS through a ring of NB tiles (each wavefront loads its
// share, issued NB - 1 tiles ahead, one barrier per tile).  Two tiles (64 KB)
// leave room for a second workgroup on the CU, whose work covers this one's
// waits (232 registers: two wavefronts a SIMD); a 3-deep ring with one
// workgroup a CU was 3-7 % slower.  Each lane keeps
// its query row of Q and dO (the B operands of S^T = K Q^T and dP^T =
// V dO^T) in registers, forms P and dS for one 32-key half of the tile at a
// time, and accumulates dQ^T += K^T dS^T (K^T by LDS transpose reads).  It
// also writes D_i = dO_i . O_i, which the dK/dV kernel reads.  (Four heads
// in one workgroup of 8 wavefronts need more than the 256 registers a
// wavefront may then hold.)
__global__ void __launch_bounds__(256) bwd_dq_rows_bf16_kernel(Geom g, BwdBufs a) {
  constexpr int NW = 4, NB = 2, TILE = 64 * 256;
  constexpr int LPT = 16 / NW;   // 1 KB slices of K (and as many of V) per wavefront and tile
  static_assert(NW * LPT * 1024 == TILE, "the wavefronts' slices cover the tile once");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NB][2][TILE];   // [slot][K, V]
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row = blockIdx.x;
  const RowInfo ri = decode_row(g, row);
  const int kvh = ri.h;   // shared routing: the routing head is the KV head
  const int head = kvh * g.group + 2 * (int)blockIdx.y + wave / 2;
  const int qpos = ri.r * kBlock + (wave & 1) * 32 + l32;
  const bool qvalid = qpos < ri.len;
  const int qsrc = min(qpos, ri.len - 1);   // rows past the end read the last row (masked)
  const float c = 0.08838834764831845f, cl2 = c * kLog2e;
  const int t0 = a.row_ptr[row], nt = a.row_ptr[row + 1] - t0;
  const int jl0 = lane < nt ? a.col_idx[t0 + lane] : 0;
  const int jl1 = lane + 64 < nt ? a.col_idx[t0 + 64 + lane] : 0;
  auto tile_id = [&](int t) {
    return t < 64 ? __builtin_amdgcn_readlane(jl0, t) : __builtin_amdgcn_readlane(jl1, t - 64);
  };

  // this wavefront's 1 KB slices of a tile: slice sl = wave + NW * ii holds
  // rows 4 sl .. 4 sl + 3; lane l lands at row 4 sl + l / 16, chunk slot l % 16
  // (K swizzled for row and transpose reads, V for row reads)
  const unsigned char* const kbytes = (const unsigned char*)a.k;
  const unsigned char* const vbytes = (const unsigned char*)a.v;
  auto issue_tile = [&](int t, int slot) {
    const int j = tile_id(t);
    const int cnt = min(kBlock, ri.len - j * kBlock);
    const int64_t kb = kv_block_offset(g, ri.s, kvh, ri.tok0, j) * 2;
    const unsigned char* kbase = bwd_uniform(kbytes + kb);
    const unsigned char* vbase = bwd_uniform(vbytes + kb);
#pragma unroll
    for (int ii = 0; ii < LPT; ++ii) {
      const int sl = wave + NW * ii, r4 = 4 * sl + (lane >> 4), p = lane & 15;
      const uint32_t rb = (uint32_t)min(r4, cnt - 1) * 256;   // keys past the end: a valid row (masked)
      bwd_load_lds16(kbase, rb + ((p ^ tsw(r4)) << 4), &ring[slot][0][sl * 1024]);
      bwd_load_lds16(vbase, rb + ((p ^ rsw(r4)) << 4), &ring[slot][1][sl * 1024]);
    }
  };
  for (int t = 0; t < NB - 1; ++t)
    if (t < nt) issue_tile(t, t);

  // this lane's Q and dO row (d = 16 ks + 8 half .. + 8), D_i and lse
  bf16x8 qreg[8], doreg[8];
  float delta, lse2;
  {
    const int64_t qo = q_offset(g, ri.s, head, ri.tok0, qsrc) + 8 * half;
    const __bf16* qp = (const __bf16*)a.q + qo;
    const __bf16* dp = (const __bf16*)a.dout + qo;
    const __bf16* op = (const __bf16*)a.o + qo;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
      doreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dp + 16 * ks));
      const bf16x8 ov = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * ks));
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)doreg[ks][e], (float)ov[e], part);
    }
    delta = part + __shfl_xor(part, 32);
    const int64_t lo = lse_offset(g, ri.s, head, ri.tok0, qsrc);
    lse2 = a.lse[lo] * kLog2e;
    if (qvalid) {
      if (half == 0) a.delta[lo] = delta;
      else a.nlse2[lo] = -lse2;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks]), "v"(doreg[ks]));
    asm volatile("" ::"v"(lse2), "v"(jl0), "v"(jl1));
  }

  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
  const TileReadOffsets ko = tile_read_offsets<true>(lane), vo = tile_read_offsets<false>(lane);
  // tiles before the row's query block need no mask when all its rows are valid
  const int jfree = (ri.r + 1) * kBlock <= ri.len ? ri.r : 0;

  int slot = 0;   // t % NB, stepped (a modulo of the loop counter is rebuilt per address)
  for (int t = 0; t < nt; ++t) {
    const int younger = min(NB - 2, nt - 1 - t);   // tiles issued after t
    if (younger >= 1) bwd_wait_vmcnt<2 * LPT>();
    else bwd_wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");   // tile t landed for every wave; slot (t - 1) % NB is read
    if (t + NB - 1 < nt) issue_tile(t + NB - 1, slot == 0 ? NB - 1 : slot - 1);
    const lds_ptr kt = to_lds(ring[slot][0]);
    const lds_ptr vt = to_lds(ring[slot][1]);
    const int j = tile_id(t);
    bf16x8 dsb[2][2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      // S^T and dP^T for keys 32 b2 .. + 32 of the tile; the K and V rows of
      // step ks + 1 are read while step ks multiplies
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
      bf16x8 ok_[2], ov_[2];
      auto rd = [&](int ks) {
        ok_[ks & 1] = row8_at(kt + 8192 * b2, ko.row[ks]);
        ov_[ks & 1] = row8_at(vt + 8192 * b2, vo.row[ks]);
      };
      rd(0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 1 < 8) rd(ks + 1);
        sacc = mfma(ok_[ks & 1], qreg[ks], sacc);
        dpacc = mfma(ov_[ks & 1], doreg[ks], dpacc);
        if (ks + 1 < 8) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
      }
      // dS^T of this lane's query over the half's keys, as B operands
      if (j < jfree) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[i], cl2, -lse2));
          dsb[b2][i / 8][i % 8] = (__bf16)(p * (dpacc[i] - delta));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kpos = j * kBlock + b2 * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          const bool ok = qvalid && kpos <= qpos;
          const float p = __builtin_amdgcn_exp2f(ok ? fmaf(sacc[i], cl2, -lse2) : -INFINITY);
          dsb[b2][i / 8][i % 8] = (__bf16)(p * (dpacc[i] - delta));
        }
      }
    }
    // dQ^T += K^T dS^T: the transpose reads run four MFMAs ahead
    bf16x8 ta[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ta[i] = tr8_at(kt + 8192 * ((i >> 1) & 1) + 4096 * (i & 1), ko.tr[i >> 2]);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int db = i >> 2, b2 = (i >> 1) & 1, ks = i & 1;
      const bf16x8 av = ta[i & 3];
      if (i + 4 < 16)
        ta[i & 3] = tr8_at(kt + 8192 * (((i + 4) >> 1) & 1) + 4096 * ((i + 4) & 1), ko.tr[(i + 4) >> 2]);
      dq[db] = mfma(av, dsb[b2][ks], dq[db]);
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (i + 4 < 16) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
    slot = slot == NB - 1 ? 0 : slot + 1;
  }
  if (qvalid) store_acc(dq, c, (__bf16*)a.dq + q_offset(g, ri.s, head, ri.tok0, qpos), half);
}

// Worklist row id of (sequence s, routing head h, query block r).
__device__ __forceinline__ int64_t row_id(const Geom& g, int s, int h, int r, int blk0, int nb) {
  if (!g.varlen) return ((int64_t)s * g.hr + h) * (nb - g.qblk0) + (r - g.qblk0);
  return (int64_t)g.hr * blk0 + (int64_t)h * nb + r;
}

// Key block slot x (of one KV head) -> sequence, block and the sequence's
// length, first token, first block slot and block count.
struct KeySlot {
  int s, j, len, tok0, blk0, nb;
};
__device__ __forceinline__ KeySlot key_slot(const Geom& g, int x) {
  KeySlot k;
  if (!g.varlen) {
    k.nb = ceil_div(g.n, kBlock);
    k.s = x / k.nb;
    k.j = x % k.nb;
    k.len = g.n;
    k.tok0 = 0;
    k.blk0 = 0;
  } else {
    int lo = 0, hi = g.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.cu_blocks[mid] <= x) lo = mid; else hi = mid - 1;
    }
    k.s = lo;
    k.blk0 = g.cu_blocks[lo];
    k.nb = g.cu_blocks[lo + 1] - k.blk0;
    k.j = x - k.blk0;
    k.tok0 = g.cu_seqlens[lo];
    k.len = g.cu_seqlens[lo + 1] - k.tok0;
  }
  return k;
}

// (row, head) pairs per key block: one wavefront per worklist row, whose
// lanes add the query heads the row serves to the blocks it lists.
__global__ void __launch_bounds__(256) bwd_count_kernel(Geom g, BwdBufs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.rows) return;
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  const int64_t slot0 = g.varlen ? (int64_t)ri.blk0 : (int64_t)ri.s * ri.nblk;
  const int t1 = a.row_ptr[row + 1];
  for (int t = a.row_ptr[row] + (int)(threadIdx.x & 63); t < t1; t += 64)
    atomicAdd(a.kcount + (slot0 + a.col_idx[t]) * g.hkv + kvh, g.hpr);
}

// Workgroups that share a key block add into the fp32 accumulators: clear
// those blocks' rows.
__global__ void __launch_bounds__(256) bwd_split_clear_kernel(Geom g, BwdBufs a) {
  const int kvh = blockIdx.y;
  if (a.kcount[(int64_t)blockIdx.x * g.hkv + kvh] <= a.split_target) return;
  const KeySlot ks = key_slot(g, (int)blockIdx.x);
  const int cnt = min(kBlock, ks.len - ks.j * kBlock);
  const int64_t kb = kv_block_offset(g, ks.s, kvh, ks.tok0, ks.j);
  for (int e = threadIdx.x; e < cnt * 128; e += 256) {
    a.dk_acc[kb + e] = 0.f;
    a.dv_acc[kb + e] = 0.f;
  }
}

// Key-major pair lists.  kcount holds the (row, head) pairs listing each
// (key block slot, KV head); a row serves ngh of them (the KV head's query
// heads when routing is shared, else one), so the rows listing it number
// kcount / ngh.  One workgroup turns those counts into exclusive offsets kptr
// ([slots x Hkv + 1]; the last entry is the total, the worklist's nnz), and
// lists the dK/dV workgroups: one per (slot, KV head), or nch of them for a
// block with more pairs than split_target, as witem entries (index << 4 |
// chunk), -1 up to witems.  The workgroups go out KV head by KV head (all
// slots of one KV head, then the next), so the query rows that the
// workgroups in flight read belong to one KV head's query heads.
__device__ __forceinline__ int bwd_chunks(int units, int split_target, int max_chunks) {
  return units > split_target ? min(max_chunks, (units + split_target - 1) / split_target) : 1;
}

__global__ void __launch_bounds__(1024) bwd_kscan_kernel(const int* __restrict__ kcount, int* __restrict__ kptr,
                                                         int* __restrict__ witem, int n, int ngh, int split_target,
                                                         int max_chunks, int witems, int hkv) {
  __shared__ int part[1024], cpart[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int b = min(tid * per, n), e = min(b + per, n);
  int sum = 0, csum = 0;
  const int nslots = n / hkv;
  auto item = [&](int i) { return (i % nslots) * hkv + i / nslots; };   // KV-head-major position -> list
  for (int i = b; i < e; ++i) {
    sum += kcount[i] / ngh;
    csum += bwd_chunks(kcount[item(i)], split_target, max_chunks);
  }
  part[tid] = sum;
  cpart[tid] = csum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // inclusive scans of the thread sums
    const int v = tid >= off ? part[tid - off] : 0;
    const int cv = tid >= off ? cpart[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    cpart[tid] += cv;
    __syncthreads();
  }
  int run = part[tid] - sum, crun = cpart[tid] - csum;
  for (int i = b; i < e; ++i) {
    kptr[i] = run;
    run += kcount[i] / ngh;
    const int it = item(i);
    const int nc = bwd_chunks(kcount[it], split_target, max_chunks);
    for (int z = 0; z < nc; ++z) witem[crun + z] = (it << 4) | z;
    crun += nc;
  }
  if (tid == 1023) kptr[n] = part[1023];
  for (int w = cpart[1023] + tid; w < witems; w += 1024) witem[w] = -1;
}

// One wavefront per (key block slot x, KV head): the rows whose (sorted)
// lists hold block j, in visiting order (routing heads of the KV head, then
// query blocks ascending), written as r * nrh + hh to klist[kptr ..).  Each
// lane takes one candidate row of a run of 64 and binary-searches its list;
// a ballot orders the hits.  Slots the search does not fill (a worklist whose
// lists are not sorted and unique) are set to -1 and skipped.
__global__ void __launch_bounds__(256) bwd_klist_kernel(Geom g, BwdBufs a, int n) {
  const int idx = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (idx >= n) return;
  const int lane = threadIdx.x & 63;
  const int x = idx / g.hkv, kvh = idx % g.hkv;
  const KeySlot ks = key_slot(g, x);
  const int nrh = g.share ? 1 : g.group;
  const int rfirst = max(ks.j, g.qblk0);   // causal: only query blocks r >= j list block j
  const int p0 = a.kptr[idx], p1 = a.kptr[idx + 1];
  const uint64_t below = lanes_below();
  int w = p0;
  for (int hh = 0; hh < nrh; ++hh) {
    const int hr = g.share ? kvh : kvh * g.group + hh;
    for (int r0 = rfirst; r0 < ks.nb; r0 += 64) {
      const int r = r0 + lane;
      bool has = false;
      if (r < ks.nb) {
        const int64_t rw = row_id(g, ks.s, hr, r, ks.blk0, ks.nb);
        int lo = a.row_ptr[rw], hi = a.row_ptr[rw + 1] - 1;
        while (lo <= hi) {
          const int mid = (lo + hi) >> 1, cj = a.col_idx[mid];
          if (cj == ks.j) {
            has = true;
            break;
          }
          if (cj < ks.j) lo = mid + 1; else hi = mid - 1;
        }
      }
      const uint64_t m = __ballot(has);
      const int at = w + __popcll(m & below);
      if (has && at < p1) a.klist[at] = r * nrh + hh;
      w += __popcll(m);
    }
  }
  for (int t = w + lane; t < p1; t += 64) a.klist[t] = -1;
}

// One workgroup per (key block slot, KV head, chunk), 4 wavefronts: wave w
// owns keys 32 (w & 1) .. + 32 and query rows 32 (w >> 1) .. + 32 of every
// pair, forms that 32 x 32 block of S = Q K^T and dP = dO V^T (one key per
// lane) and accumulates dV^T += dO^T P and dK^T += Q^T dS for its keys over
// its query half; the halves are added through LDS at the end.  Each lane
// keeps its key's K row (the B operand of S) in registers for the whole
// workgroup; V is staged in LDS once.  The pairs come from the key-major list and stream
// through a ring of NB LDS buffers: a pair's Q, dO, lse and D go global ->
// LDS NB - 1 pairs ahead of its products, one barrier per pair.  A pair's
// rows past the sequence end load the last valid row (finite values, masked
// to zero weight).  A key block with more pairs than split_target is shared
// by up to max_chunks workgroups, each taking an equal run of its pairs: they
// add into fp32 accumulators with atomics and the last one to finish
// converts them.
__global__ void __launch_bounds__(256) bwd_dkdv_bf16_kernel(Geom g, BwdBufs a) {
  constexpr int NDB = 4, TILE = 64 * 256, NB = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char qd[NB][2][TILE];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(1024))) unsigned char vt[TILE];          // V of the key block
  __shared__ __attribute__((aligned(256))) float lds_ld[NB][2][64];          // [buffer][lse, D][query row]
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1, qh = wave >> 1;
  const int wi = a.witem[blockIdx.x];   // (slot x KV head) << 4 | chunk, or -1
  if (wi < 0) return;
  const int64_t kidx = wi >> 4;
  const int chunk = wi & 15;
  const int kvh = (int)(kidx % g.hkv);
  const int ngh = g.share ? g.group : 1;   // query heads per row
  const int nrh = g.share ? 1 : g.group;   // routing heads of the KV head
  const int e0 = a.kptr[kidx], nent = a.kptr[kidx + 1] - e0, units = nent * ngh;
  const int nch = bwd_chunks(units, a.split_target, a.max_chunks);
  const int ord_lo = (int)((int64_t)units * chunk / nch);
  const int ord_hi = (int)((int64_t)units * (chunk + 1) / nch);
  const KeySlot ksl = key_slot(g, (int)(kidx / g.hkv));
  const int s = ksl.s, j = ksl.j, len = ksl.len, tok0 = ksl.tok0;
  const int cnt = min(kBlock, len - j * kBlock);
  const int64_t kb = kv_block_offset(g, s, kvh, tok0, j);
  const float c = 0.08838834764831845f, cl2 = c * kLog2e;
  const int key = kh * 32 + l32, kpos = j * kBlock + key;

  // a pair's loads per wavefront: four 1 KB slices of the Q and of the dO
  // tile, and (waves 0, 1) the 64 lse / D values
  constexpr int LPP = 9;   // loads per pair, every wavefront (waves 2, 3 repeat their last slice)
  const unsigned char* const qbytes = (const unsigned char*)a.q;
  const unsigned char* const dbytes = (const unsigned char*)a.dout;
  auto slice_off = [&](int ii, int rows) {   // byte offset of this lane's slice ii (rows clamped)
    const int row = 4 * (wave + 4 * ii) + (lane >> 4), p = lane & 15;
    return (uint32_t)(min(row, rows - 1) * 256 + ((p ^ tsw(row)) << 4));
  };
  uint32_t ofull[4];   // a whole query block's offsets
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) ofull[ii] = slice_off(ii, kBlock);
  // element offsets of (head 0, token 0) of the sequence in Q / dO and in lse / D
  const int64_t qbase = q_offset(g, s, 0, tok0, 0), lbase = lse_offset(g, s, 0, tok0, 0);
  // entries of the list, 64 at a time in a register (lane i: entry base + i);
  // pair ord = entry e x ngh + query head gh, walked in order by a cursor
  int ce = ord_lo / ngh, cg = ord_lo - ce * ngh;
  int ebase = ce;
  int ent = ebase + lane < nent ? a.klist[e0 + ebase + lane] : -1;
  asm volatile("" ::"v"(ent));
  struct Pair {
    int r, head, qrows;
    bool ok;
  };
  auto next_pair = [&]() {
    Pair pr;
    if (ce - ebase >= 64) {   // uniform: refill the entry window
      ebase = ce;
      ent = ebase + lane < nent ? a.klist[e0 + ebase + lane] : -1;
      // consumed here, so no path reaches the loop's reads with it pending
      // (the compiler's wait insertion would otherwise wait for every load
      // in flight, the ring's prefetches included, on every pair)
      asm volatile("" ::"v"(ent));
    }
    const int v = __builtin_amdgcn_readlane(ent, ce - ebase);
    pr.ok = v >= 0;
    const int vv = pr.ok ? v : 0;   // a skipped entry still loads a valid tile (uniform wait counts)
    if (nrh == 1) {
      pr.r = vv;
      pr.head = kvh * g.group + cg;
    } else {
      pr.r = vv / nrh;
      pr.head = kvh * g.group + (vv - pr.r * nrh);
    }
    pr.qrows = min(kBlock, len - pr.r * kBlock);
    if (++cg == ngh) {
      cg = 0;
      ++ce;
    }
    return pr;
  };
  auto issue_pair = [&](const Pair& pr, int b) {
    const int64_t qo = (qbase + (int64_t)pr.head * g.q_head + (int64_t)(pr.r * kBlock * 128)) * 2;
    const unsigned char* qb = bwd_uniform(qbytes + qo);
    const unsigned char* db = bwd_uniform(dbytes + qo);
    if (pr.qrows == kBlock) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        bwd_load_lds16(qb, ofull[ii], &qd[b][0][(wave + 4 * ii) * 1024]);
        bwd_load_lds16(db, ofull[ii], &qd[b][1][(wave + 4 * ii) * 1024]);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t o = slice_off(ii, pr.qrows);
        bwd_load_lds16(qb, o, &qd[b][0][(wave + 4 * ii) * 1024]);
        bwd_load_lds16(db, o, &qd[b][1][(wave + 4 * ii) * 1024]);
      }
    }
    const int64_t lo = (lbase + (int64_t)pr.head * g.lse_head + pr.r * kBlock) * 4;
    const unsigned char* lb = bwd_uniform((const unsigned char*)(wave == 1 ? a.delta : a.nlse2) + lo);
    // waves 0 and 1 bring -lse log2(e) and D; waves 2 and 3 load the first
    // again into their own unused slot so every wavefront has LPP loads per pair
    bwd_load_lds4(lb, (uint32_t)min(lane, pr.qrows - 1) * 4,
                  (const unsigned char*)(wave < 2 ? &lds_ld[b][wave][0] : &lds_ld[b][0][0]));
  };

  // ring prologue: the first NB - 1 pairs, kept as a shift register of the
  // pairs whose loads are in flight (compile-time indices: it stays in registers)
  Pair pipe[NB - 1];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    pipe[u] = Pair{0, 0, 1, false};
    if (ord_lo + u < ord_hi) {
      pipe[u] = next_pair();
      issue_pair(pipe[u], u);
    }
  }
  // this lane's K row (row `key`, clamped into the block): the B operand of
  // S = Q K^T for d = 16 ks + 8 half .. + 8; and the block's V in LDS
  bf16x8 kreg[8];
  {
    const int krow = min(key, cnt - 1);
    const __bf16* kp = (const __bf16*)a.k + kb + (int64_t)krow * 128 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 16 * ks));
  }
  stage_tile<false, 256>(vt, (const __bf16*)a.v + kb, cnt, tid);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(kreg[ks]));

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  int bc = 0;   // ring buffer of pair ord: (ord - ord_lo) % NB
  for (int ord = ord_lo; ord < ord_hi; ++ord) {
    const int bn = bc == 0 ? NB - 1 : bc - 1;   // buffer of pair ord + NB - 1
    const int ahead = ord + NB - 1;   // the pair whose loads go out in this iteration
    Pair nxt = {0, 0, 1, false};
    if (ahead < ord_hi) nxt = next_pair();
    bwd_wait_pairs<LPP>(min(NB - 2, ord_hi - 1 - ord));   // this wave's loads of pair ord
    // every wave's loads of pair ord landed; buffer (ord - 1) % NB is read.  A
    // bare s_barrier: __syncthreads would also wait for the younger pairs' loads
    asm volatile("s_barrier" ::: "memory");
    if (ahead < ord_hi) issue_pair(nxt, bn);
    const Pair cur = pipe[0];
#pragma unroll
    for (int i = 0; i + 1 < NB - 1; ++i) pipe[i] = pipe[i + 1];
    pipe[NB - 2] = nxt;
    if (cur.ok) {
      const unsigned char* qt = qd[bc][0];
      const unsigned char* dot = qd[bc][1];
      const float* lse_s = lds_ld[bc][0];
      const float* del_s = lds_ld[bc][1];
      // S = Q K^T and dP = dO V^T: this wave's 32 query rows x 32 keys (one
      // key per lane); the Q and dO operands of step ks + 2 are read while
      // step ks multiplies (an order pinned with sched_group_barrier: left
      // alone the compiler reads each operand just before its MFMA)
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
      bf16x8 oq[3], od[3], ov[3];
      auto rd = [&](int ks) {
        oq[ks % 3] = row8<true>(qt, qh * 32 + l32, 2 * ks + half);
        od[ks % 3] = row8<true>(dot, qh * 32 + l32, 2 * ks + half);
        ov[ks % 3] = row8<false>(vt, key, 2 * ks + half);
      };
      rd(0);
      rd(1);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 2 < 8) rd(ks + 2);
        sacc = mfma(oq[ks % 3], kreg[ks], sacc);
        dpacc = mfma(od[ks % 3], ov[ks % 3], dpacc);
        if (ks + 2 < 8) __builtin_amdgcn_sched_group_barrier(kDsRead, 3, 0);
        __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
      }
      // -lse log2(e) and D of this lane's 16 query rows, four runs of 4 read
      // one run ahead.  Pairs below the diagonal with a whole query block need
      // no mask (every key precedes every query row)
      bf16x8 pb[2], dsb[2];
      auto weights = [&](auto full) {
        f32x4 lsv[2], dlv[2];
        lsv[0] = *reinterpret_cast<const f32x4*>(lse_s + qh * 32 + 4 * half);
        dlv[0] = *reinterpret_cast<const f32x4*>(del_s + qh * 32 + 4 * half);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          if (gq + 1 < 4) {
            lsv[(gq + 1) & 1] = *reinterpret_cast<const f32x4*>(lse_s + qh * 32 + 8 * (gq + 1) + 4 * half);
            dlv[(gq + 1) & 1] = *reinterpret_cast<const f32x4*>(del_s + qh * 32 + 8 * (gq + 1) + 4 * half);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * gq + e;
            const float x = fmaf(sacc[i], cl2, lsv[gq & 1][e]);
            float p;
            if constexpr (decltype(full)::value) {
              p = __builtin_amdgcn_exp2f(x);
            } else {
              const int q = qh * 32 + 8 * gq + 4 * half + e;
              const bool ok = q < cur.qrows && kpos <= cur.r * kBlock + q;
              // masked weights exponentiate -inf (no branch per element)
              p = __builtin_amdgcn_exp2f(ok ? x : -INFINITY);
            }
            pb[i / 8][i % 8] = (__bf16)p;
            dsb[i / 8][i % 8] = (__bf16)(p * (dpacc[i] - dlv[gq & 1][e]));
          }
        }
      };
      if (cur.r > j && cur.qrows == kBlock) weights(std::true_type{});
      else weights(std::false_type{});
      // dV^T += dO^T P and dK^T += Q^T dS: MFMA i takes d block i / 4, step
      // (i / 2) % 2, dV for even i and dK for odd; its transposed A operand
      // is read four MFMAs ahead
      auto ta_of = [&](int i) {
        return (i & 1) ? tr8(qt, qh, (i >> 1) & 1, i >> 2, lane) : tr8(dot, qh, (i >> 1) & 1, i >> 2, lane);
      };
      bf16x8 ta[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ta[i] = ta_of(i);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16x8 av = ta[i & 3];
        if (i + 4 < 16) ta[i & 3] = ta_of(i + 4);
        const int db = i >> 2, ks = (i >> 1) & 1;
        if (i & 1) dk[db] = mfma(av, dsb[ks], dk[db]);
        else dv[db] = mfma(av, pb[ks], dv[db]);
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        if (i + 4 < 16) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
      }
    }
    bc = bc == NB - 1 ? 0 : bc + 1;
  }
  // add the query halves: waves 2, 3 hand their sums to waves 0, 1 through
  // LDS (element-major, so the lanes of a store hit consecutive banks)
  // [16 NDB elements][2 key halves][64 lanes] = 32 KB
  float* red = reinterpret_cast<float*>(&qd[0][0][0]);   // 32 KB: ring buffer 0
  auto ri = [&](int e) { return (e * 2 + kh) * 64 + lane; };
  const bool out = key < cnt;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16 (&acc)[NDB] = pass == 0 ? dk : dv;
    __syncthreads();
    if (qh == 1)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[ri(db * 16 + i)] = acc[db][i];
    __syncthreads();
    if (qh == 0 && out) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] += red[ri(db * 16 + i)];
      const int64_t row0 = kb + (int64_t)key * 128;
      if (nch == 1) {
        __bf16* dst = (__bf16*)(pass == 0 ? a.dk : a.dv) + row0;
        const float sc = pass == 0 ? c : 1.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][4 * gq + e] * sc);
            *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * gq + 4 * half) = v4;
          }
      } else {   // shared block: add this run's sums into the fp32 accumulators
        float* dst = (pass == 0 ? a.dk_acc : a.dv_acc) + row0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            atomicAdd(dst + db * 32 + 8 * (i / 4) + 4 * half + (i % 4), acc[db][i]);
      }
    }
  }
  if (nch == 1) return;
  // the last of the block's workgroups converts the accumulated sums
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(a.kdone + kidx, 1) == nch - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int e = tid; e < cnt * 128; e += 256) {
    const float vk = __hip_atomic_load(a.dk_acc + kb + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float vv = __hip_atomic_load(a.dv_acc + kb + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ((__bf16*)a.dk)[kb + e] = (__bf16)(vk * c);
    ((__bf16*)a.dv)[kb + e] = (__bf16)vv;
  }
}

__global__ void __launch_bounds__(256) bwd_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

int launch_bwd(const Geom& g, int dtype, const BwdBufs& b, int64_t kv_elems, int kv_tail, hipStream_t st) {
  const unsigned fill_grid = (unsigned)std::min<int64_t>((kv_elems + 255) / 256, 65536);
  if (dtype == SA_BF16) {
    // keys past the sequence end (capacity tail) are never attended: dK = dV = 0
    if (kv_tail) {
      const int64_t words = kv_elems / 2;
      const unsigned zg = (unsigned)std::min<int64_t>((words + 255) / 256, 65536);
      bwd_zero_kernel<<<zg, 256, 0, st>>>((uint32_t*)b.dk, words);
      bwd_zero_kernel<<<zg, 256, 0, st>>>((uint32_t*)b.dv, words);
    }
    if (g.rows > 0) {
      const unsigned slots = g.varlen ? (unsigned)g.total_blocks : (unsigned)(g.batch * ((g.n + kBlock - 1) / kBlock));
      const int64_t counters = 2 * (int64_t)slots * g.hkv;   // kcount and kdone, adjacent
      bwd_zero_kernel<<<(unsigned)std::min<int64_t>((counters + 255) / 256, 65536), 256, 0, st>>>(
          (uint32_t*)b.kcount, counters);
      const int nk = (int)slots * g.hkv;   // (key block slot, KV head) lists
      bwd_count_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, st>>>(g, b);
      bwd_kscan_kernel<<<1, 1024, 0, st>>>(b.kcount, b.kptr, b.witem, nk, g.share ? g.group : 1, b.split_target,
                                           b.max_chunks, b.witems, g.hkv);
      bwd_klist_kernel<<<(unsigned)((nk + 3) / 4), 256, 0, st>>>(g, b, nk);
      bwd_split_clear_kernel<<<dim3(slots, (unsigned)g.hkv), 256, 0, st>>>(g, b);
      if (g.share && (g.hpr == 2 || g.hpr == 4 || g.hpr == 8))
        bwd_dq_rows_bf16_kernel<<<dim3((unsigned)g.rows, (unsigned)(g.hpr / 2)), 256, 0, st>>>(g, b);
      else
        bwd_dq_bf16_kernel<<<dim3((unsigned)g.rows, (unsigned)g.hpr), 128, 0, st>>>(g, b);
      bwd_dkdv_bf16_kernel<<<(unsigned)b.witems, 256, 0, st>>>(g, b);
    }
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
  }
  bwd_fill_kernel<<<fill_grid, 256, 0, st>>>(b.dk_acc, kv_elems);
  bwd_fill_kernel<<<fill_grid, 256, 0, st>>>(b.dv_acc, kv_elems);
  if (g.rows > 0)
    attn_bwd_simt_kernel<float, 64><<<dim3((unsigned)g.rows, (unsigned)g.hpr), 64, 0, st>>>(g, b);
  bwd_convert_kernel<float><<<fill_grid, 256, 0, st>>>(b.dk_acc, (float*)b.dk, kv_elems);
  bwd_convert_kernel<float><<<fill_grid, 256, 0, st>>>(b.dv_acc, (float*)b.dv, kv_elems);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
