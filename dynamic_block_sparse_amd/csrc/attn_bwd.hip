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
        const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sacc[b2][i], cl2, -lse2)) : 0.f;
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

// NW = 4 or 8 wavefronts: wave w owns keys 32 (w & 1) .. + 32, the 32 query
// rows 32 ((w >> 1) & 1) .. + 32 of every staged row and (NW = 8) one half of
// the d columns of the accumulators, so each wave forms one 32 x 32 block of S
// and dP per (row, head) (the two d halves form the same block) and
// accumulates dK^T, dV^T of its keys and columns over its query half; the two
// query halves are added through LDS at the end.
template <int NW>
__global__ void __launch_bounds__(64 * NW) bwd_dkdv_bf16_kernel(Geom g, BwdBufs a) {
  constexpr int NT = 64 * NW, NDB = 16 / NW;   // threads; 32-column d blocks per wave
  __shared__ __attribute__((aligned(16))) unsigned char kt[64 * 256], vt[64 * 256], qd[2][64 * 256];
  __shared__ float lse_s[64], del_s[64];
  unsigned char* qt = qd[0];
  unsigned char* dot = qd[1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int kh = w & 1, qh = (w >> 1) & 1, dh = w >> 2;
  const int kvh = blockIdx.y;
  // a key block listed by more than split_target (row, head) pairs is shared
  // by nch workgroups, each taking an equal run of its pairs in visiting order
  const int64_t kidx = (int64_t)blockIdx.x * g.hkv + kvh;
  const int units = a.kcount[kidx];
  const int nch = units > a.split_target ? min(a.max_chunks, (units + a.split_target - 1) / a.split_target) : 1;
  if ((int)blockIdx.z >= nch) return;
  const int ord_lo = (int)((int64_t)units * blockIdx.z / nch);
  const int ord_hi = (int)((int64_t)units * (blockIdx.z + 1) / nch);
  const KeySlot ksl = key_slot(g, (int)blockIdx.x);
  const int s = ksl.s, j = ksl.j, len = ksl.len, tok0 = ksl.tok0, blk0 = ksl.blk0, nb = ksl.nb;
  const int cnt = min(kBlock, len - j * kBlock);
  const int64_t kb = kv_block_offset(g, s, kvh, tok0, j);
  stage_tile<false, NT>(kt, (const __bf16*)a.k + kb, cnt, tid);
  stage_tile<false, NT>(vt, (const __bf16*)a.v + kb, cnt, tid);
  const float c = 0.08838834764831845f, cl2 = c * kLog2e;
  const int key = kh * 32 + l32, kpos = j * kBlock + key;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const int nrh = g.share ? 1 : g.group;   // routing heads whose rows may list this block
  const int ngh = g.share ? g.group : 1;   // query heads per row
  const int rfirst = max(j, g.qblk0);      // causal: only query blocks r >= j list block j
  int ord = 0;                             // visiting-order index of the next pair
  for (int hh = 0; hh < nrh && ord < ord_hi; ++hh) {
    const int hr = g.share ? kvh : kvh * g.group + hh;
    for (int r0 = rfirst; r0 < nb && ord < ord_hi; r0 += 64) {
      // one candidate row per lane: does its (sorted) list hold block j?
      const int r = r0 + lane;
      bool has = false;
      if (r < nb) {
        const int64_t rw = row_id(g, s, hr, r, blk0, nb);
        int lo = a.row_ptr[rw], hi = a.row_ptr[rw + 1] - 1;
        while (lo <= hi) {
          const int mid = (lo + hi) >> 1, cj = a.col_idx[mid];
          if (cj == j) { has = true; break; }
          if (cj < j) lo = mid + 1; else hi = mid - 1;
        }
      }
      uint64_t m = __ballot(has);
      const int in_m = __popcll(m) * ngh;
      if (ord + in_m <= ord_lo) {   // all before this workgroup's run
        ord += in_m;
        continue;
      }
      while (m) {
        const int rr = r0 + __builtin_ctzll(m);
        m &= m - 1;
        const int qrows = min(kBlock, len - rr * kBlock);
        for (int gh = 0; gh < ngh; ++gh, ++ord) {
          if (ord < ord_lo || ord >= ord_hi) continue;
          const int head = g.share ? kvh * g.group + gh : hr;
          const int64_t qo = q_offset(g, s, head, tok0, rr * kBlock);
          __syncthreads();   // the previous pair's tiles are no longer read
          stage_tile<true, NT>(qt, (const __bf16*)a.q + qo, qrows, tid);
          stage_tile<true, NT>(dot, (const __bf16*)a.dout + qo, qrows, tid);
          if (tid < 64) {
            const bool ok = tid < qrows;
            const int64_t lo = ok ? lse_offset(g, s, head, tok0, rr * kBlock + tid) : 0;
            lse_s[tid] = ok ? a.lse[lo] * kLog2e : 0.f;
            del_s[tid] = ok ? a.delta[lo] : 0.f;
          }
          __syncthreads();
          // S = Q K^T and dP = dO V^T: this wave's 32 query rows x 32 keys (one key per lane)
          f32x16 sacc, dpacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.f;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            sacc = mfma(row8<true>(qt, qh * 32 + l32, 2 * ks + half), row8<false>(kt, key, 2 * ks + half), sacc);
            dpacc = mfma(row8<true>(dot, qh * 32 + l32, 2 * ks + half), row8<false>(vt, key, 2 * ks + half),
                         dpacc);
          }
          bf16x8 pb[2], dsb[2];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = qh * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            const bool ok = q < qrows && kpos <= rr * kBlock + q;
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sacc[i], cl2, -lse_s[q])) : 0.f;
            pb[i / 8][i % 8] = (__bf16)p;
            dsb[i / 8][i % 8] = (__bf16)(p * (dpacc[i] - del_s[q]));
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              dv[db] = mfma(tr8(dot, qh, ks, dh * NDB + db, lane), pb[ks], dv[db]);
              dk[db] = mfma(tr8(qt, qh, ks, dh * NDB + db, lane), dsb[ks], dk[db]);
            }
        }
      }
    }
  }
  // add the query halves: waves 2, 3 hand their sums to waves 0, 1 through
  // LDS (element-major, so the lanes of a store hit consecutive banks)
  // [16 NDB elements][2 key halves][NW / 4 d halves][64 lanes] = 32 KB
  float* red = reinterpret_cast<float*>(&qd[0][0]);
  auto ri = [&](int e) { return ((e * 2 + kh) * (NW / 4) + dh) * 64 + lane; };
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
            *reinterpret_cast<bf16x4*>(dst + (dh * NDB + db) * 32 + 8 * gq + 4 * half) = v4;
          }
      } else {   // shared block: add this run's sums into the fp32 accumulators
        float* dst = (pass == 0 ? a.dk_acc : a.dv_acc) + row0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            atomicAdd(dst + (dh * NDB + db) * 32 + 8 * (i / 4) + 4 * half + (i % 4), acc[db][i]);
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
  for (int e = tid; e < cnt * 128; e += NT) {
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
      bwd_count_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, st>>>(g, b);
      bwd_split_clear_kernel<<<dim3(slots, (unsigned)g.hkv), 256, 0, st>>>(g, b);
      bwd_dq_bf16_kernel<<<dim3((unsigned)g.rows, (unsigned)g.hpr), 128, 0, st>>>(g, b);
      bwd_dkdv_bf16_kernel<4><<<dim3(slots, (unsigned)g.hkv, (unsigned)b.max_chunks), 256, 0, st>>>(g, b);
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
