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
// One wavefront per (worklist row, query head), one lane per query row
// (fp32 arithmetic throughout).  Per listed tile the K, V tiles are staged in
// LDS (in the input dtype, lossless), each lane forms its row of P and dS
// over the tile's 64 keys, accumulates dQ in registers and writes P and dS
// transposed to LDS; then lane t takes key t and reduces dV_t = sum_i P_it
// dO_i and dK_t = c sum_i dS_it q_i over the row's 64 queries (Q and dO rows
// staged once per row), in chunks of 32 columns, and adds them to fp32
// accumulators with atomics: a key block is listed by many rows (and, with
// shared GQA routing, by every query head of the group).  A last pass
// converts the accumulators to the output dtype.
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

template <typename T, int D>
__global__ void __launch_bounds__(64) attn_bwd_kernel(Geom g, BwdBufs a) {
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

int launch_bwd(const Geom& g, int dtype, const BwdBufs& b, int64_t kv_elems, hipStream_t st) {
  const unsigned fill_grid = (unsigned)std::min<int64_t>((kv_elems + 255) / 256, 65536);
  bwd_fill_kernel<<<fill_grid, 256, 0, st>>>(b.dk_acc, kv_elems);
  bwd_fill_kernel<<<fill_grid, 256, 0, st>>>(b.dv_acc, kv_elems);
  if (g.rows > 0) {
    const dim3 grid((unsigned)g.rows, (unsigned)g.hpr);
    if (dtype == SA_BF16)
      attn_bwd_kernel<__bf16, 128><<<grid, 64, 0, st>>>(g, b);
    else
      attn_bwd_kernel<float, 64><<<grid, 64, 0, st>>>(g, b);
  }
  if (dtype == SA_BF16) {
    bwd_convert_kernel<__bf16><<<fill_grid, 256, 0, st>>>(b.dk_acc, (__bf16*)b.dk, kv_elems);
    bwd_convert_kernel<__bf16><<<fill_grid, 256, 0, st>>>(b.dv_acc, (__bf16*)b.dv, kv_elems);
  } else {
    bwd_convert_kernel<float><<<fill_grid, 256, 0, st>>>(b.dk_acc, (float*)b.dk, kv_elems);
    bwd_convert_kernel<float><<<fill_grid, 256, 0, st>>>(b.dv_acc, (float*)b.dv, kv_elems);
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
