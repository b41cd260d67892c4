// Split-KV decode over a worklist, then an Eq 3-5 merge of the split partials.
//
// [P2] §2.2 "decode": one query per step, the cost is reading the selected
// history K/V; [P3] "sparse softmax numerics": tiles (here: groups of tiles)
// produce partial (max, exp-sum, weighted value) states merged by [P2] Eq 3-5;
// [P3] "specialised kernels vs programmable abstraction": decode is bound by
// KV reads and launches.
//
// One wavefront per (row, split), row = (sequence, routing head); the row's
// query heads (the KV head's group when routing is shared) share every K/V
// tile it streams.  Per 64-key tile:
//   * S = Q K^T on v_mfma_f32_16x16x32_bf16 with the heads as the M dimension
//     (K goes straight from HBM into the B operand in 16-byte loads);
//   * softmax in the log2 domain, one lane per key, per-head max / sum by
//     wavefront reductions;
//   * P V on the vector ALU: lane = (8-column chunk, key phase), each 16-byte
//     V load feeds G * 8 FMAs; phases are summed once per split.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

size_t decode_partials_bytes(const Geom& g, int splits) {
  return (size_t)g.rows * splits * g.hpr * (g.d + 2) * sizeof(float);
}

template <int G>
__global__ void __launch_bounds__(64) decode_split_kernel(Geom g, FwdBufs a, int splits) {
  constexpr int D = 128;
  __shared__ float sbuf[16][64];    // S[head][key] (log2-scaled)
  __shared__ float pbuf[64][G];     // P[key][head]
  const int lane = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int64_t row = item / splits;
  const int sp = (int)(item % splits);
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  const int h0 = g.share ? ri.h * g.group : ri.h;
  const int t0 = a.row_ptr[row], nt = a.row_ptr[row + 1] - t0;
  const int per = (nt + splits - 1) / splits;
  const int tb = t0 + min(sp * per, nt), te = t0 + min((sp + 1) * per, nt);
  const __bf16* q = (const __bf16*)a.q;
  const __bf16* k = (const __bf16*)a.k;
  const __bf16* v = (const __bf16*)a.v;
  const float c2 = kLog2eD / sqrtf((float)D);

  // A operand: Q[head slot = lane % 16][d = 32 ks + 8 (lane / 16) .. +8]
  bf16x8 qa[4];
  {
    const int hs = lane % 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 x = {0, 0, 0, 0};
      if (hs < G) x = *reinterpret_cast<const u32x4*>(q + q_offset(g, ri.s, h0 + hs, 0, 0) + ks * 32 + (lane / 16) * 8);
      qa[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const int chunk = lane % 16, phase = lane / 16;

  for (int t = tb; t < te; ++t) {
    const int j = a.col_idx[t];
    const int cnt = min(kBlock, ri.len - j * kBlock);
    const __bf16* kb = k + kv_offset(g, ri.s, kvh, 0, j * kBlock);
    const __bf16* vb = v + kv_offset(g, ri.s, kvh, 0, j * kBlock);
    // V loads for this lane's 16 keys (issued before the QK products)
    u32x4 vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 4 * i + phase;
      vr[i] = key < cnt ? *reinterpret_cast<const u32x4*>(vb + key * D + chunk * 8) : u32x4{0, 0, 0, 0};
    }
    // S[head][key] for keys nb*16 + lane%16, heads 4*(lane/16) + i
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const int key = nb * 16 + (lane % 16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 x = key < cnt ? *reinterpret_cast<const u32x4*>(kb + key * D + ks * 32 + (lane / 16) * 8)
                            : u32x4{0, 0, 0, 0};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, x), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sbuf[4 * (lane / 16) + i][key] = sacc[i] * c2;
    }
    __syncthreads();
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = lane < cnt ? sbuf[h][lane] : -INFINITY;
      const float mt = wave_max(x);
      const float mnew = fmaxf(m[h], mt);
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      alpha[h] = exp2f(m[h] - msafe);
      const float p = exp2f(x - msafe);
      pbuf[lane][h] = p;
      l[h] = l[h] * alpha[h] + wave_sum(p);
      m[h] = mnew;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 4 * i + phase;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = pbuf[key][h];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = bf16_lo(vr[i][w]), hi = bf16_hi(vr[i][w]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * w] = fmaf(pv[h], lo, acc[h][2 * w]);
          acc[h][2 * w + 1] = fmaf(pv[h], hi, acc[h][2 * w + 1]);
        }
      }
    }
  }
  // sum the four key phases
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16, kWave);
      acc[h][e] += __shfl_xor(acc[h][e], 32, kWave);
    }
  float* part = a.part + ((int64_t)row * splits + sp) * G * (D + 2);
  if (phase == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      f32x4 u0, u1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u0[e] = acc[h][e];
        u1[e] = acc[h][4 + e];
      }
      float* ph = part + h * (D + 2);
      *reinterpret_cast<f32x4*>(ph + chunk * 8) = u0;
      *reinterpret_cast<f32x4*>(ph + chunk * 8 + 4) = u1;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      part[h * (D + 2) + D] = m[h];
      part[h * (D + 2) + D + 1] = l[h];
    }
  }
}

// Merge the split partials of one (row, head) with Eq 3-5 and normalise.
__global__ void __launch_bounds__(64) decode_merge_kernel(Geom g, FwdBufs a, int splits) {
  constexpr int D = 128;
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int hh = blockIdx.y;
  const RowInfo ri = decode_row(g, row);
  const int head = (g.share ? ri.h * g.group : ri.h) + hh;
  const int G = g.hpr;
  const float* base = a.part + (int64_t)row * splits * G * (D + 2) + hh * (D + 2);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, base[(int64_t)s * G * (D + 2) + D]);
  const float msafe = mx == -INFINITY ? 0.f : mx;
  float L = 0.f, u0 = 0.f, u1 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* ps = base + (int64_t)s * G * (D + 2);
    const float ms = ps[D];
    if (ms == -INFINITY) continue;
    const float w = exp2f(ms - msafe);
    L += w * ps[D + 1];
    u0 += w * ps[2 * lane];
    u1 += w * ps[2 * lane + 1];
  }
  const float inv = 1.f / L;
  __bf16* op = (__bf16*)a.o + q_offset(g, ri.s, head, 0, 0);
  op[2 * lane] = (__bf16)(u0 * inv);
  op[2 * lane + 1] = (__bf16)(u1 * inv);
  if (a.lse && lane == 0) a.lse[lse_offset(g, ri.s, head, 0, 0)] = msafe * kLn2 + logf(L);
}

int launch_decode(const Geom& g, int dtype, const FwdBufs& b, int splits, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (dtype == SA_F32) return launch_prefill(g, dtype, b, st);   // SIMT kernel handles decode
  if (g.d != 128) return SA_ERR_UNSUPPORTED;
  const unsigned items = (unsigned)(g.rows * splits);
  switch (g.hpr) {
    case 1: decode_split_kernel<1><<<items, 64, 0, st>>>(g, b, splits); break;
    case 2: decode_split_kernel<2><<<items, 64, 0, st>>>(g, b, splits); break;
    case 4: decode_split_kernel<4><<<items, 64, 0, st>>>(g, b, splits); break;
    case 8: decode_split_kernel<8><<<items, 64, 0, st>>>(g, b, splits); break;
    default: return SA_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  decode_merge_kernel<<<dim3((unsigned)g.rows, g.hpr), 64, 0, st>>>(g, b, splits);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
