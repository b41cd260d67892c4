// Prefill block-sparse attention over a worklist.
//
// [P2] §1.2 Eq 2: S = Q_r K_j^T / sqrt(d) per selected tile; the causal,
// padding and sequence masks apply before the softmax ([P2] §1.2, §2.1 causal
// boundary, §4.1); tiles merge with the online softmax of Eq 3-5 and the output
// is u / l.  [P3] "sparse softmax numerics": per-tile max / exp-sum / weighted
// value combined across non-contiguous tiles.
//
// bf16 path (d = 128), one workgroup per worklist row:
//   * the row covers HPR query heads (the KV head's group when routing is
//     shared, else one head) x 64 query rows; 2*HPR wavefronts, each owning 32
//     query rows of one head, so every gathered K/V tile is loaded once into
//     LDS and read by all of the row's heads;
//   * the products are computed transposed: S^T = K Q^T and O^T = V^T P^T on
//     v_mfma_f32_32x32x16_bf16.  In that form every lane owns one query row of
//     both accumulators, so the row max, exp-sum and rescale need no
//     cross-lane traffic except one swap between the two half-waves, and the
//     S^T accumulator converts in place into the P^T operand;
//   * K is staged row-major, V transposed (V^T), each with an XOR swizzle on
//     16-byte / 8-byte units so the MFMA operand reads are bank-conflict free;
//   * tiles are visited in the worklist's ascending address order ([P2] §1.2).
// fp32 path: a plain SIMT kernel (one lane per query row), exact-fp32 softmax.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

// --------------------------------------------------------------------------
// bf16 MFMA prefill kernel (d = 128).
template <int HPR>
__global__ void __launch_bounds__(128 * HPR) prefill_bf16_kernel(Geom g, FwdBufs a) {
  constexpr int D = 128;
  constexpr int NT = 128 * HPR;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * 64 * D * 2];
  unsigned char* kt = lds;                 // K  [64 keys][128 d]  16-byte units swizzled
  unsigned char* vt = lds + 64 * D * 2;    // V^T [128 d][64 keys]  8-byte units swizzled

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t row = a.row_perm[g.rows - 1 - (int64_t)blockIdx.x];   // longest rows first
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  const int head = (g.share ? ri.h * g.group : ri.h) + wave / 2;
  const int half = lane / 32, l32 = lane % 32;
  const int qpos = ri.r * kBlock + (wave % 2) * 32 + l32;    // this lane's query token
  const bool qvalid = qpos < ri.len;
  const __bf16* q = (const __bf16*)a.q;
  const __bf16* k = (const __bf16*)a.k;
  const __bf16* v = (const __bf16*)a.v;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qpos][16 ks + 8 half .. +8]
  bf16x8 qreg[8];
  {
    const __bf16* qp = q + q_offset(g, ri.s, head, ri.tok0, qvalid ? qpos : 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = qvalid ? *reinterpret_cast<const u32x4*>(qp + ks * 16 + half * 8) : u32x4{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const float c2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float m = -INFINITY, lsum = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};

  const int t_begin = a.row_ptr[row], t_end = a.row_ptr[row + 1];
  for (int t = t_begin; t < t_end; ++t) {
    const int j = a.col_idx[t];
    const int cnt = min(kBlock, ri.len - j * kBlock);     // valid keys in the tile
    __syncthreads();   // previous tile fully consumed
    {
      const __bf16* kb = k + kv_offset(g, ri.s, kvh, ri.tok0, j * kBlock);
      for (int qi = tid; qi < 64 * 16; qi += NT) {
        const int key = qi >> 4, c = qi & 15;
        u32x4 x = key < cnt ? *reinterpret_cast<const u32x4*>(kb + key * D + c * 8) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(kt + key * 256 + ((c ^ (key & 15)) << 4)) = x;
      }
      const __bf16* vb = v + kv_offset(g, ri.s, kvh, ri.tok0, j * kBlock);
      for (int p = tid; p < 256; p += NT) {
        const int kq = p >> 4, c = p & 15;
        u32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kq * 4 + i;
          x[i] = key < cnt ? *reinterpret_cast<const u32x4*>(vb + key * D + c * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int w = dd >> 1;
          uint32_t lo, hi;
          if (dd & 1) {
            lo = (x[0][w] >> 16) | (x[1][w] & 0xffff0000u);
            hi = (x[2][w] >> 16) | (x[3][w] & 0xffff0000u);
          } else {
            lo = (x[0][w] & 0xffffu) | (x[1][w] << 16);
            hi = (x[2][w] & 0xffffu) | (x[3][w] << 16);
          }
          const int d = c * 8 + dd;
          const int sw = (d & 15) ^ (d >> 4);
          *reinterpret_cast<u32x2*>(vt + d * 128 + ((kq ^ sw) << 3)) = u32x2{lo, hi};
        }
      }
    }
    __syncthreads();

    // S^T[key][row] for keys kb*32 + (8*(i/4) + 4*half + i%4), row = l32
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int key = kb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int c = ks * 2 + half;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(kt + key * 256 + ((c ^ (key & 15)) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[ks], sacc[kb], 0, 0, 0);
      }
    }
    // masks: only the diagonal tile (causal) or a tile past the sequence end
    if (j == ri.r || j * kBlock + kBlock > ri.len) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kpos = j * kBlock + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          if (kpos > qpos || kpos >= ri.len) sacc[kb][i] = -INFINITY;
        }
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float mnew = fmaxf(m, mt);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f((m - msafe) * c2);
    const float moff = -msafe * c2;
    float rs = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(fmaf(sacc[kb][i], c2, moff));
        rs += p;
        pb[kb][i / 8][i % 8] = (__bf16)p;
      }
    }
    rs += __shfl_xor(rs, 32, kWave);
    lsum = lsum * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T[d][row] += V^T[d][keys] P^T[keys][row]; k-slot (half, e) of step
    // (kb, ks) is key kb*32 + 16 ks + 8 (e/4) + 4 half + e%4, matching the
    // P^T values this lane holds in sacc[kb][8 ks + e].
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + l32;
      const int sw = (d & 15) ^ (d >> 4);
      const unsigned char* vrow = vt + d * 128;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int u1 = 8 * kb + 4 * ks + half;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + ((u1 ^ sw) << 3));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (((u1 + 2) ^ sw) << 3));
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kb][ks], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  if (qvalid) {
    const float inv = 1.f / lsum;
    __bf16* op = (__bf16*)a.o + q_offset(g, ri.s, head, ri.tok0, qpos);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[db][i4 * 4 + e] * inv);
        const int d = db * 32 + 8 * i4 + 4 * half;
        *reinterpret_cast<bf16x4*>(op + d) = ov;
      }
    }
    if (a.lse && half == 0)
      a.lse[lse_offset(g, ri.s, head, ri.tok0, qpos)] = m * 0.08838834764831845f + logf(lsum);
  }
}

// --------------------------------------------------------------------------
// fp32 SIMT kernel: one wavefront per (row, head), one lane per query row.
// Used for fp32 problems (prefill and decode); exact fp32 exp.
template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(Geom g, FwdBufs a) {
  __shared__ float ks[64][D + 1];
  __shared__ float vs[64][D];
  const int lane = threadIdx.x;
  const int64_t row = a.row_perm[g.rows - 1 - (int64_t)blockIdx.x];
  const RowInfo ri = decode_row(g, row);
  const int head = (g.share ? ri.h * g.group : ri.h) + blockIdx.y;
  const int kvh = head / g.group;
  const bool dec = g.mode == SA_DECODE;
  const int qpos = dec ? ri.len - 1 : ri.r * kBlock + lane;
  const bool qvalid = dec ? lane == 0 : qpos < ri.len;
  const float* q = (const float*)a.q;
  const float* k = (const float*)a.k;
  const float* v = (const float*)a.v;
  const float scale = 1.0f / sqrtf((float)D);

  float qr[D], o[D];
  const float* qp = q + q_offset(g, ri.s, head, ri.tok0, dec ? 0 : (qvalid ? qpos : 0));
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = qvalid ? qp[e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = a.row_ptr[row]; t < a.row_ptr[row + 1]; ++t) {
    const int j = a.col_idx[t];
    const int cnt = min(kBlock, ri.len - j * kBlock);
    __syncthreads();
    const float* kb = k + kv_offset(g, ri.s, kvh, ri.tok0, j * kBlock);
    const float* vb = v + kv_offset(g, ri.s, kvh, ri.tok0, j * kBlock);
    for (int e = lane; e < 64 * D; e += 64) {
      const int key = e / D, dd = e % D;
      ks[key][dd] = key < cnt ? kb[e] : 0.f;
      vs[key][dd] = key < cnt ? vb[e] : 0.f;
    }
    __syncthreads();
    float s[64];
    float mt = -INFINITY;
    for (int key = 0; key < 64; ++key) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = fmaf(qr[e], ks[key][e], acc);
      const int kpos = j * kBlock + key;
      const bool ok = kpos < ri.len && (dec || kpos <= qpos);
      s[key] = ok ? acc * scale : -INFINITY;
      mt = fmaxf(mt, s[key]);
    }
    const float mnew = fmaxf(m, mt);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = expf(m - msafe);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
    for (int key = 0; key < 64; ++key) {
      const float p = expf(s[key] - msafe);
      rs += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[key][e], o[e]);
    }
    l = l * alpha + rs;
    m = mnew;
  }
  if (qvalid) {
    float* op = (float*)a.o + q_offset(g, ri.s, head, ri.tok0, dec ? 0 : qpos);
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) op[e] = o[e] * inv;
    if (a.lse) a.lse[lse_offset(g, ri.s, head, ri.tok0, dec ? 0 : qpos)] = m + logf(l);
  }
}

int launch_f32(const Geom& g, const FwdBufs& b, hipStream_t st) {
  dim3 grid((unsigned)g.rows, g.hpr);
  if (g.d == 64)
    attn_f32_kernel<64><<<grid, 64, 0, st>>>(g, b);
  else
    attn_f32_kernel<128><<<grid, 64, 0, st>>>(g, b);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int launch_prefill(const Geom& g, int dtype, const FwdBufs& b, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (dtype == SA_F32) return launch_f32(g, b, st);
  if (g.d != 128) return SA_ERR_UNSUPPORTED;
  dim3 grid((unsigned)g.rows);
  switch (g.hpr) {
    case 1: prefill_bf16_kernel<1><<<grid, 128, 0, st>>>(g, b); break;
    case 2: prefill_bf16_kernel<2><<<grid, 256, 0, st>>>(g, b); break;
    case 4: prefill_bf16_kernel<4><<<grid, 512, 0, st>>>(g, b); break;
    default: return SA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
