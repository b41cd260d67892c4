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
// tile it streams.  Per 64-key tile, with the heads as the N dimension of
// v_mfma_f32_16x16x32_bf16 (16 slots, the first G used):
//   * S^T = K Q^T: K goes straight from HBM into the A operand in 16-byte
//     loads (key = lane % 16 of each 16-key block), so each lane ends up
//     with 16 scores of one head;
//   * softmax in the log2 domain: the per-head max / sum over 64 keys is the
//     lane's own 16 values plus two cross-row swaps;
//   * O^T = V^T P^T: V is copied HBM -> LDS with 16-byte global->LDS loads
//     (16 KB per wavefront, chunk-swizzled) and read back transposed with
//     ds_read_b64_tr_b16; P^T is the S^T accumulator converted in place.
// Up to ten wavefronts per CU (LDS-bound) keep ~300 KB of loads in flight.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFusedSplits = 8;   // up to this many splits merge inside one workgroup

size_t decode_partials_bytes(const Geom& g, int splits) {
  if (splits <= kFusedSplits) return 0;   // states merge in LDS
  return (size_t)g.rows * splits * g.hpr * (g.d + 2) * sizeof(float);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define SA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ void dec_load_lds16(const void* g, const unsigned char* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SA_LDS const unsigned char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void dec_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// V rows: the 8 rows two 16-lane groups read together map to 16 distinct slots
__device__ __forceinline__ int dec_vsw(int key) { return (key & 7) << 1; }

// Partial state of one split of a row, per lane: oacc[db][i] = u of head
// slot lane % 16 at d = 16 db + 4 (lane / 16) + i; m, l of that head slot.
struct DecodePartial {
  f32x4 oacc[8];
  float m, l;
};

// Stream tiles [tb, te) of split sp of `row` (one wavefront; vt = its 16 KB
// of LDS for the V tile) and return its unnormalised state.
template <int G>
__device__ __forceinline__ void decode_split(const Geom& g, const FwdBufs& a, int64_t row, int sp, int splits,
                                             unsigned char* vt, DecodePartial& out) {
  constexpr int D = 128;
  const int lane = threadIdx.x % kWave;
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  const int h0 = g.share ? ri.h * g.group : ri.h;
  const int t0 = a.row_ptr[row], nt = a.row_ptr[row + 1] - t0;
  const int per = (nt + splits - 1) / splits;
  const int tb = min(sp * per, nt), te = min((sp + 1) * per, nt);
  const __bf16* q = (const __bf16*)a.q;
  const unsigned char* kbytes = (const unsigned char*)a.k;
  const unsigned char* vbytes = (const unsigned char*)a.v;
  const float c2 = kLog2eD / sqrtf((float)D);
  const int hs = lane & 15, grp = lane >> 4;

  // tile ids of this split, one per lane (a split holds at most 64 tiles), and
  // for a paged cache their pages, looked up once here rather than per tile
  const int jl = tb + lane < te ? a.col_idx[t0 + tb + lane] : 0;
  const int pgl = g.block_table && tb + lane < te ? g.block_table[(int64_t)ri.s * g.table_stride + jl] : 0;

  // B operand of S^T = K Q^T: Q[head slot = lane % 16][d = 32 ks + 8 grp .. +8]
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 x = {0, 0, 0, 0};
    if (hs < g.hpr) x = *reinterpret_cast<const u32x4*>(q + q_offset(g, ri.s, h0 + hs, 0, 0) + ks * 32 + grp * 8);
    qb[ks] = __builtin_bit_cast(bf16x8, x);
  }
  const float grow = 8.0f;   // log2 headroom before the running max must move
  float m = -INFINITY, l = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < te - tb; ++t) {
    const int j = __builtin_amdgcn_readlane(jl, t);
    const int cnt = min(kBlock, ri.len - j * kBlock);
    const int64_t off = (g.block_table ? page_offset(g, __builtin_amdgcn_readlane(pgl, t), kvh)
                                       : kv_offset(g, ri.s, kvh, 0, j * kBlock)) * 2;
    // K: A operand of S^T, key = 16 mb + lane % 16, d = 32 ks + 8 grp.  The
    // tile's four 16-key blocks are fetched in two halves (the second after
    // the first half's MFMAs are issued): at 3 wavefronts per SIMD the
    // kernel has 168 VGPRs, and a whole tile of K operands would spill, and
    // a scratch reload waits for every load in flight.
    u32x4 kr[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int key = min(16 * mb + hs, cnt - 1);   // rows past the end: any valid row (masked)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kr[mb][ks] = *reinterpret_cast<const u32x4*>(kbytes + off + key * 256 + ks * 64 + grp * 16);
    }
    // V: HBM -> LDS, 16 wave loads of 1 KB (4 key rows each)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 4 * i + grp;
      const int kc = min(key, cnt - 1);
      dec_load_lds16(vbytes + off + kc * 256 + (((lane & 15) ^ dec_vsw(key)) << 4), vt + i * 1024);
    }
    // S^T[key = 16 mb + 4 grp + i][head = lane % 16]
    f32x4 sacc[4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (hb == 1) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int key = min(16 * (mb + 2) + hs, cnt - 1);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            kr[mb][ks] = *reinterpret_cast<const u32x4*>(kbytes + off + key * 256 + ks * 64 + grp * 16);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sacc[2 * hb + mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sacc[2 * hb + mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[mb][ks]), qb[ks],
                                                                    sacc[2 * hb + mb], 0, 0, 0);
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[mb][i] * c2;
        if (16 * mb + 4 * grp + i >= cnt) x = -INFINITY;
        sacc[mb][i] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = max_xor32(max_xor16(mt));
    if (__any(mt > m + grow)) {
      const float mnew = fmaxf(m, mt);
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m - msafe);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
      m = mnew;
    }
    const float moff = m == -INFINITY ? 0.f : m;
    float rs = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[mb][i] - moff);
        rs += p;
        pb[mb >> 1][(mb & 1) * 4 + i] = (__bf16)p;
      }
    }
    l += sum_xor32(sum_xor16(rs));
    dec_wait_vmcnt<0>();   // V landed in LDS
    // O^T[d = 16 db + 4 grp + i][head] += V^T P^T; k-slot (grp, e) of step ks
    // is key 32 ks + 16 (e / 4) + 4 grp + e % 4, as held in sacc[2 ks + e / 4][e % 4]
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + 4 * (hs & 3);
      const int chunk = d >> 3, h8 = (d >> 2) & 1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int key0 = 32 * ks + 4 * grp + (hs >> 2);
        const int key1 = key0 + 16;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SA_LDS i16x4*)(vt + key0 * 256 + ((chunk ^ dec_vsw(key0)) << 4) + h8 * 8));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (SA_LDS i16x4*)(vt + key1 * 256 + ((chunk ^ dec_vsw(key1)) << 4) + h8 * 8));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[ks], oacc[db], 0, 0, 0);
      }
    }
    // the next tile's V loads overwrite vt: every transpose read above has
    // returned (the MFMAs consumed them), so no further wait is needed
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) out.oacc[db] = oacc[db];
  out.m = m;
  out.l = l;
}

// Write a lane's share of a split state: slot hs < nh (the row's heads) of
// `dst`, laid out as [head][D + 2] floats (u[0..D), m, l).
__device__ __forceinline__ void store_partial(float* dst, const DecodePartial& st, int lane, int nh) {
  constexpr int D = 128;
  const int hs = lane & 15, grp = lane >> 4;
  if (hs < nh) {
    float* ph = dst + hs * (D + 2);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4*>(ph + 16 * db + 4 * grp) = st.oacc[db];
    if (grp == 0) {
      ph[D] = st.m;
      ph[D + 1] = st.l;
    }
  }
}

// Eq 3-5 merge of `splits` states of one head (stride between splits:
// `sstride` floats) for d = 2 e, 2 e + 1; writes o (and lse when e == 0).
__device__ __forceinline__ void merge_states(const Geom& g, const FwdBufs& a, const RowInfo& ri, int head,
                                             const float* base, int64_t sstride, int splits, int e) {
  constexpr int D = 128;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, base[s * sstride + D]);
  const float msafe = mx == -INFINITY ? 0.f : mx;
  float L = 0.f, u0 = 0.f, u1 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* ps = base + s * sstride;
    const float ms = ps[D];
    if (ms == -INFINITY) continue;
    const float w = exp2f(ms - msafe);
    L += w * ps[D + 1];
    u0 += w * ps[2 * e];
    u1 += w * ps[2 * e + 1];
  }
  const float inv = 1.f / L;
  __bf16* op = (__bf16*)a.o + q_offset(g, ri.s, head, 0, 0);
  op[2 * e] = (__bf16)(u0 * inv);
  op[2 * e + 1] = (__bf16)(u1 * inv);
  if (a.lse && e == 0) a.lse[lse_offset(g, ri.s, head, 0, 0)] = msafe * kLn2 + logf(L);
}

// One wavefront per (row, split); partial states go to the workspace and
// decode_merge_kernel combines them.  Used for more than kFusedSplits splits.
template <int G>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) decode_split_kernel(Geom g, FwdBufs a, int splits) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) unsigned char vt[64 * D * 2];
  const int64_t row = blockIdx.x / splits;
  const int sp = (int)(blockIdx.x % splits);
  DecodePartial st;
  decode_split<G>(g, a, row, sp, splits, vt, st);
  store_partial(a.part + ((int64_t)row * splits + sp) * g.hpr * (D + 2), st, threadIdx.x, g.hpr);
}

// One workgroup per row, one wavefront per split (splits <= kFusedSplits),
// each with its own 16 KB LDS slice for V tiles.  The split states meet in
// LDS (each wavefront overwrites its own slice once its tiles are done) and
// the workgroup merges them: no workspace round trip and no second launch.
template <int G>
__global__ void __launch_bounds__(64 * kFusedSplits) __attribute__((amdgpu_waves_per_eu(3)))
decode_fused_kernel(Geom g, FwdBufs a) {
  constexpr int D = 128, SLICE = 64 * D * 2;
  extern __shared__ __attribute__((aligned(1024))) unsigned char dyn_lds[];
  const int splits = blockDim.x / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int64_t row = blockIdx.x;
  unsigned char* slice = dyn_lds + wave * SLICE;
  DecodePartial st;
  decode_split<G>(g, a, row, wave, splits, slice, st);
  store_partial(reinterpret_cast<float*>(slice), st, lane, g.hpr);
  __syncthreads();
  const RowInfo ri = decode_row(g, row);
  const int h0 = g.share ? ri.h * g.group : ri.h;
  for (int item = threadIdx.x; item < g.hpr * (D / 2); item += blockDim.x) {
    const int hh = item / (D / 2), e = item % (D / 2);
    merge_states(g, a, ri, h0 + hh, reinterpret_cast<const float*>(dyn_lds) + hh * (D + 2), SLICE / 4, splits, e);
  }
}

// Merge the split partials of one (row, head) with Eq 3-5 and normalise.
__global__ void __launch_bounds__(64) decode_merge_kernel(Geom g, FwdBufs a, int splits) {
  constexpr int D = 128;
  const int64_t row = blockIdx.x;
  const int hh = blockIdx.y;
  const RowInfo ri = decode_row(g, row);
  const int head = (g.share ? ri.h * g.group : ri.h) + hh;
  const int G = g.hpr;
  const float* base = a.part + (int64_t)row * splits * G * (D + 2) + hh * (D + 2);
  merge_states(g, a, ri, head, base, (int64_t)G * (D + 2), splits, threadIdx.x);
}

// Head slots of the 16-slot MFMA N dimension a kernel instance covers: the
// smallest of 1, 2, 4, 8, 16 holding the row's query heads (0: more than 16).
static int head_slots(int hpr) {
  for (int s = 1; s <= 16; s *= 2)
    if (hpr <= s) return s;
  return 0;
}

int launch_decode(const Geom& g, int dtype, const FwdBufs& b, int splits, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (dtype == SA_F32) return launch_prefill(g, dtype, b, st);   // SIMT kernel handles decode
  if (g.d != 128) return SA_ERR_UNSUPPORTED;
  if (splits <= kFusedSplits) {
    const unsigned threads = (unsigned)(64 * splits);
    const size_t lds = (size_t)splits * 64 * 128 * 2;
    const unsigned rows = (unsigned)g.rows;
    switch (head_slots(g.hpr)) {
      case 1: decode_fused_kernel<1><<<rows, threads, lds, st>>>(g, b); break;
      case 2: decode_fused_kernel<2><<<rows, threads, lds, st>>>(g, b); break;
      case 4: decode_fused_kernel<4><<<rows, threads, lds, st>>>(g, b); break;
      case 8: decode_fused_kernel<8><<<rows, threads, lds, st>>>(g, b); break;
      case 16: decode_fused_kernel<16><<<rows, threads, lds, st>>>(g, b); break;
      default: return SA_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
  }
  const unsigned items = (unsigned)(g.rows * splits);
  switch (head_slots(g.hpr)) {
    case 1: decode_split_kernel<1><<<items, 64, 0, st>>>(g, b, splits); break;
    case 2: decode_split_kernel<2><<<items, 64, 0, st>>>(g, b, splits); break;
    case 4: decode_split_kernel<4><<<items, 64, 0, st>>>(g, b, splits); break;
    case 8: decode_split_kernel<8><<<items, 64, 0, st>>>(g, b, splits); break;
    case 16: decode_split_kernel<16><<<items, 64, 0, st>>>(g, b, splits); break;
    default: return SA_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  decode_merge_kernel<<<dim3((unsigned)g.rows, g.hpr), 64, 0, st>>>(g, b, splits);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
