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
#include <algorithm>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

// --------------------------------------------------------------------------
// bf16 MFMA prefill kernel (d = 128).
//
// LDS per stage: K [64 keys][128 d] and V [64 keys][128 d], both row-major in
// 16-byte chunks with an XOR swizzle on the chunk index, filled straight from
// HBM with 16-byte global->LDS loads (no staging registers; the swizzle is
// applied by permuting the per-lane source addresses).  The lock-step kernel
// keeps one stage and overlaps the next tile's K and this tile's V with the
// products; the ping-pong kernel keeps 4-deep K and V rings.  V^T operands
// come from the LDS transpose read (ds_read_b64_tr_b16): in each 16-lane group
// it returns, to lane i, the i-th column of the 4 x 16 block that the group's
// lanes read row-wise.

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define SA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int ksw(int key) { return key & 15; }
// V rows: the four rows a transpose read touches land in distinct bank groups
__device__ __forceinline__ int vsw(int key) { return ((key & 3) << 2) + ((key & 2)); }

// 16-byte global->LDS load: lane l's 16 bytes, read from base + off (base a
// wave-uniform address in SGPRs, off the lane's 32-bit byte offset), land at
// lds_wave_base + 16 l.  The tile loops keep every lane's offset in a register
// for the whole row, so a tile's loads take no vector address arithmetic.
// Issued as inline assembly so that the compiler's wait-count insertion does
// not treat every later LDS read as dependent on it (it would otherwise wait
// for all loads, including the next tile's prefetch); the kernel waits for
// these loads explicitly with wait_vmcnt before each barrier.
__device__ __forceinline__ void load_lds16_sv(const unsigned char* base, uint32_t off,
                                              const unsigned char* lds_wave_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(SA_LDS const unsigned char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

// A wave-uniform pointer the compiler cannot prove uniform, moved to SGPRs.
__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const unsigned char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block -> position in the worklist's (longest-first) row order.  Runs of G
// consecutive rows (same KV head, neighbouring query blocks) go to one XCD:
// workgroups are dispatched round-robin over the 8 XCDs, so block b runs on
// XCD b % 8 and its run is [8G m + (b % 8) G, ... + G).
__device__ __forceinline__ int64_t xcd_schedule(int64_t b, int64_t rows, int G) {
  const int64_t span = 8 * (int64_t)G;
  const int64_t base = (b / span) * span;
  if (G <= 1 || base + span > rows) return b;
  return base + (b % 8) * G + (b / 8) % G;
}

// The worklist row a workgroup takes at position pos (0 = first): the
// worklist's rows longest first (row_perm is in ascending bucket order).
// Dense attention (row r walks r + 1 tiles): with fixed-length sequences, the
// rows in groups of `run` consecutive query blocks of one (sequence, head),
// the groups of the latest query blocks first over all (sequence, head)
// pairs, each group from its last query block down.  A group is one XCD's run
// of positions (see xcd_schedule), so its rows share the K/V prefix in that
// XCD's L2, and the rows start roughly longest first over the whole grid.
// Otherwise (packed varlen, or run not dividing the rows of a sequence) the
// rows in reverse order: each (sequence, head) from its last query block down.
template <bool DENSE>
__device__ __forceinline__ int64_t dense_or_listed_row(const Geom& g, const FwdBufs& a, int64_t pos,
                                                       int run = 0) {
  if constexpr (DENSE) {
    if (!g.varlen && run > 0) {
      const int64_t R = ceil_div(g.n, kBlock) - g.qblk0;   // rows per (sequence, head)
      if (R % run == 0) {
        const int64_t P = g.rows / R;                      // (sequence, head) pairs
        const int64_t grp = pos / run, i = pos % run;
        const int64_t qg = R / run - 1 - grp / P, pair = P - 1 - grp % P;
        return pair * R + qg * run + (run - 1 - i);
      }
    }
    return g.rows - 1 - pos;
  }
  return a.row_perm[g.rows - 1 - pos];
}

// --------------------------------------------------------------------------
// Tile steps shared by the bf16 kernels.  Layouts:
//   S^T accumulator sacc[kb][i] of a lane = key kb*32 + 8*(i/4) + 4*half + i%4
//     of query row l32 (v_mfma_f32_32x32x16_bf16 output layout);
//   P^T operand pb[kb][ks] = the same values rounded to bf16, k-slot (half, e)
//     of step (kb, ks) = key kb*32 + 16 ks + 8 (e/4) + 4 half + e%4;
//   O^T accumulator oacc[db] = d in block db, query row l32.
//
// Scores come out of the MFMA in log2 units and already offset by the row's
// running reference m: Q is pre-scaled by log2(e)/sqrt(d) when it is loaded,
// and the S^T accumulator starts at -m instead of 0 (m = -inf before a row's
// first tile, when it starts at 0).  The softmax then needs one exp2 per
// score and no multiply-add.  m is set by a row's first tile and moves only
// when a later tile's weights outgrow it (see softmax_tile), so most tiles
// take no row maximum and skip the rescale of O.

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// P = exp2(S) in bf16 for the tile's scores (already offset by the row's
// reference m) and this lane's sum of those bf16 weights, the ones P V uses.
__device__ __forceinline__ float exp_tile(const f32x16 (&sacc)[2], bf16x8 (&pb)[2][2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) pb[kb][i / 8][i % 8] = (__bf16)__builtin_amdgcn_exp2f(sacc[kb][i]);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2 pair;
        pair[0] = pb[kb][h][2 * e];
        pair[1] = pb[kb][h][2 * e + 1];
        r[e] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, r[e], false);
      }
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// Row maximum of the tile's scores (both half-waves hold halves of a row).
__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[2]) {
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m0 = fmaxf(m0, sacc[0][i]);
    m1 = fmaxf(m1, sacc[1][i]);
  }
  return max_xor32(fmaxf(m0, m1));
}

// Mask, P = exp2(S - m) in bf16 and the row sum of those weights, with the
// online-softmax reference m of [P2] §1.2 Eq 3-5.  Eq 3-5 give the same u / l
// for any reference that keeps the weights finite, so m need not track the
// running maximum: the row's first tile sets m to its maximum, and later tiles
// exponentiate against the current m without a maximum.  A lane's partial row
// sum bounds every weight it holds, so while it stays <= 2^16 no score rose
// more than 16 (log2 units) above m; otherwise (also on inf) a rare branch
// takes the row maximum, rescales u and l by 2^-shift, moves m and recomputes
// P.  Weights stay <= 2^16, far from fp32 and bf16 overflow.  `kbase` is the
// tile's first key position; `masked` says whether any key of the tile can be
// masked for this row (the diagonal block, or one that runs past the end).
constexpr float kBigSum = 65536.0f;

__device__ __forceinline__ void softmax_tile(f32x16 (&sacc)[2], bf16x8 (&pb)[2][2], f32x16 (&oacc)[4],
                                             float& m, f32x16& negm, float& lsum, bool masked, int kbase, int qpos,
                                             int len, int half) {
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kpos = kbase + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        if (kpos > qpos || kpos >= len) sacc[kb][i] = -INFINITY;
      }
    }
  }
  if (__any(m == -INFINITY)) {   // the row's first tile (every lane of the wave starts its row together)
    asm volatile("");
    const float mt = tile_max(sacc);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] -= mt;
    m = mt;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m;
  }
  float rs = exp_tile(sacc, pb);
  if (__any(!(rs <= kBigSum))) {
    asm volatile("");   // a real branch: the rescale is rare, never speculate it
    const float shift = fmaxf(tile_max(sacc), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-shift);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] -= shift;
    m += shift;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m;
    rs = exp_tile(sacc, pb);
  }
  // this lane's half of the row's keys; the two halves are added once, at the end
  lsum += rs;
}

// LDS reads behind operand i of an MFMA phase (two transpose reads for a V^T
// operand, one read for a K operand) and behind operands 0 .. n-1
template <int NPV, int N>
constexpr int mfma_reads(int i) { return i >= N ? 0 : i < NPV ? 2 : 1; }
template <int NPV, int N>
constexpr int mfma_reads_before(int n) {
  int r = 0;
  for (int i = 0; i < n; ++i) r += mfma_reads<NPV, N>(i);
  return r;
}

// One MFMA phase: O^T += V^T P^T for the V tile at vt (when PV), then
// S^T = K Q^T onto the reference offset -m for the K tile at kt (when S): 16 +
// 16 MFMAs whose LDS operands are read DEPTH MFMAs ahead of use.  Left to
// itself the compiler reads each operand right before its MFMA into the same
// few registers, so nearly every MFMA waits out a full LDS latency; here the
// read for MFMA i + DEPTH is issued right after MFMA i (scheduling groups pin
// that order).  V^T operands come from LDS transpose reads of the row-major V
// tile.  Each accumulator sees its MFMAs in the order (kb, ks).
template <bool PV, bool S, int DEPTH>
__device__ __forceinline__ void mfma_phase(f32x16 (&oacc)[4], const bf16x8 (&pb)[2][2], const unsigned char* vt,
                                           f32x16 (&sacc)[2], const unsigned char* kt, const bf16x8 (&qreg)[8],
                                           const f32x16& negm, int lane) {
  constexpr int NPV = PV ? 16 : 0, NS = S ? 16 : 0, N = NPV + NS;
  const int l32 = lane & 31, half = lane >> 5;
  const int gi = lane >> 4, li = lane & 15, vh = gi >> 1, vdh = gi & 1;
  // operand i < NPV: V^T block (kb, ks, db) = (i >> 3, (i >> 2) & 1, i & 3);
  // operand NPV + j: K block (ks, kb) = (j >> 1, j & 1)
  auto operand = [&](int i) -> bf16x8 {
    if (i < NPV) {
      const int kb = i >> 3, ks = (i >> 2) & 1, db = i & 3;
      const int d = db * 32 + 16 * vdh + 4 * (li & 3);
      const int chunk = d >> 3, h8 = (d >> 2) & 1;
      const int key0 = kb * 32 + 16 * ks + 4 * vh + (li >> 2), key1 = key0 + 8;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (SA_LDS i16x4*)(vt + key0 * 256 + ((chunk ^ vsw(key0)) << 4) + h8 * 8));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (SA_LDS i16x4*)(vt + key1 * 256 + ((chunk ^ vsw(key1)) << 4) + h8 * 8));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int j = i - NPV, ks = j >> 1, kb = j & 1;
    const int key = kb * 32 + l32, c = ks * 2 + half;
    return *reinterpret_cast<const bf16x8*>(kt + key * 256 + ((c ^ ksw(key)) << 4));
  };
  constexpr int kMfma = 0x008, kDsRead = 0x100;   // scheduling-group masks
  bf16x8 buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (i < N) buf[i] = operand(i);
  __builtin_amdgcn_sched_group_barrier(kDsRead, mfma_reads_before<NPV, N>(DEPTH), 0);
  auto step = [&]<int I>() {
    const bf16x8 av = buf[I % DEPTH];
    if constexpr (I + DEPTH < N) buf[I % DEPTH] = operand(I + DEPTH);
    if constexpr (I < NPV) {
      constexpr int kb = I >> 3, ks = (I >> 2) & 1, db = I & 3;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kb][ks], oacc[db], 0, 0, 0);
    } else {
      constexpr int ks = (I - NPV) >> 1, kb = (I - NPV) & 1;
      // the accumulator starts at the reference offset -m (0 before the first tile)
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[ks], ks == 0 ? negm : sacc[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    if constexpr (mfma_reads<NPV, N>(I + DEPTH) > 0)
      __builtin_amdgcn_sched_group_barrier(kDsRead, mfma_reads<NPV, N>(I + DEPTH), 0);
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (step.template operator()<Is>(), ...);
  }(std::make_integer_sequence<int, N>{});
}

// Q rows of this lane as the B operand of S^T = K Q^T, pre-scaled by
// log2(e)/sqrt(128): lane holds Q[qpos][16 ks + 8 half .. +8] * c
__device__ __forceinline__ void load_q(bf16x8 (&qreg)[8], const __bf16* qp, bool qvalid, int half) {
  constexpr float c = kLog2e * 0.08838834764831845f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 x = qvalid ? *reinterpret_cast<const u32x4*>(qp + ks * 16 + half * 8) : u32x4{0, 0, 0, 0};
    qreg[ks] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) qreg[ks][e] = (__bf16)((float)qreg[ks][e] * c);
}

// o = u / l in bf16 and lse = ln(sum_j exp(s_j / sqrt(d))) for this lane's row
__device__ __forceinline__ void store_row(const f32x16 (&oacc)[4], float m, float lsum, __bf16* op, float* lse,
                                          int half) {
  const float inv = 1.f / lsum;
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
  if (lse && half == 0) *lse = (m + __log2f(lsum)) * 0.6931471805599453f;
}

// --------------------------------------------------------------------------
// Lock-step kernel, one LDS stage.  PIPE = 0: loads, then the tile's products;
// PIPE = 2: V(t) and K(t+1) loads overlap S(t) / softmax / P V(t).
template <int HPR, int PIPE, bool DENSE>
__global__ void __launch_bounds__(128 * HPR) prefill_bf16_kernel(Geom g, FwdBufs a, int xcd_run) {
  static_assert(PIPE == 0 || PIPE == 2, "pipeline form");
  constexpr int D = 128;
  constexpr int NW = 2 * HPR;               // wavefronts: 2 per query head
  constexpr int TILE = 64 * D * 2;          // bytes of one K (or V) tile
  constexpr int HALF_LOADS = (TILE / 1024) / NW;  // 1 KB wave loads of a K (or V) tile per wave
  constexpr int kDepth = 6;                       // MFMAs of lead for the LDS operand reads
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * TILE];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // Workgroup b takes one worklist position in each pass over the grid (G =
  // gridDim.x; G = rows unless the launch is persistent, see prefill_grid):
  // b in even passes and its mirror m(b) = (G/8 - 1 - b/8) * 8 + b % 8 in odd
  // ones.  The positions run longest first, so a workgroup that took one of
  // the longest rows of a pass takes one of the shortest of the next, and the
  // workgroups' shares even out (a dense causal walk's rows r and N - 1 - r
  // pair up to N + 1 tiles).  m(b) keeps b's XCD (b % 8; a persistent G is a
  // multiple of 8, and a grid of G = rows makes one pass only).
  for (int64_t base = 0; base < g.rows; base += gridDim.x) {
    const int64_t vb = base + (((base / gridDim.x) & 1)
                                   ? (int64_t)(gridDim.x / 8 - 1 - blockIdx.x / 8) * 8 + blockIdx.x % 8
                                   : (int64_t)blockIdx.x);
    if (base != 0) block_barrier();   // the previous row's LDS reads are done
    if (vb >= g.rows) continue;
    const int64_t pos = xcd_schedule(vb, g.rows, xcd_run);
    const int64_t row = dense_or_listed_row<DENSE>(g, a, pos, xcd_run);
    const RowInfo ri = decode_row(g, row);
    const int kvh = g.share ? ri.h : ri.h / g.group;
    const int head = (g.share ? ri.h * g.group : ri.h) + wave / 2;
    const int half = lane / 32, l32 = lane % 32;
    const int qpos = ri.r * kBlock + (wave % 2) * 32 + l32;
    const bool qvalid = qpos < ri.len;
    const unsigned char* kbytes = (const unsigned char*)a.k;
    const unsigned char* vbytes = (const unsigned char*)a.v;

    const int t_begin = DENSE ? 0 : a.row_ptr[row];
    const int ntiles = DENSE ? ri.r + 1 : a.row_ptr[row + 1] - t_begin;
    // the row's tile ids, one per lane (a listed row holds at most 128 tiles);
    // read back with readlane so the loop issues no memory load (and no wait)
    // for them.  A dense row visits tiles 0 .. r in order.
    const int jl0 = !DENSE && lane < ntiles ? a.col_idx[t_begin + lane] : 0;
    const int jl1 = !DENSE && lane + 64 < ntiles ? a.col_idx[t_begin + 64 + lane] : 0;
    // Consume the loads here, on every path: the compiler's wait-count pass is
    // path-insensitive, and a register that may still be pending at the loop
    // header makes it wait for all vector loads (the tile prefetch included)
    // inside the loop on every iteration.
    asm volatile("" ::"v"(jl0), "v"(jl1));
    auto tile_id = [&](int it) {
      if constexpr (DENSE) return it;
      return it < 64 ? __builtin_amdgcn_readlane(jl0, it) : __builtin_amdgcn_readlane(jl1, it - 64);
    };

    // 16-byte global->LDS loads of tile `it`: K into kt, V into vt.  Wave w
    // loads the 1 KB slices w, w + NW, ... of a tile; in slice i lane (sub, cl)
    // carries 16-byte chunk cl of key 4 i + sub to its swizzled slot.  The
    // per-lane byte offsets of a full tile are fixed for the row.
    constexpr int NLD = 16 / NW;
    const int sub = lane >> 4, cl = lane & 15;
    uint32_t koff[NLD], voff[NLD];
  #pragma unroll
    for (int ii = 0; ii < NLD; ++ii) {
      const int key = 4 * (wave + NW * ii) + sub;
      koff[ii] = key * 256 + ((cl ^ ksw(key)) << 4);
      voff[ii] = key * 256 + ((cl ^ vsw(key)) << 4);
    }
    const int64_t kv_row = kv_offset(g, ri.s, kvh, ri.tok0, 0) * 2;
    const unsigned char* const krow = uniform_ptr(kbytes + kv_row);
    const unsigned char* const vrow = uniform_ptr(vbytes + kv_row);
    const int len_u = __builtin_amdgcn_readfirstlane(ri.len);
    auto issue = [&](int it, const unsigned char* src, const uint32_t (&off)[NLD], unsigned char* dst, bool is_v) {
      const int j = tile_id(it);
      const unsigned char* base = src + (int64_t)j * TILE;
      const int cnt = len_u - j * kBlock;
      if (cnt >= kBlock) {
  #pragma unroll
        for (int ii = 0; ii < NLD; ++ii) load_lds16_sv(base, off[ii], dst + (wave + NW * ii) * 1024);
      } else {
        asm volatile("");   // the sequence's last, partial block: a real branch
  #pragma unroll
        for (int ii = 0; ii < NLD; ++ii) {
          const int key = 4 * (wave + NW * ii) + sub;
          const int kc = min(key, cnt - 1);   // rows past the end: any valid row (masked later)
          const uint32_t o = kc * 256 + ((cl ^ (is_v ? vsw(key) : ksw(key))) << 4);
          load_lds16_sv(base, o, dst + (wave + NW * ii) * 1024);
        }
      }
    };
    auto issue_k = [&](int it, unsigned char* kt) { issue(it, krow, koff, kt, false); };
    auto issue_v = [&](int it, unsigned char* vt) { issue(it, vrow, voff, vt, true); };
    unsigned char* const kt = lds;
    unsigned char* const vt = lds + TILE;
    if (ntiles > 0) {
      issue_k(0, kt);
      if (PIPE == 0) issue_v(0, vt);
    }

    bf16x8 qreg[8];
    load_q(qreg, (const __bf16*)a.q + q_offset(g, ri.s, head, ri.tok0, qvalid ? qpos : 0), qvalid, half);
  #pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks]));   // see the tile ids above

    float m = -INFINITY, lsum = 0.f;
    f32x16 negm = {};   // -m in every slot: the S^T accumulator's start (0 before the first tile)
    f32x16 oacc[4];
  #pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    f32x16 sacc[2];
    bf16x8 pb[2][2];

    for (int it = 0; it < ntiles; ++it) {
      if (PIPE == 2) {
        // K(it) landed (only it is outstanding); every wave is past P V(it-1)
        wait_vmcnt<0>();
        block_barrier();
        issue_v(it, vt);
      } else {
        if (it > 0) {   // the previous iteration ended with a barrier
          issue_k(it, kt);
          issue_v(it, vt);
        }
        wait_vmcnt<0>();
        block_barrier();
      }
      const int j = tile_id(it);
      mfma_phase<false, true, kDepth>(oacc, pb, vt, sacc, kt, qreg, negm, lane);
      if (PIPE == 2 && it + 1 < ntiles) {
        block_barrier();          // every wave has read K(it): refill it with K(it+1)
        issue_k(it + 1, kt);
      }
      softmax_tile(sacc, pb, oacc, m, negm, lsum, j == ri.r || j * kBlock + kBlock > ri.len, j * kBlock, qpos, ri.len,
                   half);
      if (PIPE == 2) {
        // V(it) landed; K(it+1) may still be in flight
        if (it + 1 < ntiles) wait_vmcnt<HALF_LOADS>();
        else wait_vmcnt<0>();
        block_barrier();
      }
      mfma_phase<true, false, kDepth>(oacc, pb, vt, sacc, kt, qreg, negm, lane);
      if (PIPE != 2) block_barrier();   // every wave is done with this stage before it is refilled
    }

    lsum = sum_xor32(lsum);
    if (qvalid)
      store_row(oacc, m, lsum, (__bf16*)a.o + q_offset(g, ri.s, head, ri.tok0, qpos),
                a.lse ? a.lse + lse_offset(g, ri.s, head, ri.tok0, qpos) : nullptr, half);
  }
}

// --------------------------------------------------------------------------
// Ping-pong bf16 prefill kernel for rows of four query heads (8 wavefronts).
//
// At ~200 VGPRs a SIMD holds two wavefronts, and in an 8-wavefront workgroup
// they are waves w and w + 4 of the same row.  Run in lock step, both would
// issue MFMAs at the same time and then both run the softmax on the vector ALU,
// so the two units never overlap.  Here waves 0-3 (group 0) and 4-7 (group 1)
// run half a tile apart: the tile loop is cut into slots separated by
// barriers, and in every slot one group runs an MFMA phase while the other
// runs a softmax phase.
//   phases of one wavefront: S(0) X(0) M(0) X(1) M(1) ... X(n-1) M(n-1), where
//     S(t) = K(t) Q^T (MFMA), X(t) = mask / max / exp / sum of tile t (VALU),
//     M(t) = P(t) V(t) followed by S(t+1) (MFMA);
//   group g runs phase p in slot p + g, slots 0 .. 2n+1.
// K and V have separate NB-deep LDS rings.  Load round r = {K(r), V(r-1)}:
// rounds 0 .. NB-1 are issued before the loop and round u+NB-1 right after the
// barrier that opens slot 2u (u >= 1), when K(u-1) and V(u-2) have had their
// last reads (slot 2u-1).  Round u is waited for before slot 2u, the first
// slot that reads K(u) or V(u-1).
template <int N>
__device__ __forceinline__ void wait_vm_halves(int halves) {
  // N = loads per half tile per wavefront; at most 7 half tiles in flight
  switch (halves) {
    case 7: wait_vmcnt<7 * N>(); break;
    case 6: wait_vmcnt<6 * N>(); break;
    case 5: wait_vmcnt<5 * N>(); break;
    case 4: wait_vmcnt<4 * N>(); break;
    case 3: wait_vmcnt<3 * N>(); break;
    case 2: wait_vmcnt<2 * N>(); break;
    case 1: wait_vmcnt<N>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

template <int NB, bool DENSE>
__global__ void __launch_bounds__(512) prefill_bf16_pp_kernel(Geom g, FwdBufs a, int xcd_run) {
  constexpr int NW = 8, D = 128;
  constexpr int TILE = 64 * D * 2;
  constexpr int HALF_LOADS = (TILE / 1024) / NW;   // 1 KB wave loads per K (or V) tile per wave
  static_assert(NB >= 3 && NB <= 4, "ring depth");
  constexpr int kDepth = 6;   // MFMAs of lead for the LDS operand reads
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * NB * TILE];
  unsigned char* const kring = lds;
  unsigned char* const vring = lds + NB * TILE;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave >> 2;
  const int64_t pos = xcd_schedule(blockIdx.x, g.rows, xcd_run);
  const int64_t row = dense_or_listed_row<DENSE>(g, a, pos, xcd_run);
  const RowInfo ri = decode_row(g, row);
  const int kvh = g.share ? ri.h : ri.h / g.group;
  // heads 4 blockIdx.y .. + 3 of the row (rows of more than 4 heads take
  // several workgroups); slots past the row's last head compute a copy of that
  // head and store nothing
  const int hslot = 4 * (int)blockIdx.y + wave / 2;
  const bool hvalid = hslot < g.hpr;
  const int head = (g.share ? ri.h * g.group : ri.h) + min(hslot, g.hpr - 1);
  const int half = lane / 32, l32 = lane % 32;
  const int qpos = ri.r * kBlock + (wave % 2) * 32 + l32;
  const bool qvalid = qpos < ri.len;
  const unsigned char* kbytes = (const unsigned char*)a.k;
  const unsigned char* vbytes = (const unsigned char*)a.v;

  const int t_begin = DENSE ? 0 : a.row_ptr[row];
  const int ntiles = DENSE ? ri.r + 1 : a.row_ptr[row + 1] - t_begin;
  const int jl0 = !DENSE && lane < ntiles ? a.col_idx[t_begin + lane] : 0;
  const int jl1 = !DENSE && lane + 64 < ntiles ? a.col_idx[t_begin + 64 + lane] : 0;
  asm volatile("" ::"v"(jl0), "v"(jl1));   // consumed on every path (see prefill_bf16_kernel)
  auto tile_id = [&](int it) {
    if constexpr (DENSE) return it;
    return it < 64 ? __builtin_amdgcn_readlane(jl0, it) : __builtin_amdgcn_readlane(jl1, it - 64);
  };

  // per-lane byte offsets of this wave's 1 KB slices of a full tile (see
  // prefill_bf16_kernel)
  constexpr int NLD = 16 / NW;
  const int sub = lane >> 4, cl = lane & 15;
  uint32_t koff[NLD], voff[NLD];
#pragma unroll
  for (int ii = 0; ii < NLD; ++ii) {
    const int key = 4 * (wave + NW * ii) + sub;
    koff[ii] = key * 256 + ((cl ^ ksw(key)) << 4);
    voff[ii] = key * 256 + ((cl ^ vsw(key)) << 4);
  }
  const int64_t kv_row = kv_offset(g, ri.s, kvh, ri.tok0, 0) * 2;
  const unsigned char* const krow = uniform_ptr(kbytes + kv_row);
  const unsigned char* const vrow = uniform_ptr(vbytes + kv_row);
  const int len_u = __builtin_amdgcn_readfirstlane(ri.len);
  auto issue_half = [&](int it, const unsigned char* src, unsigned char* dst, bool is_v) {
    const int j = tile_id(it);
    const unsigned char* base = src + (int64_t)j * TILE;
    const int cnt = len_u - j * kBlock;
    if (cnt >= kBlock) {
#pragma unroll
      for (int ii = 0; ii < NLD; ++ii)
        load_lds16_sv(base, is_v ? voff[ii] : koff[ii], dst + (wave + NW * ii) * 1024);
    } else {
      asm volatile("");   // the sequence's last, partial block: a real branch
#pragma unroll
      for (int ii = 0; ii < NLD; ++ii) {
        const int key = 4 * (wave + NW * ii) + sub;
        const int kc = min(key, cnt - 1);   // rows past the end: any valid row (masked later)
        const uint32_t o = kc * 256 + ((cl ^ (is_v ? vsw(key) : ksw(key))) << 4);
        load_lds16_sv(base, o, dst + (wave + NW * ii) * 1024);
      }
    }
  };
  auto issue_round = [&](int r) {
    if (r < ntiles) issue_half(r, krow, kring + (r % NB) * TILE, false);
    if (r >= 1) issue_half(r - 1, vrow, vring + ((r - 1) % NB) * TILE, true);
  };
  // half rounds issued after round u, when rounds 0 .. hi are out
  auto younger_halves = [&](int u, int hi) {
    if (hi <= u) return 0;
    return 2 * (hi - u) - (hi == ntiles ? 1 : 0);
  };
  if (ntiles > 0) issue_round(0);

  bf16x8 qreg[8];
  load_q(qreg, (const __bf16*)a.q + q_offset(g, ri.s, head, ri.tok0, qvalid ? qpos : 0), qvalid, half);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks]));
  if (ntiles > 0) {
#pragma unroll
    for (int r = 1; r < NB; ++r)
      if (r <= ntiles) issue_round(r);
  }

  float m = -INFINITY, lsum = 0.f;
  f32x16 negm = {};   // -m in every slot: the S^T accumulator's start (0 before the first tile)
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  f32x16 sacc[2];
  bf16x8 pb[2][2];

  // Both groups run  M(u) | barrier | X(u) | barrier  for u = 0 .. n, with
  // M(u) = P(u-1) then S(u); group 1 passes one barrier before its first
  // M and group 0 one after its last X, which sets the half-tile offset.  In
  // the global barrier count, group 0's M(u) follows barrier 2u and group 1's
  // follows barrier 2u+1; round u is waited for before barrier 2u and round
  // u+NB-1 issued right after it.
  auto wait_round = [&](int u) {
    const int hi = min(max(NB - 1, u + NB - 2), ntiles);
    wait_vm_halves<HALF_LOADS>(younger_halves(u, hi));
  };
  auto issue_after = [&](int u) {   // right after barrier 2u
    if (u >= 1 && u + NB - 1 <= ntiles) issue_round(u + NB - 1);
  };
  if (ntiles > 0) {
    if (grp == 1) {
      wait_round(0);
      block_barrier();                               // barrier 0
    }
    for (int u = 0; u <= ntiles; ++u) {
      if (grp == 0) {
        wait_round(u);
        block_barrier();                             // barrier 2u
        issue_after(u);
      } else {
        block_barrier();                             // barrier 2u+1
      }
      {
        const unsigned char* vt = vring + ((u + NB - 1) % NB) * TILE;   // V(u-1)
        const unsigned char* kt = kring + (u % NB) * TILE;              // K(u)
        if (u >= 1) mfma_phase<true, false, kDepth>(oacc, pb, vt, sacc, kt, qreg, negm, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (u < ntiles) mfma_phase<false, true, kDepth>(oacc, pb, vt, sacc, kt, qreg, negm, lane);
      }
      if (grp == 0) {
        block_barrier();                             // barrier 2u+1
      } else if (u < ntiles) {
        wait_round(u + 1);
        block_barrier();                             // barrier 2u+2
        issue_after(u + 1);
      } else {
        block_barrier();                             // barrier 2n+2
      }
      if (u < ntiles) {
        const int j = tile_id(u);
        softmax_tile(sacc, pb, oacc, m, negm, lsum, j == ri.r || j * kBlock + kBlock > ri.len, j * kBlock, qpos,
                     ri.len, half);
      }
    }
    if (grp == 0) block_barrier();                   // barrier 2n+2
  }

  lsum = sum_xor32(lsum);
  if (qvalid && hvalid)
    store_row(oacc, m, lsum, (__bf16*)a.o + q_offset(g, ri.s, head, ri.tok0, qpos),
              a.lse ? a.lse + lse_offset(g, ri.s, head, ri.tok0, qpos) : nullptr, half);
}

// --------------------------------------------------------------------------
// fp32 SIMT kernel: one wavefront per (row, head), one lane per query row.
// Used for fp32 problems (prefill and decode); exact fp32 exp.
template <int D, bool DENSE>
__global__ void __launch_bounds__(64) attn_f32_kernel(Geom g, FwdBufs a) {
  __shared__ float ks[64][D + 1];
  __shared__ float vs[64][D];
  const int lane = threadIdx.x;
  const int64_t row = dense_or_listed_row<DENSE>(g, a, (int64_t)blockIdx.x);
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
  const int t0 = DENSE ? 0 : a.row_ptr[row], t1 = DENSE ? ri.r + 1 : a.row_ptr[row + 1];
  for (int t = t0; t < t1; ++t) {
    const int j = DENSE ? t : a.col_idx[t];
    const int cnt = min(kBlock, ri.len - j * kBlock);
    __syncthreads();
    const float* kb = k + kv_block_offset(g, ri.s, kvh, ri.tok0, j);
    const float* vb = v + kv_block_offset(g, ri.s, kvh, ri.tok0, j);
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

template <bool DENSE>
int launch_f32(const Geom& g, const FwdBufs& b, hipStream_t st) {
  dim3 grid((unsigned)g.rows, g.hpr);
  if (g.d == 64)
    attn_f32_kernel<64, DENSE><<<grid, 64, 0, st>>>(g, b);
  else
    attn_f32_kernel<128, DENSE><<<grid, 64, 0, st>>>(g, b);
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// Grid for `rows` worklist rows.  With few generations of workgroups (rows
// <= 4 x the co-resident slots) the run ends with a tail of staggered late
// starts, so the grid is the slots (at least 8, a multiple of 8 so position v
// stays on XCD v % 8) and each workgroup loops over its rows.  With many
// generations the dispatcher's first-come assignment balances the CUs better
// than a fixed share does, and the grid is one workgroup per row.
template <typename K>
unsigned prefill_grid(K kernel, int threads, int64_t rows) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess) {
    return (unsigned)rows;
  }
  int64_t slots = (int64_t)std::max(per, 1) * std::max(cus, 1);
  slots = std::max<int64_t>(8, slots / 8 * 8);
  return (unsigned)(rows <= 4 * slots ? std::min(rows, slots) : rows);
}

template <bool DENSE>
int launch_prefill_t(const Geom& g, int dtype, const FwdBufs& b, hipStream_t st) {
  if (g.rows <= 0) return SA_OK;
  if (dtype == SA_F32) return launch_f32<DENSE>(g, b, st);
  if (g.d != 128) return SA_ERR_UNSUPPORTED;
  // One-head rows: one LDS stage (32 KB) per workgroup, so four workgroups fit
  // on a CU and each SIMD runs two wavefronts of different rows; V(t) and
  // K(t+1) loads overlap S(t) and the softmax.  Measured on MI355X this beats
  // a 2-4 stage ring (64-128 KB, fewer workgroups per CU).  Runs of 128 rows
  // per XCD keep one head's K/V (4 MB at n = 8192) in that XCD's L2.
  // Four-head rows: the ping-pong kernel with 4-deep K and V rings (128 KB, one
  // workgroup per CU); its two wavefronts per SIMD alternate MFMA and softmax
  // phases (eight-head rows: two of its workgroups per row).  Two-head rows:
  // the lock-step kernel, one stage.
  // The lock-step kernel's grid comes from prefill_grid (persistent when the
  // rows fill few generations).
  const int run = g.hpr == 1 ? 128 : 32;   // rows per XCD run
  switch (g.hpr) {
    case 1: {
      auto k = prefill_bf16_kernel<1, 2, DENSE>;
      k<<<prefill_grid(k, 128, g.rows), 128, 0, st>>>(g, b, run);
      break;
    }
    case 2: {
      auto k = prefill_bf16_kernel<2, 0, DENSE>;
      k<<<prefill_grid(k, 256, g.rows), 256, 0, st>>>(g, b, run);
      break;
    }
    default:
      // three or more heads: the four-head kernel, one workgroup per row and
      // head quad (each loads the row's tiles; a last partial quad computes
      // copies of the row's last head and stores nothing for them).  One
      // workgroup per row: the outer row loop of the persistent form costs
      // this kernel ~14 % in code generation, and with one workgroup per CU
      // its rows always fill many generations
      prefill_bf16_pp_kernel<4, DENSE><<<dim3((unsigned)g.rows, (unsigned)((g.hpr + 3) / 4)), 512, 0, st>>>(
          g, b, run);
      break;
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int launch_prefill(const Geom& g, int dtype, const FwdBufs& b, hipStream_t st, bool dense) {
  return dense ? launch_prefill_t<true>(g, dtype, b, st) : launch_prefill_t<false>(g, dtype, b, st);
}

}  // namespace sa
