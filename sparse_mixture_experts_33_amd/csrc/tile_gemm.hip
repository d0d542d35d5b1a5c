// Tiled grouped GEMM for large expert groups (prefill): the same two projections as the
// streaming kernel (SwiGLU expert, xyznot.com summary "Método"; only routed rows exist, ja.news.hada.io
// summary on zero-gate experts), shaped for the matrix cores instead of for the weight stream.
//
//   C[w][t] = sum_k W[w][k] * X[t][k]     (w: weight row = output column, t: token row of the group)
//
// Workgroup tile: BW weight rows x BT tokens (SwiGLU: BW/2 rows of w1 and the same BW/2 rows of
// w3, so that silu(a)*b is formed in registers), 128 KB of LDS stages. Eight wavefronts
// (two per SIMD, so one's LDS and memory waits overlap the other's MFMAs) in a 2 x 4
// arrangement, each BW/2 weight rows x BT/4 tokens, 16x16x32 bf16 MFMAs accumulating in fp32.
//
// LDS holds both operands in matrix-core fragment order: a fragment is 16 rows x 32 k, 1 KB,
// lane l holding row l%16 and k = 8*(l/16)..+7. Every global->LDS write and every LDS->register
// read of a wavefront is then one contiguous 1 KB, free of bank conflicts for any bank count.
// Weights in the packed layout arrive already in that order (1 KB contiguous global loads).
//
// Tiles are numbered expert-major, then in bands of 4 token tiles, then weight tile, then token
// tile within the band, so that the 32 tiles an XCD runs at once share 4 token and 8 weight row
// blocks; the linear index is remapped so that adjacent tiles go to workgroups on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs), which keeps those blocks in that XCD's L2.
//
// Token blocks (16 rows) are dealt to the four token wavefronts round-robin (wavefront t owns
// blocks t, t+4, t+8, t+12), so the partly filled last tile of a group spreads its rows over the
// SIMDs; a wavefront skips the MFMAs (and fragment reads) of blocks that lie wholly past the
// group's end. Token rows past the end still load a valid row and are never stored.
//
// Forward products (weights [E][N][K], packed or row-major): k-steps of 32 through four LDS stages
// of 32 KB, filled by direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land at
// the destination + 16 l, which is fragment order), so three steps are in flight while one is
// multiplied and no registers stage the data. Per step s: wait until this wavefront's loads of
// step s have landed (vmcnt, counting the loads issued after them), barrier (then every
// wavefront's have), issue step s+3 into the stage that step s-1 used, read the fragments of step
// s, multiply. The fragment reads are inline assembly that waits for its own results: the
// compiler cannot tell them apart from the asynchronous LDS writes and would otherwise wait for
// every load in flight before each read; for the same reason the barrier is a bare s_barrier
// (a workgroup fence makes the compiler drain all loads first).
//
// Backward products (WT, WGRAD): k-steps of 64 through two stages staged in registers. Per step s:
// write step s+1 (loaded during step s-1) to the free stage, load step s+2, multiply step s,
// barrier. Writing at the start of the step lets the LDS writes complete under the MFMAs instead
// of holding every wavefront at the barrier.
#include "common.hpp"
#include "launch.hpp"

#include <cmath>
#include <type_traits>

namespace moe {
namespace {

constexpr int kXcds = 8;

__device__ inline float silu_t(float z) { return z / (1.0f + expf(-z)); }

// WGRAD: weight-gradient mode of the backward pass. Per expert e the product runs over the rows of
// e's group instead of over a fixed K: out[e][m][n] = sum over the group's rows r of
// act[r][m] * wa[r][n], with act [rows][.] (row stride K) and wa [rows][.] (row stride ldw) the
// group-sorted rows as they lie (WGRAD requires WT: both operands k-major, read through transposing
// LDS reads). A k-step takes 64 rows of the group; rows past its end are zeroed in registers. The
// group sizes come from `offsets` on the device. Tiles are (expert, n tile, m tile), one 256 x 256
// output tile each.
//
// WT: the weight operand is stored transposed, [E][K][N] with the N columns contiguous (the layout
// in which the backward pass holds w2 and w1, w3 for its products): wa holds k < KA = K/2 and wb
// the rest when wb is given (KA = K otherwise). A k-step of the weight block is staged in LDS as
// it lies in memory (64 rows of 256 columns, rows padded by 16 elements), and each matrix-core
// operand is assembled by two transposing LDS reads (ds_read_b64_tr_b16): in each group of 16
// lanes, lanes 4a..4a+3 address the 16 columns of row a, and lane i receives column i of the 4
// rows, which is 4 consecutive k of weight row i.
template <int BW, int BT, bool PACKED, bool SWIGLU, bool WGRAD, bool WT, typename OutT>
__global__ __launch_bounds__(512, 1) void tile_gemm_kernel(const bf16_t* __restrict__ act,
                                                           const int32_t* __restrict__ row_src,
                                                           const int32_t* __restrict__ offsets,
                                                           const bf16_t* __restrict__ wa,
                                                           const bf16_t* __restrict__ wb, OutT* __restrict__ out,
                                                           int K, int N, int E, int ksplit, float* __restrict__ part,
                                                           int64_t part_stride, int M, int ldw,
                                                           bf16_t* __restrict__ hout) {
  static_assert(!WGRAD || (!SWIGLU && !PACKED && WT), "the weight-gradient mode reads both operands k-major");
  static_assert(!WT || (!SWIGLU && !PACKED), "transposed weights: plain product only");
  constexpr int NW = SWIGLU ? BW / 2 : BW;  // output columns per tile
  constexpr int WF = BW / 16 * 2;           // weight fragments per k-step (16-row blocks x 2)
  constexpr int TF = BT / 16 * 2;           // token fragments per k-step
  constexpr int NWV = 8;                    // wavefronts: 2 over weight rows x 4 over tokens
  constexpr int WL = WF / NWV;              // weight fragment loads per wavefront per step
  constexpr int TL = TF / NWV;              // token fragment loads per wavefront per step
  constexpr int AB = BW / 32;               // weight blocks per wavefront
  constexpr int BB = BT / 64;               // token blocks per wavefront
  constexpr int WROW = BW + 16;             // WT: LDS row of the weight block (elements, padded)
  constexpr int WPART = WT ? 64 * WROW * 2 : WF * 1024;  // bytes of the weight block per stage
  constexpr int TROW = BT + 16;             // WGRAD: LDS row of the token block (elements, padded)
  constexpr int TPART = WGRAD ? 64 * TROW * 2 : TF * 1024;
  constexpr int STAGE = WPART + TPART;      // bytes per LDS stage

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_tile0[kMaxExperts + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave >> 2, wt = wave & 3;

  if (threadIdx.x <= E) s_off[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  const int NT = N / NW;
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      s_tile0[e] = acc;  // first tile of the group
      acc += WGRAD ? 0 : (s_off[e + 1] - s_off[e] + BT - 1) / BT * NT;
    }
    s_tile0[E] = acc;
  }
  __syncthreads();
  // Split-K (down projection only): every tile is computed as `ksplit` independent k-ranges;
  // range p > 0 writes its partial sums to part + (p-1)*part_stride, to be added in a fixed
  // order by the consumer.
  const int MT = WGRAD ? M / BT : 0;
  const int total = WGRAD ? E * MT * NT : s_tile0[E];
  const int Q = (total * ksplit + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  if (j >= Q) return;
  const int tsplit = xcd * Q + j;
  if (tsplit >= total * ksplit) return;
  const int p = tsplit / total, tile = tsplit - p * total;
  int e = 0, nt, mt, r0, nrows;
  int64_t kcol0 = 0;  // first column of the tile's k range in both operands
  int nsteps_all;
  if constexpr (WGRAD) {
    e = tile / (MT * NT);
    const int local = tile - e * MT * NT;
    // 32 consecutive tiles (the ones an XCD runs at once) form a 4 x 8 block of m x n tiles, so
    // they share 4 + 8 operand row blocks instead of 32 + 1
    constexpr int GM = 4, GN = 8;
    if (MT % GM == 0 && NT % GN == 0) {
      const int g = local / (GM * GN), w = local - g * (GM * GN);
      const int gm = g % (MT / GM), gn = g / (MT / GM);
      mt = gm * GM + w % GM;
      nt = gn * GN + w / GM;
    } else {
      nt = local / MT;
      mt = local - nt * MT;
    }
    r0 = mt * BT;
    nrows = min(BT, M - r0);
    kcol0 = s_off[e];  // first row of the group: the k range starts there
    nsteps_all = (s_off[e + 1] - s_off[e] + 63) / 64;
    out += (int64_t)e * M * N;
  } else {
    while (tile >= s_tile0[e + 1]) ++e;
    const int mtiles = (s_off[e + 1] - s_off[e] + BT - 1) / BT;
    const int local = tile - s_tile0[e];
    // token tiles in bands of 4: within a band the token tile varies fastest, then the weight
    // tile, so the 32 tiles an XCD runs at once cover 4 token x 8 weight tiles even for a group
    // of many token tiles (a group of at most 4 is a single band: weight-tile major)
    const int band = local / (4 * NT), mb = band * 4, bs = min(4, mtiles - mb);
    const int w = local - band * 4 * NT;
    mt = mb + w % bs;
    nt = w / bs;
    r0 = s_off[e] + mt * BT;
    nrows = min(BT, s_off[e + 1] - r0);
    nsteps_all = K / 64;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  kcol0 = __builtin_amdgcn_readfirstlane((int)kcol0);
  nsteps_all = __builtin_amdgcn_readfirstlane(nsteps_all);
  // token blocks of this wavefront that hold at least one row of the group
  const int nbv = min(BB, max(0, ((nrows + 15) / 16 - wt + 3) / 4));
  const int n0 = nt * NW;
  if constexpr (!SWIGLU) {
    if (p > 0) out = reinterpret_cast<OutT*>(part + (int64_t)(p - 1) * part_stride);
  }

  // This wavefront loads fragments g = wave + 8*i of each stage: 16-row block (wave>>1) + 4*i at
  // the fixed k-half (wave & 1). Addresses = scalar (wave-uniform) parts + one lane offset.
  const int qh = wave & 1, b0 = wave >> 1;
  // first element of the tile's weights (row-major and packed layouts)
  const int64_t wrow0 = ((int64_t)e * N + n0) * K;
  const int w_lane = PACKED ? qh * 512 + lane * 8 : (lane & 15) * K + qh * 32 + (lane >> 4) * 8;
  int32_t tsrc[TL];
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int rr = (b0 + 4 * i) * 16 + (lane & 15);
    const int r = r0 + (rr < nrows ? rr : 0);
    tsrc[i] = row_src ? row_src[r] : r;
  }
  const int t_lane = qh * 32 + (lane >> 4) * 8;
  // k advance per step: packed weights move 2 fragments (1024 elements) per 16-row block
  constexpr int64_t kWStep = PACKED ? 1024 : 64;

  // WT: thread loads 8 consecutive columns nc.. of k rows kr0 + 16*i of the step (coalesced rows)
  const int kr0 = threadIdx.x / (BW / 8), nc = (threadIdx.x % (BW / 8)) * 8;
  const int KA = (WT && wb) ? K / 2 : K;
  u32x4_t wreg[WL], treg[TL];
  const int kend = WGRAD ? s_off[e + 1] : 0, klast = WGRAD ? s_off[E] - 1 : 0;  // group end, last row
  auto gload = [&](int s) {
    if constexpr (WGRAD) {
      // both operands: rows kcol0 + 64 s + kr of the group, zero past its end (loads clamped in bounds)
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int kr = (int)kcol0 + s * 64 + kr0 + (512 / (BW / 8)) * i;
        const int64_t kc = min(kr, klast);
        const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t wv = load16_nt(wa + kc * ldw + n0 + nc);
        const u32x4_t tv = load16(act + kc * K + r0 + nc);
        wreg[i] = kr < kend ? wv : z;
        treg[i] = kr < kend ? tv : z;
      }
      return;
    }
    if constexpr (WT) {
      const bool second = wb && s * 64 >= KA;  // uniform over the step (KA is a multiple of 64)
      const bf16_t* w = second ? wb : wa;
      const int64_t k0 = (int64_t)s * 64 - (second ? KA : 0);
#pragma unroll
      for (int i = 0; i < WL; ++i)
        wreg[i] = load16_nt(w + ((int64_t)e * KA + k0 + kr0 + (512 / (BW / 8)) * i) * ldw + n0 + nc);
    } else
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      int blk = b0 + 4 * i;
      const bf16_t* w = wa;
      if constexpr (SWIGLU) {
        if (i >= WL / 2) {  // blocks BW/32.. hold w3 (b0 + 4i >= BW/32 exactly when i >= WL/2)
          w = wb;
          blk -= BW / 32;
        }
      }
      wreg[i] = load16_nt(w + wrow0 + (int64_t)blk * 16 * K + (int64_t)s * kWStep + w_lane);
    }
#pragma unroll
    for (int i = 0; i < TL; ++i) treg[i] = load16(act + (int64_t)tsrc[i] * K + kcol0 + (int64_t)s * 64 + t_lane);
  };
  auto lstore = [&](int stage) {
    uint8_t* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      if constexpr (WT)
        store16(base + ((kr0 + (512 / (BW / 8)) * i) * WROW + nc) * 2, wreg[i]);
      else
        store16(base + (wave + 8 * i) * 1024 + lane * 16, wreg[i]);
    }
#pragma unroll
    for (int i = 0; i < TL; ++i) {
      if constexpr (WGRAD)
        store16(base + WPART + ((kr0 + (512 / (BT / 8)) * i) * TROW + nc) * 2, treg[i]);
      else
        store16(base + WPART + (wave + 8 * i) * 1024 + lane * 16, treg[i]);
    }
  };
  // Matrix-core operand from a k-major block in LDS (64 rows of `row` elements): 16 columns
  // blk*16.. at k-half q, lane l gets column l%16 at k = 8(l/16)..+7 (two transposing reads).
  auto trfrag = [&](const uint8_t* blkbase, int row, int blk, int q) -> u32x4_t {
    typedef __attribute__((ext_vector_type(4))) short v4s;
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const int g = lane >> 4, a = (lane >> 2) & 3, c = lane & 3;
    const uint8_t* p = blkbase + ((q * 32 + 8 * g + a) * row + blk * 16 + 4 * c) * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * row * 2));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  };
  // Weight operand of 16-row block blk at k-half q (16 rows x 32 k, lane l: row l%16, k 8(l/16)..+7).
  auto wfrag = [&](const uint8_t* base, int blk, int q) -> u32x4_t {
    if constexpr (WT)
      return trfrag(base, WROW, blk, q);
    else
      return load16(base + (blk * 2 + q) * 1024 + lane * 16);
  };

  f32x4_t acc[AB][BB];
#pragma unroll
  for (int a = 0; a < AB; ++a)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // weight block of the wavefront's a-th A fragment
  auto wblock = [&](int a) -> int {
    if constexpr (SWIGLU) return a < AB / 2 ? wr * (AB / 2) + a : BW / 32 + wr * (AB / 2) + (a - AB / 2);
    else return wr * AB + a;
  };

  // Token fragment of the wavefront's b-th token block (block wt + 4b) at k-half q.
  auto tfrag = [&](const uint8_t* base, int b, int q) -> u32x4_t {
    if constexpr (WGRAD)
      return trfrag(base + WPART, TROW, wt + 4 * b, q);
    else
      return load16(base + WPART + ((wt + 4 * b) * 2 + q) * 1024 + lane * 16);
  };
  // Multiply one LDS stage. FULL: all BB token blocks of the wavefront hold rows; otherwise only
  // the first nbv do (the last, partly filled tile of a group).
  auto compute = [&](const uint8_t* base, auto full) {
#pragma unroll 1
    for (int q = 0; q < 2; ++q) {
      u32x4_t A[AB];
#pragma unroll
      for (int a = 0; a < AB; ++a) A[a] = wfrag(base, wblock(a), q);
      if constexpr (decltype(full)::value) {
        u32x4_t B[BB];
#pragma unroll
        for (int b = 0; b < BB; ++b) B[b] = tfrag(base, b, q);
#pragma unroll
        for (int a = 0; a < AB; ++a)
#pragma unroll
          for (int b = 0; b < BB; ++b) acc[a][b] = mfma_bf16(A[a], B[b], acc[a][b]);
      } else {
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          if (b < nbv) {
            const u32x4_t Bb = tfrag(base, b, q);
#pragma unroll
            for (int a = 0; a < AB; ++a) acc[a][b] = mfma_bf16(A[a], Bb, acc[a][b]);
          }
        }
      }
    }
  };

  const int s_lo = p * nsteps_all / ksplit, s_hi = (p + 1) * nsteps_all / ksplit;
  if constexpr (!WT && !WGRAD) {
    // forward: k-steps of 32, four stages of 32 KB (16 weight then 16 token fragments), direct loads
    constexpr int SB = 32768;
    static_assert(BW == 256 && BT == 256, "stage layout below assumes 256 x 256 tiles");
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int s0 = s_lo * 2, s1 = s_hi * 2;
    int32_t trow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = (wave + 8 * i) * 16 + (lane & 15);
      const int r = r0 + (rr < nrows ? rr : 0);
      trow[i] = row_src ? row_src[r] : r;
    }
    const int wl32 = PACKED ? lane * 8 : (lane & 15) * K + (lane >> 4) * 8;
    constexpr int64_t kW32 = PACKED ? 512 : 32;
    auto dma = [&](int s) {
      uint8_t* base = smem + (s & 3) * SB;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int blk = wave + 8 * i;
        const bf16_t* w = wa;
        if constexpr (SWIGLU) {
          if (i == 1) {
            w = wb;
            blk -= 8;
          }
        }
        __builtin_amdgcn_global_load_lds((const void*)(w + wrow0 + (int64_t)blk * 16 * K + (int64_t)s * kW32 + wl32),
                                         (lds_ptr)(base + (wave + 8 * i) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(act + (int64_t)trow[i] * K + kcol0 + (int64_t)s * 32 + (lane >> 4) * 8),
            (lds_ptr)(base + 16384 + (wave + 8 * i) * 1024), 16, 0, 0);
    };
    // LDS byte addresses of this lane's first weight fragment (block wblock(0)) and first token
    // fragment (block wt); the others are at the constant offsets in the reads below
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);
    const uint32_t aoff = lds0 + lane * 16 + (SWIGLU ? wr * 4 : wr * 8) * 1024;
    const uint32_t boff = lds0 + 16384 + wt * 1024 + lane * 16;
    auto run = [&](auto full) {
      for (int i = 0; i < 3; ++i)
        if (s0 + i < s1) dma(s0 + i);
      for (int s = s0; s < s1; ++s) {
        const int ahead = min(2, s1 - 1 - s);  // steps issued after s (4 loads each)
        if (ahead >= 2)
          __builtin_amdgcn_s_waitcnt(0xF78);  // vmcnt(8)
        else if (ahead == 1)
          __builtin_amdgcn_s_waitcnt(0xF74);  // vmcnt(4)
        else
          __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        // a bare barrier: a fence here would make the compiler wait for every load in flight
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (s + 3 < s1) dma(s + 3);
        const uint32_t st = (uint32_t)(s & 3) * SB;
        const uint32_t av = aoff + st, bv = boff + st;
        // a wavefront whose token blocks are all past the group's end (in the last, partly filled
        // tile) skips its fragment reads as well as its MFMAs
        if (decltype(full)::value || nbv > 0) {
          // weight blocks wblock(0..7) (SwiGLU: 4 of w1, then the same 4 of w3, 8 blocks apart) and
          // token blocks wt + 4b; early-clobber outputs, since the reads are in flight together
          u32x4_t A0, A1, A2, A3, A4, A5, A6, A7, B0, B1, B2, B3;
          if constexpr (SWIGLU) {
            asm volatile(
                "ds_read_b128 %0, %12 offset:0\n"
                "ds_read_b128 %1, %12 offset:1024\n"
                "ds_read_b128 %2, %12 offset:2048\n"
                "ds_read_b128 %3, %12 offset:3072\n"
                "ds_read_b128 %4, %12 offset:8192\n"
                "ds_read_b128 %5, %12 offset:9216\n"
                "ds_read_b128 %6, %12 offset:10240\n"
                "ds_read_b128 %7, %12 offset:11264\n"
                "ds_read_b128 %8, %13 offset:0\n"
                "ds_read_b128 %9, %13 offset:4096\n"
                "ds_read_b128 %10, %13 offset:8192\n"
                "ds_read_b128 %11, %13 offset:12288\n"
                "s_waitcnt lgkmcnt(0)\n"
                : "=&v"(A0), "=&v"(A1), "=&v"(A2), "=&v"(A3), "=&v"(A4), "=&v"(A5), "=&v"(A6), "=&v"(A7),
                  "=&v"(B0), "=&v"(B1), "=&v"(B2), "=&v"(B3)
                : "v"(av), "v"(bv)
                : "memory");
          } else {
            asm volatile(
                "ds_read_b128 %0, %12 offset:0\n"
                "ds_read_b128 %1, %12 offset:1024\n"
                "ds_read_b128 %2, %12 offset:2048\n"
                "ds_read_b128 %3, %12 offset:3072\n"
                "ds_read_b128 %4, %12 offset:4096\n"
                "ds_read_b128 %5, %12 offset:5120\n"
                "ds_read_b128 %6, %12 offset:6144\n"
                "ds_read_b128 %7, %12 offset:7168\n"
                "ds_read_b128 %8, %13 offset:0\n"
                "ds_read_b128 %9, %13 offset:4096\n"
                "ds_read_b128 %10, %13 offset:8192\n"
                "ds_read_b128 %11, %13 offset:12288\n"
                "s_waitcnt lgkmcnt(0)\n"
                : "=&v"(A0), "=&v"(A1), "=&v"(A2), "=&v"(A3), "=&v"(A4), "=&v"(A5), "=&v"(A6), "=&v"(A7),
                  "=&v"(B0), "=&v"(B1), "=&v"(B2), "=&v"(B3)
                : "v"(av), "v"(bv)
                : "memory");
          }
          const u32x4_t A[8] = {A0, A1, A2, A3, A4, A5, A6, A7};
          const u32x4_t B[4] = {B0, B1, B2, B3};
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            if (decltype(full)::value || b < nbv) {
#pragma unroll
              for (int a = 0; a < AB; ++a) acc[a][b] = mfma_bf16(A[a], B[b], acc[a][b]);
            }
          }
        }
      }
    };
    if (s0 < s1) {
      if (nbv == BB)
        run(std::true_type{});
      else
        run(std::false_type{});
    }
  } else {
    auto kloop = [&](auto full) {
      gload(s_lo);
      lstore(0);
      if (s_lo + 1 < s_hi) gload(s_lo + 1);
      __syncthreads();
      for (int s = s_lo; s < s_hi; ++s) {
        const int cur = (s - s_lo) & 1;
        if (s + 1 < s_hi) lstore(cur ^ 1);
        if (s + 2 < s_hi) gload(s + 2);
        if (decltype(full)::value || nbv > 0) compute(smem + cur * STAGE, full);
        __syncthreads();
      }
    };
    if (s_lo < s_hi) {  // an empty group (WGRAD) leaves the accumulators at zero
      if (nbv == BB)
        kloop(std::true_type{});
      else
        kloop(std::false_type{});
    }
  }

  // Epilogue: lane l holds token (l%16) of each token block and weight rows 4*(l/16)..+3.
  const int li = lane & 15, lg = lane >> 4;
  if constexpr (SWIGLU && sizeof(OutT) == 4) {
    // pre-activation pair (backward pass): a = x.w1^T to out, b = x.w3^T to part, both fp32
#pragma unroll
    for (int a = 0; a < AB / 2; ++a)
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int tr = (wt + 4 * b) * 16 + li;
        if (tr >= nrows) continue;
        const int64_t o = (int64_t)(r0 + tr) * N + n0 + (wr * (AB / 2) + a) * 16 + 4 * lg;
        store16(out + o, u32x4_t{__float_as_uint(acc[a][b][0]), __float_as_uint(acc[a][b][1]),
                                 __float_as_uint(acc[a][b][2]), __float_as_uint(acc[a][b][3])});
        const f32x4_t& v = acc[a + AB / 2][b];
        store16(part + o, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                  __float_as_uint(v[3])});
        if (hout) {  // and h = bf16(silu(a) b), as the fused epilogue below forms it
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu_t(acc[a][b][q]) * v[q];
          *reinterpret_cast<u32x2_t*>(hout + o) = u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
        }
      }
  } else if constexpr (SWIGLU) {
#pragma unroll
    for (int a = 0; a < AB / 2; ++a)
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int tr = (wt + 4 * b) * 16 + li;
        if (tr >= nrows) continue;
        const int f = n0 + (wr * (AB / 2) + a) * 16 + 4 * lg;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu_t(acc[a][b][q]) * acc[a + AB / 2][b][q];
        *reinterpret_cast<u32x2_t*>(out + (int64_t)(r0 + tr) * N + f) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  } else {
#pragma unroll
    for (int a = 0; a < AB; ++a)
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int tr = (wt + 4 * b) * 16 + li;
        if (tr >= nrows) continue;
        const int n = n0 + (wr * AB + a) * 16 + 4 * lg;
        store16(out + (int64_t)(r0 + tr) * N + n, u32x4_t{__float_as_uint(acc[a][b][0]), __float_as_uint(acc[a][b][1]),
                                                          __float_as_uint(acc[a][b][2]), __float_as_uint(acc[a][b][3])});
      }
  }
}

template <int BW, int BT, bool PACKED, bool SWIGLU, typename OutT, bool WT = false>
void launch_tile(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E, const void* wa,
                 const void* wb, void* out, int K, int N, int ksplit, float* part, hipStream_t s,
                 void* hout = nullptr) {
  constexpr int NW = SWIGLU ? BW / 2 : BW;
  const int64_t max_tiles = ((rows + BT - 1) / BT + E) * (N / NW) * ksplit;
  const int64_t grid = (max_tiles + kXcds - 1) / kXcds * kXcds;
  launch_kernel((tile_gemm_kernel<BW, BT, PACKED, SWIGLU, false, WT, OutT>), dim3((unsigned)grid), dim3(512), 0, s,
                static_cast<const bf16_t*>(act), row_src, offsets, static_cast<const bf16_t*>(wa),
                static_cast<const bf16_t*>(wb), static_cast<OutT*>(out), K, N, E, ksplit, part, rows * N, 0, N,
                static_cast<bf16_t*>(hout));
}

}  // namespace

bool tile_gemm_applies(int dtype, int64_t rows, int E, int d, int F) {
  // bf16 only; large groups; shapes that the 256 x 256 tiles and 64-deep k-steps divide
  return dtype == kBF16 && rows >= 128 * (int64_t)E && F % 128 == 0 && d % 256 == 0 && F % 64 == 0;
}

int tile_down_ksplit(int dtype, int64_t rows, int E, int d, int F) {
  if (!tile_gemm_applies(dtype, rows, E, d, F)) return 1;
  // Expected tiles of the down projection (a group of n rows takes n/256 + 1/2 token tiles on
  // average), spread over 256 CUs in rounds of one tile per CU. A split into ks k-ranges turns
  // each round into 1/ks of a round; every extra range costs one more fp32 partial written and
  // read back (8*rows*d bytes at ~6.5 TB/s), expressed in tile times (a 256 x 256 x F tile at
  // ~4 TFLOP/s per CU), plus a fixed 0.2 tile times (the fill and drain of each range's k-loop
  // and output; fitted to step times measured with the split forced to 1..4: prefill T = 4096
  // is fastest at 2, the skewed T = 16384 layer at 1, the T = 2048 stack within 0.5% at 2..4).
  // The split depends on the sizes only, so the workspace size does too.
  const double per_e = (double)rows / E;
  const double tiles = (double)E * (per_e / 256.0 + 0.5) * (d / 256);
  const double tile_s = 2.0 * 256 * 256 * (double)F / 4.0e12;
  const double part_s = 8.0 * (double)rows * d / 6.5e12;
  int best = 1;
  double best_t = 1e30;
  for (int ks = 1; ks <= kMaxKSplit && F / 64 >= 8 * ks; ++ks) {
    const double t = std::ceil(tiles * ks / 256.0) / ks + (ks - 1) * (part_s / tile_s + 0.2);
    if (t < best_t) {
      best_t = t;
      best = ks;
    }
  }
  return best;
}

void launch_tile_wgrad(const void* p, int M, int ldp, const void* q, int N, int ldq, const int32_t* offsets, int E,
                       float* out, hipStream_t s) {
  const int64_t tiles = (int64_t)E * (M / 256) * (N / 256);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  launch_kernel((tile_gemm_kernel<256, 256, false, false, true, true, float>), dim3((unsigned)grid), dim3(512), 0, s,
                static_cast<const bf16_t*>(p), static_cast<const int32_t*>(nullptr), offsets,
                static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(nullptr), out, ldp, N, E, 1,
                static_cast<float*>(nullptr), (int64_t)0, M, ldq, static_cast<bf16_t*>(nullptr));
}

void launch_tile_up(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int d,
                    int F, int E, const void* w1, const void* w3, void* h, hipStream_t s) {
  if (layout == kPacked)
    launch_tile<256, 256, true, true, bf16_t>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr, s);
  else
    launch_tile<256, 256, false, true, bf16_t>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr, s);
}

void launch_tile_up_pair(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                         int d, int F, int E, const void* w1, const void* w3, float* a, float* b, hipStream_t s,
                         void* h) {
  if (layout == kPacked)
    launch_tile<256, 256, true, true, float>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
  else
    launch_tile<256, 256, false, true, float>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
}

void launch_tile_wt(const void* act, const int32_t* offsets, int64_t rows, int N, int K, int E, const void* wa,
                    const void* wb, float* out, int ksplit, float* part, hipStream_t s) {
  launch_tile<256, 256, false, false, float, true>(act, nullptr, offsets, rows, E, wa, wb, out, K, N, ksplit, part, s);
}

void launch_tile_down(int layout, const void* h, const int32_t* offsets, int64_t rows, int d, int F, int E,
                      const void* w2, float* y_perm, int ksplit, float* y_part, hipStream_t s) {
  if (layout == kPacked)
    launch_tile<256, 256, true, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, ksplit, y_part,
                                             s);
  else
    launch_tile<256, 256, false, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, ksplit, y_part,
                                              s);
}

}  // namespace moe
