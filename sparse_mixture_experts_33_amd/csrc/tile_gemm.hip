// Tiled grouped GEMM for large expert groups (prefill): the same two projections as the
// streaming kernel (SwiGLU expert, xyznot.com summary "Método"; only routed rows exist, ja.news.hada.io
// summary on zero-gate experts), shaped for the matrix cores instead of for the weight stream.
//
//   C[w][t] = sum_k W[w][k] * X[t][k]     (w: weight row = output column, t: token row of the group)
//
// Workgroup tile: BW = 256 weight rows x up to BT token rows (SwiGLU: 128 rows of w1 and the same
// 128 rows of w3, so that silu(a)*b is formed in registers); BT = 320 for the products over token
// rows (forward, and the backward's products on transposed weights), 256 for the weight gradients.
// Eight wavefronts (two per SIMD, so one's LDS and memory waits overlap the other's MFMAs) in a
// 2 x 4 arrangement, each 128 weight rows x BT/4 tokens, 16x16x32 bf16 MFMAs accumulating in fp32
// (160 accumulator registers per lane at BT = 320).
//
// LDS holds the row-major operands in matrix-core fragment order: a fragment is 16 rows x 32 k,
// 1 KB, lane l holding row l%16 and k = 8*(l/16)..+7. Every global->LDS write and every
// LDS->register read of a wavefront is then one contiguous 1 KB, free of bank conflicts. Weights in
// the packed layout arrive already in that order (1 KB contiguous global loads). Operands stored
// k-major (the backward pass's transposed weights, and both operands of the weight gradients) are
// staged as they lie, 32 rows of 256 columns per k-step, and each matrix-core operand is assembled
// by two transposing LDS reads (ds_read_b64_tr_b16: in each group of 16 lanes, lanes 4a..4a+3
// address the 16 columns of row a, and lane i receives column i of the 4 rows, which is 4
// consecutive k of output row i). Such a block is 16 slots of two 512-byte rows (rows r and r + 4,
// r = (j & 3) + 8 (j >> 2) for slot j), 1056 bytes apart: the 16 rows one transposing read touches
// then lie in 16 different slots, whose 32-byte offsets spread them over all banks. Packed
// transposed weights arrive as 1 KB fragments of 16 k rows x 32 columns and are read the same way
// (the fragment layout in the kernel below).
//
// Tiles are numbered expert-major, then in bands of 4 token tiles, then weight tile, then token
// tile within the band, so that the 32 tiles an XCD runs at once share 4 token and 8 weight row
// blocks; the linear index is remapped so that adjacent tiles go to workgroups on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs), which keeps those blocks in that XCD's L2.
//
// A group of n rows takes ceil(n / BT) token tiles and its 16-row blocks are dealt over them as
// evenly as possible, so no tile holds only a few rows (such a tile would stream a whole slice of
// the expert's weights for them). Token blocks are dealt to the four token wavefronts round-robin
// (wavefront t owns blocks t, t+4, ...), so a partly filled tile spreads its rows over the SIMDs;
// a wavefront skips the MFMAs (and fragment reads) of blocks that lie wholly past the tile's rows.
// Token rows past the end inside a block load a valid row and are never stored.
//
// Every product runs k-steps of 32 through four LDS stages (the weight block, then the token
// block), filled by direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land at
// the destination + 16 l), so three steps are in flight while one is multiplied and no registers
// stage the data. Per step s: wait until this wavefront's loads of step s have landed (vmcnt,
// counting the loads issued after them), barrier (then every wavefront's have, and every wavefront
// is done with step s-1), read the fragments of step s, multiply, then issue step s+3 into the
// stage that step s-1 used. The loads go after the MFMAs because issuing them can hold a wavefront
// for hundreds of cycles when the vector-memory queue is full; issued last, that wait overlaps the
// other wavefront's MFMAs on the same SIMD. The fragment reads are inline assembly that waits for
// its own results: the compiler cannot tell them apart from the asynchronous LDS writes and would
// otherwise wait for every load in flight before each read; for the same reason the barrier is a
// bare s_barrier (a workgroup fence makes the compiler drain all loads first). The weight
// gradients run over each group's rows: the last step of a group may be partial, and its rows past
// the group's end are loaded from valid rows and zeroed in registers before the MFMAs.
#include "common.hpp"
#include "launch.hpp"

#include <cmath>
#include <type_traits>

namespace moe {
namespace {

constexpr int kXcds = 8;
constexpr int kBT = 320;  // token rows per tile (at most) of the products over token rows

// SBWD: what the backward pass's pre-activation product finishes in its epilogue (the SwiGLU
// derivative), given dh' = w2^T dy of every row (see swiglu_bwd_elem).
struct SwigluBwdArgs {
  const float* dhp = nullptr;    // [rows][N] dh' (fp32)
  const float* row_g = nullptr;  // [rows] the gate of each row
  int64_t rows = 0;
  bf16_t* dab = nullptr;  // [rows][2N]: bf16(da) | bf16(db)
  float* dgp = nullptr;   // [N/64][rows]: gate-gradient partial of each 64-column chunk
  void* sink = nullptr;   // 16 bytes that take the stores of rows past a tile's end
};

// WGRAD: weight-gradient mode of the backward pass. Per expert e the product runs over the rows of
// e's group instead of over a fixed K: out[e][m][n] = sum over the group's rows r of
// act[r][m] * wa[r][n], with act [rows][.] (row stride K) and wa [rows][.] (row stride ldw) the
// group-sorted rows as they lie (WGRAD requires WT: both operands k-major). A k-step takes 32 rows
// of the group; rows past its end are zeroed in registers. The group sizes come from `offsets` on
// the device. Tiles are (expert, n tile, m tile), one 256 x 256 output tile each.
//
// WT: the weight operand is stored transposed, [E][K][N] with the N columns contiguous (the layout
// in which the backward pass holds w2 and w1, w3 for its products): wa holds k < KA = K/2 and wb
// the rest when wb is given (KA = K otherwise). With PACKED the [E][K][N] weights are
// fragment-packed (1 KB fragments of 16 k rows x 32 n columns, as moe_pack_weights writes them
// with N as the contiguous dimension): a k-step's 32 x 256 block is 16 whole fragments, which the
// transposing reads take apart like the row-major block.
// WGRAD with PACKED writes out[e] in that same fragment-packed element order ([M][N] weights:
// 16 m rows x 32 n columns per 512-element fragment), so a gradient lines up with packed weights.
// HPK: the hidden activations h between the two forward products are fragment-packed: the up
// product stores h (and the pair product its h output) and the down product reads it as its token
// operand in 1 KB fragments of 16 rows x 32 columns (lane l: row l % 16, columns 8 (l / 16)..+7),
// fragments of a 16-row block consecutive along F. Each group's rows start a new block: row r of
// group e is packed row hpk_row0(e) + r - offsets[e], hpk_row0(e) = sum over e' < e of the group
// sizes rounded up to 16. Packed rows past a group's end are never written; the down product reads
// them with their block, and the output rows they produce are not stored.
// SBWD (backward pass, SWIGLU): instead of storing a = x.w1^T and b = x.w3^T, the epilogue reads dh'
// at the same elements and stores h = bf16(silu(a) b) to out (row-major [rows][N]), [da | db] and the
// gate-gradient partials (swiglu_bwd_elem, dg_quad: the lane's four 16-column blocks pairwise, then
// the four lanes of a row pairwise, one partial per 64-column chunk of a wavefront).
template <int BW, int BT, bool PACKED, bool SWIGLU, bool WGRAD, bool WT, typename OutT, bool HPK = false,
          bool SBWD = false>
__global__ __launch_bounds__(512, 1) void tile_gemm_kernel(const bf16_t* __restrict__ act,
                                                           const int32_t* __restrict__ row_src,
                                                           const int32_t* __restrict__ offsets,
                                                           const bf16_t* __restrict__ wa,
                                                           const bf16_t* __restrict__ wb, OutT* __restrict__ out,
                                                           int K, int N, int E, int ksplit, float* __restrict__ part,
                                                           int64_t part_stride, int M, int ldw,
                                                           bf16_t* __restrict__ hout, SwigluBwdArgs sb) {
  static_assert(!WGRAD || (!SWIGLU && WT), "the weight-gradient mode reads both operands k-major");
  static_assert(!WT || !SWIGLU, "transposed weights: plain product only");
  static_assert(!HPK || (!WT && !WGRAD), "packed h: forward products only");
  static_assert(!SBWD || (SWIGLU && !HPK && sizeof(OutT) == 2), "SwiGLU derivative: the pair product, h row-major");
  static_assert(BW == 256 && (BT == 256 || (BT == 320 && !WGRAD)), "tiles are 256 x 256, or 256 x 320 but for WGRAD");
  constexpr int NW = SWIGLU ? BW / 2 : BW;  // output columns per tile
  constexpr int AB = BW / 32;               // weight blocks per wavefront
  constexpr int BB = BT / 64;               // token blocks per wavefront
  constexpr int TB = BT / 16;               // token fragments per stage (fragment-order tokens)
  constexpr int TI = (TB + 7) / 8;          // token fragment slots per wavefront
  // A k-major operand block (WT weights, WGRAD tokens) takes 16 slots of two 512-byte rows, 32
  // bytes apart beyond 1 KB so that the 16 rows one transposing read touches spread over the banks.
  constexpr int KSLOT = 1056;
  constexpr int WPB = WT ? 16 * KSLOT : 16 * 1024;     // bytes of the weight block per stage
  constexpr int TPB = WGRAD ? 16 * KSLOT : TB * 1024;  // bytes of the token block per stage
  constexpr int SB = WPB + TPB;                        // bytes per stage

  __shared__ __attribute__((aligned(16))) uint8_t smem[WGRAD ? SB : 4 * SB];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_tile0[kMaxExperts + 1];
  __shared__ int32_t s_hpk0[HPK ? kMaxExperts + 1 : 1];  // HPK: first packed row of each group
  // WGRAD's other three stages are separate arrays, so that in its steady-state loop (below) the
  // compiler can tell, for a stage named statically, that the direct loads in flight into the other
  // stages do not write what it reads; the other modes keep the four stages in smem
  __shared__ __attribute__((aligned(16))) uint8_t stg1[WGRAD ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t stg2[WGRAD ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t stg3[WGRAD ? SB : 16];

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
    if constexpr (HPK) {
      int p0 = 0;
      for (int e = 0; e < E; ++e) {
        s_hpk0[e] = p0;
        p0 += (s_off[e + 1] - s_off[e] + 15) & ~15;
      }
    }
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
    const int n_e = s_off[e + 1] - s_off[e];
    const int mtiles = (n_e + BT - 1) / BT;
    // the group's rows are dealt over its mtiles token tiles in whole 16-row blocks, as evenly as
    // possible (q blocks per tile, the last tile the rest), so no tile holds only a few rows
    const int q = ((n_e + 15) / 16 + mtiles - 1) / mtiles;
    const int local = tile - s_tile0[e];
    // token tiles in bands of 4: within a band the token tile varies fastest, then the weight
    // tile, so the 32 tiles an XCD runs at once cover 4 token x 8 weight tiles even for a group
    // of many token tiles (a group of at most 4 is a single band: weight-tile major)
    const int band = local / (4 * NT), mb = band * 4, bs = min(4, mtiles - mb);
    const int w = local - band * 4 * NT;
    mt = mb + w % bs;
    nt = w / bs;
    r0 = s_off[e] + mt * q * 16;
    nrows = min(q * 16, s_off[e + 1] - r0);
    nsteps_all = K / 64;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  kcol0 = __builtin_amdgcn_readfirstlane((int)kcol0);
  nsteps_all = __builtin_amdgcn_readfirstlane(nsteps_all);
  // HPK: packed 16-row block of the tile's first row (tiles start 16-aligned within their group)
  const int pb0 = HPK ? (s_hpk0[e] + r0 - s_off[e]) >> 4 : 0;
  // token blocks of this wavefront that hold at least one row of the group
  const int nbv = min(BB, max(0, ((nrows + 15) / 16 - wt + 3) / 4));
  const int n0 = nt * NW;
  if constexpr (!SWIGLU) {
    if (p > 0) out = reinterpret_cast<OutT*>(part + (int64_t)(p - 1) * part_stride);
  }

  f32x4_t acc[AB][BB];
#pragma unroll
  for (int a = 0; a < AB; ++a)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // k-steps of 32 through four LDS stages, each the tile's weight block then its token block,
  // filled by direct global->LDS loads. Wavefront w issues the loads of fragments / slots w and
  // w + 8 of the weight block and its share of the token block.
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int n_e = s_off[e + 1] - s_off[e];
  int s0, s1;
  if constexpr (WGRAD) {
    s0 = 0;
    s1 = (n_e + 31) / 32;  // the group's rows, 32 per step; the last step may be partial
  } else {
    s0 = p * nsteps_all / ksplit * 2;  // k-range p of ksplit, split at 64-deep boundaries
    s1 = (p + 1) * nsteps_all / ksplit * 2;
  }
  s0 = __builtin_amdgcn_readfirstlane(s0);
  s1 = __builtin_amdgcn_readfirstlane(s1);
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);
  auto stage_of = [&](int s) -> uint8_t* {  // stage of step s (WGRAD: s0 = 0)
    if constexpr (WGRAD) {
      const int k = s & 3;
      return k == 0 ? smem : k == 1 ? stg1 : k == 2 ? stg2 : stg3;
    } else {
      return smem + (s & 3) * SB;
    }
  };
  // k-major operands: row R of slot j is R1(j) = (j & 3) + 8 (j >> 2) for lanes 0-31 and R1 + 4 for
  // lanes 32-63, each lane 8 consecutive columns
  const int ck = (lane & 31) * 8;
  int kR[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + 8 * i;
    kR[i] = (j & 3) + 8 * (j >> 2) + 4 * (lane >> 5);
  }
  // transposing reads of a k-major block: lane (g = l/16, a = (l/4)%4, c = l%4) addresses row
  // 8g + a (slot a + 4g) and row 8g + a + 4 (512 bytes further), columns 4c..4c+3 of the block
  const uint32_t ktr = (uint32_t)((((lane >> 2) & 3) + 4 * (lane >> 4)) * KSLOT + 8 * (lane & 3));
  // fragment-order token operand (forward, WT): fragments wave + 8 i that hold rows of the tile
  const int nblk = (nrows + 15) / 16;
  int32_t trow[TI];
  int ntl = 0;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int rr = (wave + 8 * i) * 16 + (lane & 15);
    const int r = r0 + (rr < nrows ? rr : 0);
    trow[i] = WGRAD ? 0 : (row_src ? row_src[r] : r);
    ntl += (wave + 8 * i < TB && wave + 8 * i < nblk) ? 1 : 0;
  }
  const int nl = 2 + (WGRAD ? 2 : ntl);  // loads per step (uniform over the wavefront)
  // SBWD: the gates of this lane's epilogue rows, loaded with the row indices (before the k-loop)
  float sgate[SBWD ? BB : 1];
  if constexpr (SBWD) {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const int tr = (wt + 4 * b) * 16 + (lane & 15);
      sgate[b] = sb.row_g[r0 + (tr < nrows ? tr : 0)];
    }
  }
  const int wl32 = PACKED ? lane * 8 : (lane & 15) * K + (lane >> 4) * 8;
  constexpr int64_t kW32 = PACKED ? 512 : 32;
  const int64_t wrow0 = ((int64_t)e * N + n0) * K;  // forward: first element of the tile's weights
  const int KA = (WT && wb) ? K / 2 : K;             // WT: rows of wa (wb holds the rest)
  const int klast = s_off[E] - 1;                    // WGRAD: last row of the operands
  auto dma_to = [&](uint8_t* base, int s) {  // step s into stage `base`
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = wave + 8 * i;
      const bf16_t* src;
      if constexpr (WGRAD) {
        // rows past the group's end are loaded from valid rows and masked in registers
        const int64_t kc = min((int)kcol0 + s * 32 + kR[i], klast);
        src = wa + kc * ldw + n0 + ck;
      } else if constexpr (WT) {
        const bool second = wb && s * 32 >= KA;  // uniform over the step (KA is a multiple of 32)
        const bf16_t* w = second ? wb : wa;
        if constexpr (PACKED) {
          // fragment (k block i, n block `wave`) of the step's 32 x 256 block
          const int64_t kb = 2 * ((int64_t)s - (second ? KA / 32 : 0)) + i;
          src = w + (((int64_t)e * (KA / 16) + kb) * (N / 32) + n0 / 32 + wave) * 512 + lane * 8;
        } else {
          const int64_t k = (int64_t)s * 32 - (second ? KA : 0) + kR[i];
          src = w + ((int64_t)e * KA + k) * ldw + n0 + ck;
        }
      } else {
        int blk = j;
        const bf16_t* w = wa;
        if constexpr (SWIGLU) {
          if (i == 1) {
            w = wb;
            blk -= 8;
          }
        }
        src = w + wrow0 + (int64_t)blk * 16 * K + (int64_t)s * kW32 + wl32;
      }
      // packed transposed weights: the fragments in pairs (n blocks 2p', 2p' + 1 of a k block) of 2112
      // bytes, the odd one 1088 bytes into its pair (see the reads)
      const int dst = WT && PACKED && !WGRAD ? (i * 4 + (wave >> 1)) * 2112 + (wave & 1) * 1088
                                             : j * (WT ? KSLOT : 1024);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(base + dst), 16, 0, 0);
    }
    if constexpr (WGRAD) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t kc = min((int)kcol0 + s * 32 + kR[i], klast);
        __builtin_amdgcn_global_load_lds((const void*)(act + kc * K + r0 + ck),
                                         (lds_ptr)(base + WPB + (wave + 8 * i) * KSLOT), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        if (i < ntl)  // the loaded fragments are the first ntl slots (blocks grow with i)
          __builtin_amdgcn_global_load_lds(
              (HPK && !SWIGLU)  // the down product reads packed h; the up products read x rows
                  ? (const void*)(act + ((int64_t)(pb0 + wave + 8 * i) * (K / 32) + s) * 512 + lane * 8)
                  : (const void*)(act + (int64_t)trow[i] * K + kcol0 + (int64_t)s * 32 + (lane >> 4) * 8),
              (lds_ptr)(base + WPB + (wave + 8 * i) * 1024), 16, 0, 0);
    }
  };
  auto dma = [&](int s) { dma_to(stage_of(s), s); };
  // Wait until at most n loads of this wavefront are in flight (n = a multiple of nl <= 2 * 5).
  auto wait_vm = [](int n) {
    switch (n) {
      case 10: __builtin_amdgcn_s_waitcnt(0xF7A); break;  // vmcnt(10)
      case 9: __builtin_amdgcn_s_waitcnt(0xF79); break;
      case 8: __builtin_amdgcn_s_waitcnt(0xF78); break;
      case 7: __builtin_amdgcn_s_waitcnt(0xF77); break;
      case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
      case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
      case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
      case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
      case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
      default: __builtin_amdgcn_s_waitcnt(0xF70); break;  // vmcnt(0)
    }
  };
  // LDS byte addresses of this lane's first weight fragment (block wblock(0)) and first token
  // fragment (block wt) in stage 0; the others are at the constant offsets in the reads below
  // packed transposed weights: a 16-column block of the matrix cores takes 8 columns (chunk a % 4) of
  // each of the n fragments 2 (a / 4) and 2 (a / 4) + 1 of the wavefront (columns 128 wr + 64 (a / 4) +
  // 32 h + 8 (a % 4) + 0..7, h = 0, 1). A pair of fragments takes 2112 bytes of the stage, its odd one
  // 1088 bytes in (64 bytes further modulo 256). Lane (g, a', c) of a transposing read reads row 8g + a'
  // of the step (k block g / 2, fragment row 8 (g % 2) + a') and 4 columns of fragment h = c / 2 at chunk
  // byte 16 row + 8 (c % 2): the 32 lanes of each half-wavefront touch 256 different bytes (with both
  // halves of a block in one fragment, lanes 256 bytes apart would share banks)
  constexpr bool kTrPk = WT && PACKED && !WGRAD;
  static_assert(!kTrPk || AB == 8, "packed transposed weights: 256-column weight tiles");
  constexpr int kTrH = kTrPk ? 64 : 512;  // rows + 4 of a read
  auto tr_off = [](int a) constexpr { return kTrPk ? (a / 4) * 2112 + (a % 4) * 256 : a * 32; };  // block a
  const uint32_t ktrp = (uint32_t)((lane >> 5) * (4 * 2112) + ((lane >> 1) & 1) * 1088 +
                                   (8 * ((lane >> 4) & 1) + ((lane >> 2) & 3)) * 16 + (lane & 1) * 8);
  const uint32_t aoff = WT ? lds0 + (kTrPk ? ktrp + wr * (2 * 2112) : ktr + wr * 256)
                           : lds0 + lane * 16 + (SWIGLU ? wr * 4 : wr * 8) * 1024;
  const uint32_t boff = WGRAD ? lds0 + WPB + ktr + wt * 32 : lds0 + WPB + wt * 1024 + lane * 16;
  // WGRAD steady state: four steps per iteration with the stages named statically and the
  // transposing fragment reads written as builtins, so that the compiler can schedule the reads of
  // one step among the MFMAs of the previous one (it overlaps about half of them). Every wavefront
  // issues 2 + 2 loads per step; runs while step s + 3 exists.
  auto wgrad_step = [&](auto kc, int s) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    uint8_t* cur = k == 0 ? smem : k == 1 ? stg1 : k == 2 ? stg2 : stg3;
    uint8_t* nxt = k == 0 ? stg3 : k == 1 ? smem : k == 2 ? stg1 : stg2;  // stage of step s + 3
    // vmcnt(8) and lgkmcnt(0): this wavefront's loads of steps <= s have landed and its reads of
    // step s - 1 are complete, so after the barrier every wavefront's are, and the loads issued
    // into that stage below cannot overtake a read of it
    __builtin_amdgcn_s_waitcnt(0x0078);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");      // no LDS access moves above the barrier
    typedef __attribute__((ext_vector_type(4))) short v4s;
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    auto tr = [](const uint8_t* q) __attribute__((always_inline)) -> u32x4_t {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q + 512));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
      return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
    };
    const uint32_t ao = ktr + wr * 256, bo = WPB + ktr + wt * 32;  // this lane's first fragments
    u32x4_t A[AB], B[BB];
#pragma unroll
    for (int a = 0; a < AB; ++a) A[a] = tr(cur + ao + a * 32);
#pragma unroll
    for (int b = 0; b < BB; ++b) B[b] = tr(cur + bo + b * 128);
#pragma unroll
    for (int b = 0; b < BB; ++b)
#pragma unroll
      for (int a = 0; a < AB; ++a) acc[a][b] = mfma_bf16(A[a], B[b], acc[a][b]);
    asm volatile("" ::: "memory");  // the loads of step s + 3 stay behind this step's reads
    dma_to(nxt, s + 3);
  };

  // General steps from s_begin (dynamic stage, wait count and token blocks); from s0 it issues the
  // first three steps first.
  auto run = [&](int s_begin, auto full) {
    if (s_begin == s0)
      for (int i = 0; i < 3; ++i)
        if (s0 + i < s1) dma(s0 + i);
    for (int s = s_begin; s < s1; ++s) {
      const int ahead = min(2, s1 - 1 - s);  // steps issued after s (nl loads each)
      wait_vm(ahead * nl);
      // a bare barrier: a fence here would make the compiler wait for every load in flight
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t st = WGRAD ? (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)stage_of(s)) - lds0
                                : (uint32_t)(s & 3) * SB;
      const uint32_t av = aoff + st, bv = boff + st;
      // a wavefront whose token blocks are all past the tile's rows skips its fragment reads as
      // well as its MFMAs
      if (decltype(full)::value || nbv > 0) {
        // weight blocks wblock(0..7) and token blocks wt + 4b; early-clobber outputs, since the
        // reads are in flight together
        u32x4_t A[8], B[5];
        if constexpr (WT) {
          // k-major weights: two transposing reads per fragment (rows 8g + a and 8g + a + 4)
          u32x2_t L0, L1, L2, L3, L4, L5, L6, L7, H0, H1, H2, H3, H4, H5, H6, H7;
#define MOE_TR_A                                                                                              \
  "ds_read_b64_tr_b16 %[l0], %[av] offset:%[ol0]\n"                                                           \
  "ds_read_b64_tr_b16 %[h0], %[av] offset:%[oh0]\n"                                                           \
  "ds_read_b64_tr_b16 %[l1], %[av] offset:%[ol1]\n"                                                           \
  "ds_read_b64_tr_b16 %[h1], %[av] offset:%[oh1]\n"                                                           \
  "ds_read_b64_tr_b16 %[l2], %[av] offset:%[ol2]\n"                                                           \
  "ds_read_b64_tr_b16 %[h2], %[av] offset:%[oh2]\n"                                                           \
  "ds_read_b64_tr_b16 %[l3], %[av] offset:%[ol3]\n"                                                           \
  "ds_read_b64_tr_b16 %[h3], %[av] offset:%[oh3]\n"                                                           \
  "ds_read_b64_tr_b16 %[l4], %[av] offset:%[ol4]\n"                                                           \
  "ds_read_b64_tr_b16 %[h4], %[av] offset:%[oh4]\n"                                                           \
  "ds_read_b64_tr_b16 %[l5], %[av] offset:%[ol5]\n"                                                           \
  "ds_read_b64_tr_b16 %[h5], %[av] offset:%[oh5]\n"                                                           \
  "ds_read_b64_tr_b16 %[l6], %[av] offset:%[ol6]\n"                                                           \
  "ds_read_b64_tr_b16 %[h6], %[av] offset:%[oh6]\n"                                                           \
  "ds_read_b64_tr_b16 %[l7], %[av] offset:%[ol7]\n"                                                           \
  "ds_read_b64_tr_b16 %[h7], %[av] offset:%[oh7]\n"
#define MOE_TR_OUT_A                                                                                          \
  [l0] "=&v"(L0), [l1] "=&v"(L1), [l2] "=&v"(L2), [l3] "=&v"(L3), [l4] "=&v"(L4), [l5] "=&v"(L5),            \
      [l6] "=&v"(L6), [l7] "=&v"(L7), [h0] "=&v"(H0), [h1] "=&v"(H1), [h2] "=&v"(H2), [h3] "=&v"(H3),         \
      [h4] "=&v"(H4), [h5] "=&v"(H5), [h6] "=&v"(H6), [h7] "=&v"(H7)
// weight block a at tr_off(a) bytes, its rows + 4 kTrH further (row-major slots / packed fragments)
#define MOE_TR_IN_A                                                                                           \
  [ol0] "i"(tr_off(0)), [ol1] "i"(tr_off(1)), [ol2] "i"(tr_off(2)), [ol3] "i"(tr_off(3)),                    \
      [ol4] "i"(tr_off(4)), [ol5] "i"(tr_off(5)), [ol6] "i"(tr_off(6)), [ol7] "i"(tr_off(7)),               \
      [oh0] "i"(tr_off(0) + kTrH), [oh1] "i"(tr_off(1) + kTrH), [oh2] "i"(tr_off(2) + kTrH),                 \
      [oh3] "i"(tr_off(3) + kTrH), [oh4] "i"(tr_off(4) + kTrH), [oh5] "i"(tr_off(5) + kTrH),                 \
      [oh6] "i"(tr_off(6) + kTrH), [oh7] "i"(tr_off(7) + kTrH)
          if constexpr (WGRAD) {
            // k-major tokens too: blocks wt + 4b at 128-byte steps
            u32x2_t M0, M1, M2, M3, N0, N1, N2, N3;
            asm volatile(MOE_TR_A
                         "ds_read_b64_tr_b16 %[m0], %[bv] offset:0\n"
                         "ds_read_b64_tr_b16 %[n0], %[bv] offset:512\n"
                         "ds_read_b64_tr_b16 %[m1], %[bv] offset:128\n"
                         "ds_read_b64_tr_b16 %[n1], %[bv] offset:640\n"
                         "ds_read_b64_tr_b16 %[m2], %[bv] offset:256\n"
                         "ds_read_b64_tr_b16 %[n2], %[bv] offset:768\n"
                         "ds_read_b64_tr_b16 %[m3], %[bv] offset:384\n"
                         "ds_read_b64_tr_b16 %[n3], %[bv] offset:896\n"
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_TR_OUT_A, [m0] "=&v"(M0), [m1] "=&v"(M1), [m2] "=&v"(M2), [m3] "=&v"(M3),
                           [n0] "=&v"(N0), [n1] "=&v"(N1), [n2] "=&v"(N2), [n3] "=&v"(N3)
                         : [av] "v"(av), [bv] "v"(bv), MOE_TR_IN_A
                         : "memory");
            B[0] = u32x4_t{M0[0], M0[1], N0[0], N0[1]};
            B[1] = u32x4_t{M1[0], M1[1], N1[0], N1[1]};
            B[2] = u32x4_t{M2[0], M2[1], N2[0], N2[1]};
            B[3] = u32x4_t{M3[0], M3[1], N3[0], N3[1]};
          } else if constexpr (BB == 5) {
            asm volatile(MOE_TR_A
                         "ds_read_b128 %[b0], %[bv] offset:0\n"
                         "ds_read_b128 %[b1], %[bv] offset:4096\n"
                         "ds_read_b128 %[b2], %[bv] offset:8192\n"
                         "ds_read_b128 %[b3], %[bv] offset:12288\n"
                         "ds_read_b128 %[b4], %[bv] offset:16384\n"
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_TR_OUT_A, [b0] "=&v"(B[0]), [b1] "=&v"(B[1]), [b2] "=&v"(B[2]), [b3] "=&v"(B[3]),
                           [b4] "=&v"(B[4])
                         : [av] "v"(av), [bv] "v"(bv), MOE_TR_IN_A
                         : "memory");
          } else {
            asm volatile(MOE_TR_A
                         "ds_read_b128 %[b0], %[bv] offset:0\n"
                         "ds_read_b128 %[b1], %[bv] offset:4096\n"
                         "ds_read_b128 %[b2], %[bv] offset:8192\n"
                         "ds_read_b128 %[b3], %[bv] offset:12288\n"
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_TR_OUT_A, [b0] "=&v"(B[0]), [b1] "=&v"(B[1]), [b2] "=&v"(B[2]), [b3] "=&v"(B[3])
                         : [av] "v"(av), [bv] "v"(bv), MOE_TR_IN_A
                         : "memory");
          }
#undef MOE_TR_A
#undef MOE_TR_OUT_A
#undef MOE_TR_IN_A
          A[0] = u32x4_t{L0[0], L0[1], H0[0], H0[1]};
          A[1] = u32x4_t{L1[0], L1[1], H1[0], H1[1]};
          A[2] = u32x4_t{L2[0], L2[1], H2[0], H2[1]};
          A[3] = u32x4_t{L3[0], L3[1], H3[0], H3[1]};
          A[4] = u32x4_t{L4[0], L4[1], H4[0], H4[1]};
          A[5] = u32x4_t{L5[0], L5[1], H5[0], H5[1]};
          A[6] = u32x4_t{L6[0], L6[1], H6[0], H6[1]};
          A[7] = u32x4_t{L7[0], L7[1], H7[0], H7[1]};
          if constexpr (WGRAD) {
            if ((n_e & 31) && s == s1 - 1) {
              // last, partial step of the group: zero the k (row) entries past its end in both
              // operands; lane l holds k = 8(l/16)..+7, two per register
              const int lim = n_e - s * 32 - 8 * (lane >> 4);
              uint32_t m[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) m[q] = 2 * q + 1 < lim ? 0xFFFFFFFFu : (2 * q < lim ? 0x0000FFFFu : 0u);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int a = 0; a < 8; ++a) A[a][q] &= m[q];
#pragma unroll
                for (int b = 0; b < 4; ++b) B[b][q] &= m[q];
              }
            }
          }
        } else {
          // fragment-order weights (SwiGLU: 4 blocks of w1, then the same 4 of w3, 8 blocks apart)
          u32x4_t A0, A1, A2, A3, A4, A5, A6, A7, B0, B1, B2, B3, B4;
#define MOE_RD_A(o0, o1, o2, o3, o4, o5, o6, o7)                                   \
  "ds_read_b128 %[a0], %[av] offset:" #o0 "\n"                                    \
  "ds_read_b128 %[a1], %[av] offset:" #o1 "\n"                                    \
  "ds_read_b128 %[a2], %[av] offset:" #o2 "\n"                                    \
  "ds_read_b128 %[a3], %[av] offset:" #o3 "\n"                                    \
  "ds_read_b128 %[a4], %[av] offset:" #o4 "\n"                                    \
  "ds_read_b128 %[a5], %[av] offset:" #o5 "\n"                                    \
  "ds_read_b128 %[a6], %[av] offset:" #o6 "\n"                                    \
  "ds_read_b128 %[a7], %[av] offset:" #o7 "\n"
#define MOE_RD_B4                                                                  \
  "ds_read_b128 %[b0], %[bv] offset:0\n"                                          \
  "ds_read_b128 %[b1], %[bv] offset:4096\n"                                       \
  "ds_read_b128 %[b2], %[bv] offset:8192\n"                                       \
  "ds_read_b128 %[b3], %[bv] offset:12288\n"
#define MOE_RD_OUT_A                                                                                  \
  [a0] "=&v"(A0), [a1] "=&v"(A1), [a2] "=&v"(A2), [a3] "=&v"(A3), [a4] "=&v"(A4), [a5] "=&v"(A5),       \
      [a6] "=&v"(A6), [a7] "=&v"(A7), [b0] "=&v"(B0), [b1] "=&v"(B1), [b2] "=&v"(B2), [b3] "=&v"(B3)
#define MOE_RD_IN : [av] "v"(av), [bv] "v"(bv) : "memory"
          if constexpr (SWIGLU && BB == 5) {
            asm volatile(MOE_RD_A(0, 1024, 2048, 3072, 8192, 9216, 10240, 11264) MOE_RD_B4
                         "ds_read_b128 %[b4], %[bv] offset:16384\n"
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_RD_OUT_A, [b4] "=&v"(B4) MOE_RD_IN);
          } else if constexpr (SWIGLU) {
            asm volatile(MOE_RD_A(0, 1024, 2048, 3072, 8192, 9216, 10240, 11264) MOE_RD_B4
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_RD_OUT_A MOE_RD_IN);
          } else if constexpr (BB == 5) {
            asm volatile(MOE_RD_A(0, 1024, 2048, 3072, 4096, 5120, 6144, 7168) MOE_RD_B4
                         "ds_read_b128 %[b4], %[bv] offset:16384\n"
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_RD_OUT_A, [b4] "=&v"(B4) MOE_RD_IN);
          } else {
            asm volatile(MOE_RD_A(0, 1024, 2048, 3072, 4096, 5120, 6144, 7168) MOE_RD_B4
                         "s_waitcnt lgkmcnt(0)\n"
                         : MOE_RD_OUT_A MOE_RD_IN);
          }
#undef MOE_RD_A
#undef MOE_RD_B4
#undef MOE_RD_OUT_A
#undef MOE_RD_IN
          if constexpr (BB == 4) B4 = B3;  // unused: the MFMAs below take blocks b < BB only
          A[0] = A0, A[1] = A1, A[2] = A2, A[3] = A3, A[4] = A4, A[5] = A5, A[6] = A6, A[7] = A7;
          B[0] = B0, B[1] = B1, B[2] = B2, B[3] = B3, B[4] = B4;
        }
#pragma unroll
        for (int b = 0; b < BB; ++b) {
          if (decltype(full)::value || b < nbv) {
#pragma unroll
            for (int a = 0; a < AB; ++a) acc[a][b] = mfma_bf16(A[a], B[b], acc[a][b]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s + 3 < s1) dma(s + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (s0 < s1) {
    if constexpr (WGRAD) {
      const int s_fast = max(0, (s1 - 3) / 4 * 4);  // steady-state steps (s0 = 0)
      if (s_fast > 0) {
        // all three exist here; issued unconditionally (a conditional issue would cost the loop
        // below a wait for every load at its head)
        dma_to(smem, 0);
        dma_to(stg1, 1);
        dma_to(stg2, 2);
        for (int s = 0; s < s_fast; s += 4) {
          wgrad_step(std::integral_constant<int, 0>{}, s);
          wgrad_step(std::integral_constant<int, 1>{}, s + 1);
          wgrad_step(std::integral_constant<int, 2>{}, s + 2);
          wgrad_step(std::integral_constant<int, 3>{}, s + 3);
        }
      }
      run(s_fast, std::true_type{});  // the output tile's 256 rows all exist (M is a multiple of 256)
    } else {
      if (nbv == BB)
        run(s0, std::true_type{});
      else
        run(s0, std::false_type{});
    }
  }

  // Epilogue: lane l holds token (l%16) of each token block and weight rows 4*(l/16)..+3.
  const int li = lane & 15, lg = lane >> 4;
  // HPK: element offset in packed h of the 4 columns f..f+3 (f % 4 == 0) of token block tb's row li
  auto hpk_off = [&](int tb, int f) -> int64_t {
    return (((int64_t)(pb0 + tb) * (N / 32) + (f >> 5)) * 64 + li + 16 * ((f & 31) >> 3)) * 8 + (f & 7);
  };
  if constexpr (SBWD) {
    // every lane takes part in the shuffles; rows past the tile's end compute on a valid row and
    // store to the sink (stores without branches, so that the compiler keeps the arithmetic out of
    // conditional code, where its waits for the loads become waits for everything). The dh' loads run two token blocks ahead: block b + 2's go out after block b's
    // stores, so the wait for a block's loads never covers the stores of the block just before it
    // (the wait for a load also waits for every store issued before it).
    f32x4_t pvs[2][AB / 2];
    auto load_dhp = [&](int b, f32x4_t* dst) {
      const int tr = (wt + 4 * b) * 16 + li;
      const int r = r0 + (tr < nrows ? tr : 0);
#pragma unroll
      for (int a = 0; a < AB / 2; ++a)
        dst[a] = *reinterpret_cast<const f32x4_t*>(sb.dhp + (int64_t)r * N + n0 + (wr * (AB / 2) + a) * 16 + 4 * lg);
    };
    load_dhp(0, pvs[0]);
    if (BB > 1) load_dhp(1, pvs[1]);
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const int tr = (wt + 4 * b) * 16 + li;
      const bool ok = tr < nrows;
      const int r = r0 + (ok ? tr : 0);
      const float g = sgate[b];
      float v[AB / 2];
#pragma unroll
      for (int a = 0; a < AB / 2; ++a) {
        const int f = n0 + (wr * (AB / 2) + a) * 16 + 4 * lg;
        const f32x4_t pv = pvs[b & 1][a];
        float hv[4], da[4], db[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) swiglu_bwd_elem(acc[a][b][q], acc[a + AB / 2][b][q], pv[q], g, hv[q], da[q], db[q]);
        const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
        v[a] = dg_quad(pv, h01, h23);
        u32x2_t* const sink = static_cast<u32x2_t*>(sb.sink);
        u32x2_t* const ph = ok ? reinterpret_cast<u32x2_t*>(out + (int64_t)r * N + f) : sink;
        u32x2_t* const pa = ok ? reinterpret_cast<u32x2_t*>(sb.dab + (int64_t)r * 2 * N + f) : sink;
        u32x2_t* const pb = ok ? reinterpret_cast<u32x2_t*>(sb.dab + (int64_t)r * 2 * N + N + f) : sink;
        *ph = u32x2_t{h01, h23};
        *pa = u32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
        *pb = u32x2_t{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
      }
      float x = (v[0] + v[1]) + (v[2] + v[3]);
      x += __shfl_xor(x, 16, kWave);  // lanes l, l + 16, l + 32, l + 48 hold the four quads of row li
      x += __shfl_xor(x, 32, kWave);
      if (ok && lg == 0) sb.dgp[(int64_t)((n0 >> 6) + wr) * sb.rows + r] = x;
      if (b + 2 < BB) load_dhp(b + 2, pvs[b & 1]);
    }
  } else if constexpr (SWIGLU && sizeof(OutT) == 4) {
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
          for (int q = 0; q < 4; ++q) hv[q] = silu_f(acc[a][b][q]) * v[q];
          const int64_t oh = HPK ? hpk_off(wt + 4 * b, n0 + (wr * (AB / 2) + a) * 16 + 4 * lg) : o;
          *reinterpret_cast<u32x2_t*>(hout + oh) = u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
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
        for (int q = 0; q < 4; ++q) v[q] = silu_f(acc[a][b][q]) * acc[a + AB / 2][b][q];
        *reinterpret_cast<u32x2_t*>(out + (HPK ? hpk_off(wt + 4 * b, f) : (int64_t)(r0 + tr) * N + f)) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  } else {
#pragma unroll
    for (int a = 0; a < AB; ++a)
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const int tr = (wt + 4 * b) * 16 + li;
        if (tr >= nrows) continue;
        // packed transposed weights: block a holds columns 64 (a/4) + 32 h + 8 (a%4) + 0..7 of the wavefront's
        const int n = kTrPk ? n0 + wr * 128 + 64 * (a / 4) + 32 * (lg / 2) + 8 * (a % 4) + 4 * (lg % 2)
                            : n0 + (wr * AB + a) * 16 + 4 * lg;
        const int m = r0 + tr;
        // WGRAD, PACKED: fragment-packed order (16 m rows x 32 n columns per fragment)
        const int64_t o = (WGRAD && PACKED) ? ((int64_t)(m >> 4) * (N >> 5) + (n >> 5)) * 512 + ((n & 31) >> 3) * 128 +
                                                  (m & 15) * 8 + (n & 7)
                                            : (int64_t)m * N + n;
        store16(out + o, u32x4_t{__float_as_uint(acc[a][b][0]), __float_as_uint(acc[a][b][1]),
                                 __float_as_uint(acc[a][b][2]), __float_as_uint(acc[a][b][3])});
      }
  }
}

template <int BW, int BT, bool PACKED, bool SWIGLU, typename OutT, bool WT = false, bool HPK = false,
          bool SBWD = false>
void launch_tile(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E, const void* wa,
                 const void* wb, void* out, int K, int N, int ksplit, float* part, hipStream_t s,
                 void* hout = nullptr, const SwigluBwdArgs& sb = SwigluBwdArgs{}) {
  constexpr int NW = SWIGLU ? BW / 2 : BW;
  const int64_t max_tiles = ((rows + BT - 1) / BT + E) * (N / NW) * ksplit;
  const int64_t grid = (max_tiles + kXcds - 1) / kXcds * kXcds;
  launch_kernel((tile_gemm_kernel<BW, BT, PACKED, SWIGLU, false, WT, OutT, HPK, SBWD>), dim3((unsigned)grid),
                dim3(512), 0, s, static_cast<const bf16_t*>(act), row_src, offsets, static_cast<const bf16_t*>(wa),
                static_cast<const bf16_t*>(wb), static_cast<OutT*>(out), K, N, E, ksplit, part, rows * N, 0, N,
                static_cast<bf16_t*>(hout), sb);
}

}  // namespace

bool tile_gemm_applies(int dtype, int64_t rows, int E, int d, int F) {
  // bf16 only; large groups; shapes that the 256 x 256 tiles and 64-deep k-steps divide
  return dtype == kBF16 && rows >= 128 * (int64_t)E && F % 128 == 0 && d % 256 == 0 && F % 64 == 0;
}

int tile_down_ksplit(int dtype, int64_t rows, int E, int d, int F) {
  if (!tile_gemm_applies(dtype, rows, E, d, F)) return 1;
  // Expected tiles of the down projection (a group of n rows takes ceil(n/320) token tiles),
  // spread over 256 CUs in rounds of one tile per CU. A split into ks k-ranges turns
  // each round into 1/ks of a round; every extra range costs one more fp32 partial written and
  // read back (8*rows*d bytes at ~6.5 TB/s), expressed in tile times (a 256 x 256 x F tile at
  // ~4 TFLOP/s per CU), plus a fixed 0.2 tile times (the fill and drain of each range's k-loop
  // and output; fitted to step times measured with the split forced to 1..4 on 256-row token
  // tiles: prefill T = 4096 was fastest at 2, the skewed T = 16384 layer at 1, the T = 2048 stack
  // within 0.5% at 2..4). With 320-row tiles the prefill and T = 2048 shapes fill whole rounds and
  // take no split.
  // The split depends on the sizes only, so the workspace size does too.
  const double per_e = (double)rows / E;
  const double tiles = (double)E * std::ceil(per_e / kBT) * (d / 256);
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
                       float* out, hipStream_t s, bool packed_out) {
  const int64_t tiles = (int64_t)E * (M / 256) * (N / 256);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  auto go = [&](auto kernel) {
    launch_kernel(kernel, dim3((unsigned)grid), dim3(512), 0, s, static_cast<const bf16_t*>(p),
                  static_cast<const int32_t*>(nullptr), offsets, static_cast<const bf16_t*>(q),
                  static_cast<const bf16_t*>(nullptr), out, ldp, N, E, 1, static_cast<float*>(nullptr), (int64_t)0, M,
                  ldq, static_cast<bf16_t*>(nullptr), SwigluBwdArgs{});
  };
  if (packed_out)
    go(tile_gemm_kernel<256, 256, true, false, true, true, float>);
  else
    go(tile_gemm_kernel<256, 256, false, false, true, true, float>);
}

void launch_tile_up(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int d,
                    int F, int E, const void* w1, const void* w3, void* h, hipStream_t s, bool hpk) {
  if (layout == kPacked && hpk)
    launch_tile<256, kBT, true, true, bf16_t, false, true>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr, s);
  else if (layout == kPacked)
    launch_tile<256, kBT, true, true, bf16_t>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr, s);
  else if (hpk)
    launch_tile<256, kBT, false, true, bf16_t, false, true>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr,
                                                            s);
  else
    launch_tile<256, kBT, false, true, bf16_t>(act, row_src, offsets, rows, E, w1, w3, h, d, F, 1, nullptr, s);
}

void launch_tile_up_pair(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                         int d, int F, int E, const void* w1, const void* w3, float* a, float* b, hipStream_t s,
                         void* h, bool hpk) {
  if (layout == kPacked && hpk)
    launch_tile<256, kBT, true, true, float, false, true>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
  else if (layout == kPacked)
    launch_tile<256, kBT, true, true, float>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
  else if (hpk)
    launch_tile<256, kBT, false, true, float, false, true>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
  else
    launch_tile<256, kBT, false, true, float>(act, row_src, offsets, rows, E, w1, w3, a, d, F, 1, b, s, h);
}

void launch_tile_up_pair_bwd(int layout, const void* act, const int32_t* row_token, const int32_t* offsets,
                             int64_t rows, int d, int F, int E, const void* w1, const void* w3, const float* dhp,
                             const float* row_g, void* h, void* dab, float* dgp, void* sink, hipStream_t s) {
  SwigluBwdArgs sb;
  sb.dhp = dhp;
  sb.row_g = row_g;
  sb.rows = rows;
  sb.dab = static_cast<bf16_t*>(dab);
  sb.dgp = dgp;
  sb.sink = sink;
  if (layout == kPacked)
    launch_tile<256, kBT, true, true, bf16_t, false, false, true>(act, row_token, offsets, rows, E, w1, w3, h, d, F, 1,
                                                                  nullptr, s, nullptr, sb);
  else
    launch_tile<256, kBT, false, true, bf16_t, false, false, true>(act, row_token, offsets, rows, E, w1, w3, h, d, F, 1,
                                                                   nullptr, s, nullptr, sb);
}

void launch_tile_wt(int layout, const void* act, const int32_t* offsets, int64_t rows, int N, int K, int E,
                    const void* wa, const void* wb, float* out, int ksplit, float* part, hipStream_t s) {
  if (layout == kPacked)
    launch_tile<256, kBT, true, false, float, true>(act, nullptr, offsets, rows, E, wa, wb, out, K, N, ksplit, part, s);
  else
    launch_tile<256, kBT, false, false, float, true>(act, nullptr, offsets, rows, E, wa, wb, out, K, N, ksplit, part,
                                                        s);
}

void launch_tile_down(int layout, const void* h, const int32_t* offsets, int64_t rows, int d, int F, int E,
                      const void* w2, float* y_perm, int ksplit, float* y_part, hipStream_t s, bool hpk) {
  if (layout == kPacked && hpk)
    launch_tile<256, kBT, true, false, float, false, true>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d,
                                                           ksplit, y_part, s);
  else if (layout == kPacked)
    launch_tile<256, kBT, true, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, ksplit,
                                                y_part, s);
  else if (hpk)
    launch_tile<256, kBT, false, false, float, false, true>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d,
                                                            ksplit, y_part, s);
  else
    launch_tile<256, kBT, false, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, ksplit,
                                                 y_part, s);
}

}  // namespace moe
