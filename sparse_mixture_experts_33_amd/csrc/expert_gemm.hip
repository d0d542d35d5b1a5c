// Grouped expert FFN: for the rows [offsets[e], offsets[e+1]) of each expert e,
//   H = silu(X W1_e^T) * (X W3_e^T)      (stored in the input dtype)
//   Y = H W2_e^T                          (fp32)
// SwiGLU expert with hidden size F (xyznot.com summary, "Método" and "Términos clave"); only
// the selected experts' rows exist, so an expert with no tokens costs nothing (ja.news.hada.io
// summary: a zero-gate expert need not be computed).
//
// This file holds the "streaming" grouped GEMM, built for groups of a few dozen rows (decode),
// where the expert weights dominate the traffic and each weight byte must be read exactly once:
//  - the matrix-core operand A is the weight (16 rows of W per MFMA), B is the token tile
//    (16 or 32 rows), both read straight from global memory into registers: no LDS staging,
//    since nothing is reused inside a workgroup;
//  - one load instruction covers 64 contiguous bytes of each of its 16 weight rows (4 lanes
//    per row, 16 bytes each); the k values a lane feeds to successive MFMAs are therefore a
//    fixed permutation of the true k order, the same for A and B, so the contraction is
//    unchanged; weights use non-temporal loads (read once);
//  - the 4 wavefronts of a workgroup split K, taking every fourth k-step each (so together they
//    stream one contiguous run of each weight row block), and their partial sums are added in
//    LDS in a fixed order (wave 0 + 1 + 2 + 3), so results are reproducible bit for bit;
//  - the grid is persistent (as many workgroups as fit on the device at once); each workgroup
//    walks items (row tile, 16 rows of W) with a stride of the grid size, mapping tiles to
//    experts from `offsets` on the device (no host readback), so no workgroup waits in a
//    start-up round behind the others.
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace moe {
namespace {


__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

template <typename T, int LPC, int NTB, int RB>
struct Frag {
  u32x4_t a[RB][LPC];
  u32x4_t b[RB][LPC];
  u32x4_t x[NTB][LPC];
};

// RB: 16-row blocks of W per wavefront (the token fragment is reused RB times per load).
// DEPTH: register buffers in the K pipeline (DEPTH-1 steps of loads in flight ahead of the MFMAs).
// PACKED: W in the fragment-packed layout (1 KB contiguous per load instruction) or row-major.
template <typename T, int LPC, int NTB, int RB, int DEPTH, bool PACKED, bool SWIGLU, typename OutT>
__global__ __launch_bounds__(256) void stream_gemm_kernel(const T* __restrict__ act,
                                                          const int32_t* __restrict__ row_src,
                                                          const int32_t* __restrict__ offsets,
                                                          const T* __restrict__ wa, const T* __restrict__ wb,
                                                          OutT* __restrict__ out, int K, int N, int E) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte access
  constexpr int CKG = LPC * V;       // k per lane group per step
  constexpr int CK = 4 * CKG;        // k per step
  constexpr int TILE = 16 * NTB;
  constexpr int NWAVES = 4;
  static_assert(DEPTH == 2 || DEPTH == 3, "pipeline depth");

  __shared__ f32x4_t red[NWAVES - 1][SWIGLU ? 2 : 1][RB][NTB][kWave];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_tile0[kMaxExperts + 1];  // first tile index of each expert

  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) so that the K loop below is a scalar loop the compiler can pipeline
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;

  // group offsets and the tile numbering, once per workgroup
  if (threadIdx.x <= E) s_off[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      s_tile0[e] = acc;
      acc += (s_off[e + 1] - s_off[e] + TILE - 1) / TILE;
    }
    s_tile0[E] = acc;
  }
  __syncthreads();
  const int ntiles = s_tile0[E];
  const int NG = N / (16 * RB);
  const int nsteps = K / CK;
  // wavefront w takes the k-steps w, w + 4, w + 8, ... (its i-th is step w + 4 i): the four
  // wavefronts' loads of one round are then four consecutive steps, one contiguous run per weight
  // row block, which streams from HBM faster than four runs a quarter of K apart
  const int c_lo = 0, c_hi = (nsteps - wave + NWAVES - 1) / NWAVES;

  // Persistent loop over items (tile, 16*RB rows of W); consecutive workgroups take
  // consecutive row groups of the same tile, so the tile's token rows stay hot in L2.
  for (int item = blockIdx.x; item < ntiles * NG; item += gridDim.x) {
    const int tile = item / NG;
    const int n0 = (item - tile * NG) * 16 * RB;
    int e = 0;
    while (tile >= s_tile0[e + 1]) ++e;
    const int r0 = s_off[e] + (tile - s_tile0[e]) * TILE;
    const int nrows = min(TILE, s_off[e + 1] - r0);

    // Access j of step c is fragment q = c*LPC + j: lane l holds row l%16 and the V values at
    // k = 4V*q + V*(l/16). Row-major W: one load instruction covers 64 contiguous bytes of each of
    // the 16 rows. Packed W: the fragment is 1 KB contiguous in lane order.
    const T* pa[RB];
    const T* pb[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t row0 = (int64_t)e * N + n0 + rb * 16;
      const int64_t off = PACKED ? row0 * K + lane * V : (row0 + li) * K + lg * V;
      pa[rb] = wa + off;
      pb[rb] = SWIGLU ? wb + off : nullptr;
    }
    constexpr int64_t kFragStride = PACKED ? 64 * V : 4 * V;  // elements between fragments q, q+1
    // Token rows past the end of the group load the group's first row instead: output column j
    // of an MFMA depends only on token column j, and those columns are never stored. Keeping the
    // loads unconditional lets the compiler count them and overlap the next step's loads with
    // this step's MFMAs.
    const T* px[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const int rr = tb * 16 + li;
      const int r = r0 + (rr < nrows ? rr : 0);
      const int src = row_src ? row_src[r] : r;
      px[tb] = act + (int64_t)src * K + lg * V;
    }

    f32x4_t accA[RB][NTB], accB[RB][NTB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        accA[rb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accB[rb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

    using FragT = Frag<T, LPC, NTB, RB>;
    auto load = [&](FragT& f, int i) {
      const int c = wave + NWAVES * i;  // the k-step
      const int64_t ko = (int64_t)c * CK;
      // weights are read exactly once: non-temporal loads keep them from evicting the token rows
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < LPC; ++j) {
          const int64_t fo = (int64_t)(c * LPC + j) * kFragStride;
          f.a[rb][j] = load16_nt(pa[rb] + fo);
          if constexpr (SWIGLU) f.b[rb][j] = load16_nt(pb[rb] + fo);
        }
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int j = 0; j < LPC; ++j) f.x[tb][j] = load16(px[tb] + ko + j * 4 * V);
    };
    auto compute = [&](const FragT& f) {
#pragma unroll
      for (int j = 0; j < LPC; ++j)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            if constexpr (sizeof(T) == 2) {
              accA[rb][tb] = mfma_bf16(f.a[rb][j], f.x[tb][j], accA[rb][tb]);
              if constexpr (SWIGLU) accB[rb][tb] = mfma_bf16(f.b[rb][j], f.x[tb][j], accB[rb][tb]);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float xq = __uint_as_float(f.x[tb][j][q]);
                accA[rb][tb] = mfma_f32(__uint_as_float(f.a[rb][j][q]), xq, accA[rb][tb]);
                if constexpr (SWIGLU) accB[rb][tb] = mfma_f32(__uint_as_float(f.b[rb][j][q]), xq, accB[rb][tb]);
              }
            }
          }
    };

    // Register buffers used in rotation and unrolled by DEPTH: the loads of the next DEPTH-1
    // steps are in flight while the MFMAs of the current step run.
    if (c_lo < c_hi) {
      if constexpr (DEPTH == 2) {
        FragT A, B;
        load(A, c_lo);
        int c = c_lo;
        for (; c + 2 <= c_hi; c += 2) {
          load(B, c + 1);
          compute(A);
          if (c + 2 < c_hi) load(A, c + 2);
          compute(B);
        }
        if (c < c_hi) compute(A);
      } else {
        FragT A, B, C;
        load(A, c_lo);
        if (c_lo + 1 < c_hi) load(B, c_lo + 1);
        int c = c_lo;
        for (; c + 3 <= c_hi; c += 3) {
          load(C, c + 2);
          compute(A);
          if (c + 3 < c_hi) load(A, c + 3);
          compute(B);
          if (c + 4 < c_hi) load(B, c + 4);
          compute(C);
        }
        if (c < c_hi) compute(A);
        if (c + 1 < c_hi) compute(B);
      }
    }

    // the 4 partial sums are added in a fixed order: wave 0 + 1 + 2 + 3
    if (wave > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          red[wave - 1][0][rb][tb][lane] = accA[rb][tb];
          if constexpr (SWIGLU) red[wave - 1][1][rb][tb][lane] = accB[rb][tb];
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NWAVES - 1; ++w)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) {
            accA[rb][tb] += red[w][0][rb][tb][lane];
            if constexpr (SWIGLU) accB[rb][tb] += red[w][1][rb][tb][lane];
          }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const int rr = tb * 16 + li;
          if (rr >= nrows) continue;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q] = SWIGLU ? silu(accA[rb][tb][q]) * accB[rb][tb][q] : accA[rb][tb][q];
          OutT* o = out + (int64_t)(r0 + rr) * N + n0 + rb * 16 + 4 * lg;
          if constexpr (sizeof(OutT) == 2) {
            *reinterpret_cast<u32x2_t*>(o) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
            store16(o, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                               __float_as_uint(v[3])});
          }
        }
    }
    __syncthreads();  // red[] is rewritten by the next item
  }
}

// Workgroups of `kernel` that fit on the current device at once (cached per kernel and device).
template <typename Kern>
int resident_blocks(Kern kernel, int threads) {
  struct Entry {
    const void* fn;
    int dev, blocks;
  };
  static thread_local Entry cache[64];
  static thread_local int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  const void* fn = reinterpret_cast<const void*>(kernel);
  for (int i = 0; i < n; ++i)
    if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].blocks;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int blocks = cus * per_cu;
  if (n < 64) cache[n++] = Entry{fn, dev, blocks};
  return blocks;
}

template <typename T, int LPC, int NTB, int RB, bool PACKED, bool SWIGLU, typename OutT>
void launch_stream(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E,
                   const void* wa, const void* wb, void* out, int K, int N, hipStream_t s) {
  constexpr int TILE = 16 * NTB;
  auto kernel = stream_gemm_kernel<T, LPC, NTB, RB, 2, PACKED, SWIGLU, OutT>;
  const int64_t max_tiles = (rows + TILE - 1) / TILE + E;
  const int64_t max_items = max_tiles * (N / (16 * RB));
  const int blocks = (int)std::min<int64_t>(max_items, resident_blocks(kernel, 256));
  launch_kernel(kernel, dim3(blocks), dim3(256), 0, s, static_cast<const T*>(act), row_src, offsets,
                     static_cast<const T*>(wa), static_cast<const T*>(wb), static_cast<OutT*>(out), K, N, E);
}

// Shape choice (all choices are correct for any routing):
//  - 16-row token tiles when groups are expected to be small (T*K/E <= 12), else 32 rows;
//  - the down projection (one weight matrix) works on 32 weight rows per wavefront so that a
//    token fragment serves two weight fragments, as in the up projection (w1 and w3);
//  - LPC = 4 fragments per step when K allows it, else 2.
template <typename T, bool PACKED, bool SWIGLU, typename OutT>
void launch_stream_k(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E,
                     const void* wa, const void* wb, void* out, int K, int N, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  constexpr int RB = SWIGLU ? 1 : 2;
  const bool small = rows <= 12 * (int64_t)E;
  const bool rb_ok = N % (16 * RB) == 0;
  if (K % (16 * V) == 0 && rb_ok) {
    if (small) launch_stream<T, 4, 1, RB, PACKED, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
    else launch_stream<T, 4, 2, RB, PACKED, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
  } else {
    if (small) launch_stream<T, 2, 1, 1, PACKED, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
    else launch_stream<T, 2, 2, 1, PACKED, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
  }
}

template <typename T, bool SWIGLU, typename OutT>
void launch_stream_l(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                     int E, const void* wa, const void* wb, void* out, int K, int N, hipStream_t s) {
  if (layout == kPacked)
    launch_stream_k<T, true, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
  else
    launch_stream_k<T, false, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
}

}  // namespace

void launch_expert_up(int dtype, int layout, const void* act, const int32_t* row_src, const int32_t* offsets,
                      int64_t rows, int d, int F, int E, const void* w1, const void* w3, void* h, hipStream_t stream,
                      bool hpk) {
  if (tile_gemm_applies(dtype, rows, E, d, F))
    launch_tile_up(layout, act, row_src, offsets, rows, d, F, E, w1, w3, h, stream, hpk);
  else if (dtype == kBF16)
    launch_stream_l<bf16_t, true, bf16_t>(layout, act, row_src, offsets, rows, E, w1, w3, h, d, F, stream);
  else
    launch_stream_l<float, true, float>(layout, act, row_src, offsets, rows, E, w1, w3, h, d, F, stream);
}

void launch_expert_down(int dtype, int layout, const void* h, const int32_t* offsets, int64_t rows, int d, int F,
                        int E, const void* w2, float* y_perm, int ksplit, float* y_part, hipStream_t stream,
                        bool hpk) {
  if (tile_gemm_applies(dtype, rows, E, d, F))
    launch_tile_down(layout, h, offsets, rows, d, F, E, w2, y_perm, ksplit, y_part, stream, hpk);
  else if (dtype == kBF16)
    launch_stream_l<bf16_t, false, float>(layout, h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, stream);
  else
    launch_stream_l<float, false, float>(layout, h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, stream);
}

}  // namespace moe
