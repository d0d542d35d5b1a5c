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
//  - a lane reads 16*LPC contiguous bytes of one weight row per step; the k values a lane
//    feeds to successive MFMAs are a fixed permutation of the true k order, the same for A and
//    B, so the contraction is unchanged;
//  - the 4 wavefronts of a workgroup split K and their partial sums are added in LDS in a
//    fixed order (wave 0 + 1 + 2 + 3), so results are reproducible bit for bit;
//  - the grid is (N/16) x (worst-case number of row tiles); a workgroup maps its tile index to
//    an expert from `offsets` on the device and exits if it has none (no host readback).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

template <typename T, int LPC, int NTB>
struct Frag {
  u32x4_t a[LPC];
  u32x4_t b[LPC];
  u32x4_t x[NTB][LPC];
};

template <typename T, int LPC, int NTB, bool SWIGLU, typename OutT>
__global__ __launch_bounds__(256) void stream_gemm_kernel(const T* __restrict__ act,
                                                          const int32_t* __restrict__ row_src,
                                                          const int32_t* __restrict__ offsets,
                                                          const T* __restrict__ wa, const T* __restrict__ wb,
                                                          OutT* __restrict__ out, int K, int N, int E) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte access
  constexpr int CKG = LPC * V;       // contiguous k per lane group per step
  constexpr int CK = 4 * CKG;        // k per step
  constexpr int TILE = 16 * NTB;
  constexpr int NWAVES = 4;

  __shared__ f32x4_t red[NWAVES - 1][SWIGLU ? 2 : 1][NTB][kWave];

  const int lane = threadIdx.x & 63, wave = threadIdx.x / kWave;
  int e, r0, nrows;
  if (!find_tile(offsets, E, TILE, blockIdx.y, e, r0, nrows)) return;
  const int n0 = blockIdx.x * 16;
  const int li = lane & 15, lg = lane >> 4;

  const T* pa = wa + ((int64_t)e * N + n0 + li) * K + lg * CKG;
  const T* pb = SWIGLU ? wb + ((int64_t)e * N + n0 + li) * K + lg * CKG : nullptr;
  const T* px[NTB];
  bool vx[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int rr = tb * 16 + li;
    vx[tb] = rr < nrows;
    const int r = r0 + (vx[tb] ? rr : 0);
    const int src = row_src ? row_src[r] : r;
    px[tb] = act + (int64_t)src * K + lg * CKG;
  }

  const int nsteps = K / CK;
  const int c_lo = wave * nsteps / NWAVES, c_hi = (wave + 1) * nsteps / NWAVES;

  f32x4_t accA[NTB], accB[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    accA[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accB[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto load = [&](Frag<T, LPC, NTB>& f, int c) {
    const int64_t ko = (int64_t)c * CK;
#pragma unroll
    for (int j = 0; j < LPC; ++j) {
      f.a[j] = load16(pa + ko + j * V);
      if constexpr (SWIGLU) f.b[j] = load16(pb + ko + j * V);
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int j = 0; j < LPC; ++j)
        f.x[tb][j] = vx[tb] ? load16(px[tb] + ko + j * V) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto compute = [&](const Frag<T, LPC, NTB>& f) {
#pragma unroll
    for (int j = 0; j < LPC; ++j)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        if constexpr (sizeof(T) == 2) {
          accA[tb] = mfma_bf16(f.a[j], f.x[tb][j], accA[tb]);
          if constexpr (SWIGLU) accB[tb] = mfma_bf16(f.b[j], f.x[tb][j], accB[tb]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xq = __uint_as_float(f.x[tb][j][q]);
            accA[tb] = mfma_f32(__uint_as_float(f.a[j][q]), xq, accA[tb]);
            if constexpr (SWIGLU) accB[tb] = mfma_f32(__uint_as_float(f.b[j][q]), xq, accB[tb]);
          }
        }
      }
  };

  if (c_lo < c_hi) {
    Frag<T, LPC, NTB> cur, nxt;
    load(cur, c_lo);
    for (int c = c_lo; c + 1 < c_hi; ++c) {
      load(nxt, c + 1);
      compute(cur);
      cur = nxt;
    }
    compute(cur);
  }

  if (wave > 0) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      red[wave - 1][0][tb][lane] = accA[tb];
      if constexpr (SWIGLU) red[wave - 1][1][tb][lane] = accB[tb];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < NWAVES - 1; ++w)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      accA[tb] += red[w][0][tb][lane];
      if constexpr (SWIGLU) accB[tb] += red[w][1][tb][lane];
    }

#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int rr = tb * 16 + li;
    if (rr >= nrows) continue;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = SWIGLU ? silu(accA[tb][q]) * accB[tb][q] : accA[tb][q];
    OutT* o = out + (int64_t)(r0 + rr) * N + n0 + 4 * lg;
    if constexpr (sizeof(OutT) == 2) {
      *reinterpret_cast<u32x2_t*>(o) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
      store16(o, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])});
    }
  }
}

template <typename T, int LPC, int NTB, bool SWIGLU, typename OutT>
void launch_stream(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E,
                   const void* wa, const void* wb, void* out, int K, int N, hipStream_t s) {
  constexpr int TILE = 16 * NTB;
  const int64_t max_tiles = (rows + TILE - 1) / TILE + E;
  dim3 grid((unsigned)(N / 16), (unsigned)max_tiles);
  hipLaunchKernelGGL((stream_gemm_kernel<T, LPC, NTB, SWIGLU, OutT>), grid, dim3(256), 0, s,
                     static_cast<const T*>(act), row_src, offsets, static_cast<const T*>(wa),
                     static_cast<const T*>(wb), static_cast<OutT*>(out), K, N, E);
}

template <typename T, bool SWIGLU, typename OutT>
void launch_stream_k(const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int E,
                     const void* wa, const void* wb, void* out, int K, int N, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  if (K % (16 * V) == 0)
    launch_stream<T, 4, 2, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
  else
    launch_stream<T, 2, 2, SWIGLU, OutT>(act, row_src, offsets, rows, E, wa, wb, out, K, N, s);
}

}  // namespace

void launch_expert_ffn(int dtype, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                       int d, int F, int E, const void* w1, const void* w3, const void* w2, void* h, float* y_perm,
                       hipStream_t stream) {
  if (dtype == kBF16) {
    launch_stream_k<bf16_t, true, bf16_t>(act, row_src, offsets, rows, E, w1, w3, h, d, F, stream);
    launch_stream_k<bf16_t, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, stream);
  } else {
    launch_stream_k<float, true, float>(act, row_src, offsets, rows, E, w1, w3, h, d, F, stream);
    launch_stream_k<float, false, float>(h, nullptr, offsets, rows, E, w2, nullptr, y_perm, F, d, stream);
  }
}

}  // namespace moe
