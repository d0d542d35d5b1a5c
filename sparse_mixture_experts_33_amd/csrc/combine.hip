// Gate-weighted combine back to token order, y = sum_i G(x)_i E_i(x) (blog.csdn.net explainer,
// section 1; xyznot.com summary, "Método"): the expert outputs return to their original token
// positions (zh.newsflash.city article, expert-parallel paragraph) and are added.
//
// One wavefront (or, for few tokens, one workgroup) per token, 16-byte accesses along d. When the
// down projection was split along k, an expert output is first rebuilt as the sum of its k-range
// partials in range order. The K terms are then added in fp32 in slot order, s = w0*o0, then
// s = fma(w_k, o_k, s), so the result does not depend on scheduling.
// HBM-bound: T*K*d*4 bytes read, T*d*|y| written (plus T*d*4 read when accumulating).
//
// Also the RMSNorm of a residual stream for stacks of such layers (the pages describe no norm;
// unit weight): x = bf16(h / sqrt(mean(h^2) + eps)).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// MODE 0: y fp32, 1: y bf16, 2: y fp32 accumulate. TPB tokens per 256-thread block: 4 (one
// wavefront per token) for many tokens, 1 (the whole block on one token, all loads in flight at
// once) for few tokens.
template <int MODE, int TPB>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const float* __restrict__ y_part, int nparts,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w, int64_t T, int d, int K,
                                                      void* __restrict__ y) {
  constexpr int NT = 256 / TPB;  // threads per token
  const int lt = threadIdx.x % NT;
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / NT;
  if (t >= T) return;
  int rows[kMaxTopK];
  float g[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    rows[k] = (k < K) ? token_row[t * K + k] : 0;
    g[k] = (k < K) ? topk_w[t * K + k] : 0.0f;
  }
  const int64_t part_stride = (int64_t)T * K * d;
  // expert output of slot k: y_perm row plus the partial sums of the other k-ranges, in order
  auto expert_out = [&](int k, int c) {
    const int64_t off = (int64_t)rows[k] * d + c;
    f32x4_t o = *reinterpret_cast<const f32x4_t*>(y_perm + off);
    for (int p = 0; p < nparts; ++p) o = o + *reinterpret_cast<const f32x4_t*>(y_part + p * part_stride + off);
    return o;
  };
#pragma unroll 4
  for (int c = lt * 4; c < d; c += NT * 4) {
    f32x4_t s = g[0] * expert_out(0, c);
#pragma unroll
    for (int k = 1; k < kMaxTopK; ++k) {
      if (k < K) {
        const f32x4_t o = expert_out(k, c);
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] = fmaf(g[k], o[q], s[q]);
      }
    }
    if constexpr (MODE == 0) {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + t * d + c) = s;
    } else if constexpr (MODE == 1) {
      *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(y) + t * d + c) =
          u32x2_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    } else {
      f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + t * d + c);
      *p = *p + s;
    }
  }
}

// The same combine for K <= 2 and at most one k-range partial, with the slot count and the partial
// count known at compile time: each thread loads four chunks' expert outputs (and partials, and y
// when accumulating) before any arithmetic, instead of waiting out a memory round trip per chunk as
// the generic loop does (its loads sit behind run-time slot and partial checks). Same arithmetic
// in the same order as combine_kernel, so the results are bit-identical.
template <int MODE, int TPB, int KT, int NP>
__global__ __launch_bounds__(256) void combine_fast_kernel(const float* __restrict__ y_perm,
                                                           const float* __restrict__ y_part,
                                                           const int32_t* __restrict__ token_row,
                                                           const float* __restrict__ topk_w, int64_t T, int d,
                                                           void* __restrict__ y) {
  constexpr int NT = 256 / TPB;  // threads per token
  constexpr int U = 4;           // chunks of 4 columns loaded together
  const int lt = threadIdx.x % NT;
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / NT;
  if (t >= T) return;
  int64_t base[KT];
  float g[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    base[k] = (int64_t)token_row[t * KT + k] * d;
    g[k] = topk_w[t * KT + k];
  }
  for (int c0 = lt * 4; c0 < d; c0 += NT * 4 * U) {
    f32x4_t o[U][KT], pp[U][NP > 0 ? KT : 1], yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + NT * 4 * u;
      const int cc = c < d ? c : c0;  // chunks past d load a valid chunk and are not stored
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        o[u][k] = *reinterpret_cast<const f32x4_t*>(y_perm + base[k] + cc);
        if constexpr (NP > 0) pp[u][k] = *reinterpret_cast<const f32x4_t*>(y_part + base[k] + cc);
      }
      if constexpr (MODE == 2) yv[u] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(y) + t * d + cc);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + NT * 4 * u;
      if (c >= d) continue;
      f32x4_t e0 = o[u][0];
      if constexpr (NP > 0) e0 = e0 + pp[u][0];
      f32x4_t sum = g[0] * e0;
#pragma unroll
      for (int k = 1; k < KT; ++k) {
        f32x4_t ek = o[u][k];
        if constexpr (NP > 0) ek = ek + pp[u][k];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] = fmaf(g[k], ek[q], sum[q]);
      }
      if constexpr (MODE == 0) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + t * d + c) = sum;
      } else if constexpr (MODE == 1) {
        *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(y) + t * d + c) =
            u32x2_t{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
      } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + t * d + c) = yv[u] + sum;
      }
    }
  }
}

template <int MODE>
void launch_mode(const float* y_perm, const float* y_part, int nparts, const int32_t* token_row, const float* topk_w,
                 int64_t T, int d, int K, void* y, hipStream_t stream) {
  if ((K == 1 || K == 2) && nparts <= 1) {
    const unsigned blocks = (unsigned)(T <= 1024 ? T : (T + 3) / 4);
    auto go = [&](auto kernel) {
      launch_kernel(kernel, dim3(blocks), dim3(256), 0, stream, y_perm, y_part, token_row, topk_w, T, d, y);
    };
    if (T <= 1024) {
      if (K == 2)
        nparts ? go(combine_fast_kernel<MODE, 1, 2, 1>) : go(combine_fast_kernel<MODE, 1, 2, 0>);
      else
        nparts ? go(combine_fast_kernel<MODE, 1, 1, 1>) : go(combine_fast_kernel<MODE, 1, 1, 0>);
    } else {
      if (K == 2)
        nparts ? go(combine_fast_kernel<MODE, 4, 2, 1>) : go(combine_fast_kernel<MODE, 4, 2, 0>);
      else
        nparts ? go(combine_fast_kernel<MODE, 4, 1, 1>) : go(combine_fast_kernel<MODE, 4, 1, 0>);
    }
    return;
  }
  if (T <= 1024) {
    launch_kernel((combine_kernel<MODE, 1>), dim3((unsigned)T), dim3(256), 0, stream, y_perm, y_part, nparts,
                       token_row, topk_w, T, d, K, y);
  } else {
    launch_kernel((combine_kernel<MODE, 4>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, y_perm, y_part,
                       nparts, token_row, topk_w, T, d, K, y);
  }
}

// One wavefront per token; rows of up to kNormRegD values are held in registers between the sum
// of squares and the scaling. The sum runs over a lane's slices in ascending order, then the
// butterfly, whatever the path.
constexpr int kNormRegD = 4096;
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int64_t T, int d, float eps,
                                                      bf16_t* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = h + t * d;
  float ss = 0.0f;
  auto sq = [&](const f32x4_t& v) {
    ss = fmaf(v[0], v[0], ss);
    ss = fmaf(v[1], v[1], ss);
    ss = fmaf(v[2], v[2], ss);
    ss = fmaf(v[3], v[3], ss);
  };
  auto put = [&](int c, const f32x4_t& v, float inv) {
    *reinterpret_cast<u32x2_t*>(x + t * d + c) = u32x2_t{pack_bf16x2(v[0] * inv, v[1] * inv),
                                                         pack_bf16x2(v[2] * inv, v[3] * inv)};
  };
  if (d <= kNormRegD) {
    // the row in registers: one read of h, all of a lane's loads in flight together
    constexpr int kPer = kNormRegD / (kWave * 4);
    f32x4_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * 4 + kWave * 4 * i;
      v[i] = c < d ? *reinterpret_cast<const f32x4_t*>(row + c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane * 4 + kWave * 4 * i < d) sq(v[i]);
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * 4 + kWave * 4 * i;
      if (c < d) put(c, v[i], inv);
    }
    return;
  }
  for (int c = lane * 4; c < d; c += kWave * 4) sq(*reinterpret_cast<const f32x4_t*>(row + c));
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane * 4; c < d; c += kWave * 4) put(c, *reinterpret_cast<const f32x4_t*>(row + c), inv);
}

}  // namespace

void launch_combine(const float* y_perm, const float* y_part, int nparts, const int32_t* token_row, const float* topk_w,
                    int64_t T, int d, int K, int y_dtype, int accumulate, void* y, hipStream_t stream) {
  if (accumulate)
    launch_mode<2>(y_perm, y_part, nparts, token_row, topk_w, T, d, K, y, stream);
  else if (y_dtype == kBF16)
    launch_mode<1>(y_perm, y_part, nparts, token_row, topk_w, T, d, K, y, stream);
  else
    launch_mode<0>(y_perm, y_part, nparts, token_row, topk_w, T, d, K, y, stream);
}

void launch_rmsnorm(const float* h, int64_t T, int d, float eps, void* x_bf16, hipStream_t stream) {
  const unsigned blocks = (unsigned)((T + 3) / 4);
  launch_kernel(rmsnorm_kernel, dim3(blocks), dim3(256), 0, stream, h, T, d, eps, static_cast<bf16_t*>(x_bf16));
}

}  // namespace moe
