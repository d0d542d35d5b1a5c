// Router: logits = x . W_g (+ bias), TopK (the rest set to -inf), softmax over the kept logits.
// Definitions: blog.csdn.net explainer of "Mixtral of Experts", sections 2.1-2.3; xyznot.com
// summary, "Método" (n = 8, K = 2).
//
// Bandwidth kernel: it reads x once (T*d elements) and W_g (d*E elements, shared by every
// token: staged in LDS once per workgroup for bf16 with E = 8, else served from L2). One
// wavefront owns a token at a time; each lane covers 16-byte slices of d and accumulates E
// partial sums per token in fp32. Decode batches take one workgroup per token instead. A butterfly over the 64 lanes gives
// every lane the full logits; TopK is then repeated argmax over registers (ties -> lower
// index) and the softmax uses only the K kept logits, so the other experts get exactly 0.
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace moe {
namespace {

template <typename T, int V>
__device__ inline void unpack16(u32x4_t r, float (&v)[V]);

template <>
__device__ inline void unpack16<bf16_t, 8>(u32x4_t r, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(r[i]);
    v[2 * i + 1] = bf16_hi(r[i]);
  }
}
template <>
__device__ inline void unpack16<float, 4>(u32x4_t r, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
}

// W_g row k (E contiguous values) as fp32. Vector path when E == 8.
template <typename T, int EMAX>
__device__ inline void load_gate_row(const T* row, int E, float (&w)[EMAX]) {
  if constexpr (EMAX == 8) {
    if (E == 8) {
      if constexpr (sizeof(T) == 2) {
        float t[8];
        unpack16<bf16_t, 8>(load16(row), t);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = t[e];
      } else {
        float t0[4], t1[4];
        unpack16<float, 4>(load16(row), t0);
        unpack16<float, 4>(load16(row + 4), t1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = t0[e];
          w[e + 4] = t1[e];
        }
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) w[e] = (e < E) ? Elem<T>::to_f32(row[e]) : 0.0f;
}

template <int EMAX>
__device__ inline void finalize_token(const float (&acc)[EMAX], int64_t t, int E, int K, const float* bias,
                                      int32_t* topk_idx, float* topk_w, float* logits) {
  float l[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) l[e] = (e < E) ? acc[e] + (bias ? bias[e] : 0.0f) : 0.0f;
  if (logits) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) logits[t * E + e] = l[e];
  }
  uint64_t taken = 0;
  int sel[kMaxTopK];
  float sv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel[j] = 0;
    sv[j] = 0.0f;
    if (j < K) {
      int best = -1;
      float bv = 0.0f;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e < E && !((taken >> e) & 1ull) && (best < 0 || l[e] > bv)) {
          best = e;
          bv = l[e];
        }
      }
      taken |= 1ull << best;
      sel[j] = best;
      sv[j] = bv;
    }
  }
  // softmax over the kept logits, shifted by the largest (slot 0)
  float ex[kMaxTopK];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ex[j] = (j < K) ? expf(sv[j] - sv[0]) : 0.0f;
    s += ex[j];
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < K) {
      topk_idx[t * K + j] = sel[j];
      topk_w[t * K + j] = ex[j] / s;
    }
  }
}

template <typename T, int EMAX, int TPW>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                    const float* __restrict__ bias, int64_t ntok, int d, int E,
                                                    int K, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w, float* __restrict__ logits) {
  constexpr int V = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave)) * TPW;
  if (t0 >= ntok) return;

  float acc[TPW][EMAX];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[tt][e] = 0.0f;

  for (int k0 = lane * V; k0 < d; k0 += kWave * V) {
    float xv[TPW][V];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      if (t0 + tt < ntok) {
        unpack16<T, V>(load16(x + (t0 + tt) * d + k0), xv[tt]);
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) xv[tt][j] = 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float w[EMAX];
      load_gate_row<T, EMAX>(wg + (int64_t)(k0 + j) * E, E, w);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[tt][e] = fmaf(xv[tt][j], w[e], acc[tt][e]);
    }
  }

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) acc[tt][e] = wave_sum(acc[tt][e]);

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
    if (lane == tt && t0 + tt < ntok) finalize_token<EMAX>(acc[tt], t0 + tt, E, K, bias, topk_idx, topk_w, logits);
}

// Many tokens, bf16, E = 8, d <= 4096: W_g (d rows of 16 bytes) is staged in LDS once per
// workgroup and each wavefront then takes tokens in turn, so W_g is read from L2 once per
// workgroup rather than once per token. Row r sits at slot (r % 8) * (d / 8) + r / 8: the 64
// lanes, reading rows 8 l + j of their 16-byte x slices, hit consecutive slots. The accumulation
// order is that of route_kernel (lane slices k0 = 8 l + 512 i, j ascending, then the butterfly),
// so the logits are bit-identical to it.
constexpr int kRouteLdsMaxD = 4096;
__global__ __launch_bounds__(256) void route_lds_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                        const float* __restrict__ bias, int64_t ntok, int d, int K,
                                                        int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                        float* __restrict__ logits) {
  __shared__ u32x4_t wl[kRouteLdsMaxD];
  const int d8 = d / 8;
  {
    // all of a thread's W_g loads in flight together (a loop that stores each load before the
    // next one is issued waits out one L2 round trip per row slice)
    constexpr int kPer = kRouteLdsMaxD / 256;
    u32x4_t tmp[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = threadIdx.x + 256 * i;
      if (r < d) tmp[i] = load16(wg + (int64_t)r * 8);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = threadIdx.x + 256 * i;
      if (r < d) wl[(r & 7) * d8 + (r >> 3)] = tmp[i];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; t < ntok; t += waves) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll 8
    for (int k0 = lane * 8; k0 < d; k0 += kWave * 8) {
      float xv[8];
      unpack16<bf16_t, 8>(load16(x + t * d + k0), xv);
      const int r0 = k0 >> 3;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float w[8];
        unpack16<bf16_t, 8>(wl[j * d8 + r0], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(xv[j], w[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wave_sum(acc[e]);
    if (lane == 0) finalize_token<8>(acc, t, 8, K, bias, topk_idx, topk_w, logits);
  }
}

// Few tokens (decode): one workgroup per token, so all loads of a token are in flight at once.
// Each of the 256 threads covers 16-byte slices of d; partial sums are reduced across each wave
// (butterfly) and then across the 4 waves in LDS, in a fixed order.
template <typename T, int EMAX>
__global__ __launch_bounds__(256) void route_token_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                          const float* __restrict__ bias, int64_t ntok, int d,
                                                          int E, int K, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, float* __restrict__ logits) {
  constexpr int V = 16 / sizeof(T);
  __shared__ float part[4][EMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x / kWave;
  const int64_t t = blockIdx.x;
  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0f;
#pragma unroll 4
  for (int k0 = threadIdx.x * V; k0 < d; k0 += 256 * V) {
    float xv[V];
    unpack16<T, V>(load16(x + t * d + k0), xv);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float w[EMAX];
      load_gate_row<T, EMAX>(wg + (int64_t)(k0 + j) * E, E, w);
#pragma unroll
      for (int e = 0; e < EMAX; ++e) acc[e] = fmaf(xv[j], w[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) acc[e] = wave_sum(acc[e]);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) part[wave][e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    finalize_token<EMAX>(acc, t, E, K, bias, topk_idx, topk_w, logits);
  }
}

template <typename T, int EMAX, int TPW>
void launch(const void* x, const void* wg, const float* bias, int64_t T_, int d, int E, int K, int32_t* idx,
            float* w, float* logits, hipStream_t s) {
  const int64_t waves = (T_ + TPW - 1) / TPW;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  launch_kernel((route_kernel<T, EMAX, TPW>), dim3(blocks), dim3(256), 0, s, static_cast<const T*>(x),
                     static_cast<const T*>(wg), bias, T_, d, E, K, idx, w, logits);
}

template <typename T>
void launch_t(const void* x, const void* wg, const float* bias, int64_t T_, int d, int E, int K, int32_t* idx,
              float* w, float* logits, hipStream_t s) {
  if (T_ <= 512 && E <= 8) {
    launch_kernel((route_token_kernel<T, 8>), dim3((unsigned)T_), dim3(256), 0, s, static_cast<const T*>(x),
                       static_cast<const T*>(wg), bias, T_, d, E, K, idx, w, logits);
    return;
  }
  if constexpr (sizeof(T) == 2) {
    if (E == 8 && d <= kRouteLdsMaxD) {
      // two workgroups per CU (64 KB of LDS each), a few tokens per wavefront
      const int64_t blocks = std::min<int64_t>((T_ + 3) / 4, 512);
      launch_kernel(route_lds_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const bf16_t*>(x),
                    static_cast<const bf16_t*>(wg), bias, T_, d, K, idx, w, logits);
      return;
    }
  }
  // one wavefront per token: more wavefronts in flight per CU beat sharing the W_g loads among
  // several tokens (measured at T = 4096: 40 us against 48 us with 4 tokens per wavefront)
  if (E <= 8) {
    launch<T, 8, 1>(x, wg, bias, T_, d, E, K, idx, w, logits, s);
  } else {
    launch<T, 64, 1>(x, wg, bias, T_, d, E, K, idx, w, logits, s);
  }
}

}  // namespace

void launch_route(int dtype, const void* x, const void* w_gate, const float* bias, int64_t T, int d, int E, int K,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream) {
  if (dtype == kBF16)
    launch_t<bf16_t>(x, w_gate, bias, T, d, E, K, topk_idx, topk_w, logits, stream);
  else
    launch_t<float>(x, w_gate, bias, T, d, E, K, topk_idx, topk_w, logits, stream);
}

}  // namespace moe
