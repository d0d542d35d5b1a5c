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

// a.lo * b.lo + a.hi * b.hi + c for two bf16 pairs (low half first), fp32 accumulation. The
// pairs are taken by value: a bit cast of a vector element in place reads the vector's first
// element whatever the index.
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

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

// Many tokens, bf16, E = 8, d <= 4096: W_g is staged in LDS once per workgroup and each wavefront
// then takes tokens in turn, so W_g is read from L2 once per workgroup rather than once per token.
// The products run on the packed bf16 dot instruction (two products and the accumulator per
// instruction, fp32 accumulation), which takes x and W_g as they are, two consecutive k per dword:
// x's 16-byte slices already are, and the staging regroups W_g into pairs of rows, the dword of
// expert e in pair q holding (W_g[2q][e], W_g[2q+1][e]). Experts 0-3 of pair q sit in the 16-byte
// slot (q % 4) * (d / 8) + q / 4 and experts 4-7 d / 2 slots further, so the 64 lanes, each on 8
// consecutive k, read consecutive slots. Against converting every W_g value to fp32 for an fma
// (four times the vector instructions) this takes 16 instead of 27 us at T = 4096. Issuing all eight
// x slices of a token before its products, or also the next token's, measured slower (20 and 22 us).
constexpr int kRouteLdsMaxD = 4096;
template <int TPW>
__global__ __launch_bounds__(256) void route_lds_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                                        const float* __restrict__ bias, int64_t ntok, int d, int K,
                                                        int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                        float* __restrict__ logits) {
  __shared__ u32x4_t wl[kRouteLdsMaxD];
  const int d8 = d / 8, d2 = d / 2;
  {
    // all of a thread's W_g loads in flight together (a loop that stores each load before the
    // next one is issued waits out one L2 round trip per row pair)
    constexpr int kPer = kRouteLdsMaxD / 2 / 256;
    u32x4_t r0[kPer], r1[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q < d2) {
        r0[i] = load16(wg + (int64_t)q * 16);
        r1[i] = load16(wg + (int64_t)q * 16 + 8);
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q < d2) {
        // dword c of a row holds experts 2c (low half) and 2c + 1
        u32x4_t lo, hi;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          lo[2 * c] = (r0[i][c] & 0xFFFFu) | (r1[i][c] << 16);
          lo[2 * c + 1] = (r0[i][c] >> 16) | (r1[i][c] & 0xFFFF0000u);
          hi[2 * c] = (r0[i][c + 2] & 0xFFFFu) | (r1[i][c + 2] << 16);
          hi[2 * c + 1] = (r0[i][c + 2] >> 16) | (r1[i][c + 2] & 0xFFFF0000u);
        }
        const int slot = (q & 3) * d8 + (q >> 2);
        wl[slot] = lo;
        wl[d2 + slot] = hi;
      }
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  // Lane l takes the x slices k0 = 8 l + 512 i of each token. TPW consecutive tokens per pass over W_g, so that each LDS read serves TPW tokens; a token's
  // products keep the order of the single-token pass (tokens past the end compute on the last one
  // and are not stored)
  for (int64_t t0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * TPW; t0 < ntok;
       t0 += waves * TPW) {
    const bf16_t* xr[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) xr[u] = x + (t0 + u < ntok ? t0 + u : ntok - 1) * d;
    float acc[TPW][8];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
#pragma unroll 8
    for (int k0 = lane * 8; k0 < d; k0 += kWave * 8) {
      u32x4_t xv[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) xv[u] = load16(xr[u] + k0);
      const int qb = k0 >> 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t lo = wl[j * d8 + qb], hi = wl[d2 + j * d8 + qb];
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[u][e] = dot2_bf16(xv[u][j], lo[e], acc[u][e]);
            acc[u][e + 4] = dot2_bf16(xv[u][j], hi[e], acc[u][e + 4]);
          }
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = wave_sum(acc[u][e]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        if (t0 + u < ntok) finalize_token<8>(acc[u], t0 + u, 8, K, bias, topk_idx, topk_w, logits);
    }
  }
}

// Few tokens (decode): one workgroup per token, so all loads of a token are in flight at once.
// Each of the 256 threads covers 16-byte slices of d; partial sums are reduced across each wave
// (butterfly) and then across the 4 waves in LDS, in a fixed order. VEC (bf16, E = 8): a W_g row is
// one 16-byte load, and a chunk's slices and rows are all loaded before its products (rows past d
// load a valid row and meet a zeroed x slice, adding exact zeros), so the loads overlap instead of
// each waiting out a memory round trip.
template <typename T, int EMAX, bool VEC>
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
  if constexpr (VEC) {
    static_assert(V == 8 && EMAX == 8, "bf16 rows of 8 experts");
    constexpr int C = 2;  // slices per thread and chunk (d = 4096 is one chunk)
    for (int kc = threadIdx.x * 8; kc < d; kc += 256 * 8 * C) {
      u32x4_t xr[C], wr[C][8];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int k0 = kc + 256 * 8 * c;
        const int ks = k0 < d ? k0 : d - 8;
        xr[c] = load16(x + t * d + ks);
#pragma unroll
        for (int j = 0; j < 8; ++j) wr[c][j] = load16(wg + (int64_t)(ks + j) * 8);
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float xv[8];
        unpack16<bf16_t, 8>(xr[c], xv);
        const bool in = kc + 256 * 8 * c < d;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float w[8];
          unpack16<bf16_t, 8>(wr[c][j], w);
          const float xj = in ? xv[j] : 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(xj, w[e], acc[e]);
        }
      }
    }
  } else {
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
    if (sizeof(T) == 2 && E == 8)
      launch_kernel((route_token_kernel<T, 8, sizeof(T) == 2>), dim3((unsigned)T_), dim3(256), 0, s,
                    static_cast<const T*>(x), static_cast<const T*>(wg), bias, T_, d, E, K, idx, w, logits);
    else
      launch_kernel((route_token_kernel<T, 8, false>), dim3((unsigned)T_), dim3(256), 0, s, static_cast<const T*>(x),
                    static_cast<const T*>(wg), bias, T_, d, E, K, idx, w, logits);
    return;
  }
  if constexpr (sizeof(T) == 2) {
    if (E == 8 && d <= kRouteLdsMaxD) {
      // two workgroups per CU (64 KB of LDS each), a few tokens per wavefront; two or four tokens
      // per pass over W_g once there are enough tokens to fill the grid that way (router alone,
      // us per call at T = 2048 / 4096 / 16384: one token 9.2 / 16.1 / 48.1, two 12.8 / 14.6 / 40.8,
      // four 19.5 / 19.3 / 39.3)
      const int tpw = T_ >= 16384 ? 4 : T_ >= 4096 ? 2 : 1;
      const int64_t blocks = std::min<int64_t>((T_ + 4 * tpw - 1) / (4 * tpw), 512);
      auto go = [&](auto k) {
        launch_kernel(k, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const bf16_t*>(x),
                      static_cast<const bf16_t*>(wg), bias, T_, d, K, idx, w, logits);
      };
      if (tpw == 4) go(route_lds_kernel<4>);
      else if (tpw == 2) go(route_lds_kernel<2>);
      else go(route_lds_kernel<1>);
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
