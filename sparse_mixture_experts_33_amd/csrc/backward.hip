// Backward pass of the mixture-of-experts layer: the elementwise, gather and reduction kernels
// around the grouped GEMMs. The pages define only the forward layer (logits x.W_g, TopK, softmax
// over the kept logits, y = sum_k g_k E_k(x) with SwiGLU experts: blog.csdn.net explainer,
// sections 1 and 2.1-2.4; xyznot.com summary, "Método"); its gradient follows by the chain rule
// with the TopK selection held fixed. For a row r = (token t, slot k) of expert e, gate g_k:
//   dh'_r = w2[e]^T dy_t                        (grouped GEMM reading w2 as its transposed weight)
//   dg_k  = dh'_r . h_r                         (= dy_t . o_r, since o_r = w2[e] h_r)
//   dh_r  = g_k dh'_r,  da_r = dh_r * b_r * silu'(a_r),  db_r = dh_r * silu(a_r)
//   dlogit_{e_k} = g_k (dg_k - sum_j g_j dg_j)  (softmax over the kept logits)
//   dx_t  = sum_k dxp_{r_k} + W_g dlogit_t,  dxp_r = w1[e]^T da_r + w3[e]^T db_r (grouped GEMM)
//   dW_g  = x^T dlogit,  dw2[e] = sum_r (g_k dy_t) h_r^T,  dw1[e] = sum_r da_r x_t^T,  dw3 likewise
// Operands of the matrix products are bf16 (dy, g*dy, h, da, db rounded to nearest even), every
// sum is fp32, and every reduction runs in a fixed order, so results are reproducible bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// Per token t and slot k (row r = token_row[t][k], gate g_k): dy_perm[r] = bf16(dy[t]),
// do_perm[r] = bf16(g_k dy[t]), row_g[r] = g_k. One block per token, so dy[t] is read once for its K
// rows.
__global__ __launch_bounds__(256) void gather_dy_kernel(const float* __restrict__ dy, const int32_t* __restrict__ token_row,
                                                        const float* __restrict__ topk_w, int K, int d,
                                                        bf16_t* __restrict__ dy_perm, bf16_t* __restrict__ do_perm,
                                                        float* __restrict__ row_g) {
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) row_g[token_row[t * K + threadIdx.x]] = topk_w[t * K + threadIdx.x];
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(dy + t * d + c);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(dy + t * d + c + 4);
    const u32x4_t v =
        u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    for (int k = 0; k < K; ++k) {
      const int64_t r = token_row[t * K + k];
      const float g = topk_w[t * K + k];
      store16(dy_perm + r * d + c, v);
      store16(do_perm + r * d + c,
              u32x4_t{pack_bf16x2(g * a[0], g * a[1]), pack_bf16x2(g * a[2], g * a[3]), pack_bf16x2(g * b[0], g * b[1]),
                      pack_bf16x2(g * b[2], g * b[3])});
    }
  }
}

// Per row r: from its pre-activations a = A[r], b = B[r] (kept by the forward) and dh' = DHP[r]
// (fp32): h = bf16(silu(a) b) (as the forward stores it), dab[r] = [bf16(da) | bf16(db)] with
// da = g dh' b silu'(a), db = g dh' silu(a), and the gate-gradient partials of dg[r] = sum_f dh'_f h_f
// per 64-column chunk c, to dgp[c * rows + r]. One block per row; thread i takes the 4 columns
// 4 i + 1024 j, so 16 consecutive lanes hold one chunk: block a = (i / 4) % 4, quad (i % 4). The
// recomputing path forms the same values in the pre-activation product's epilogue (tile_gemm.hip).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                         const float* __restrict__ DHP,
                                                         const int32_t* __restrict__ row_token,
                                                         const int32_t* __restrict__ token_row,
                                                         const float* __restrict__ topk_w, int K, int F, int64_t rows,
                                                         bf16_t* __restrict__ h, bf16_t* __restrict__ dab,
                                                         float* __restrict__ dgp) {
  const int r = blockIdx.x;
  int t;
  const float g = row_gate(row_token, token_row, topk_w, K, r, t);
  const int64_t o = (int64_t)r * F;
  // F is a multiple of 256, so every wavefront runs the same iterations (the shuffles see whole waves)
  for (int f = threadIdx.x * 4; f < F; f += 256 * 4) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(A + o + f);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(B + o + f);
    const f32x4_t p = *reinterpret_cast<const f32x4_t*>(DHP + o + f);
    float hv[4], da[4], db[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) swiglu_bwd_elem(a[q], b[q], p[q], g, hv[q], da[q], db[q]);
    const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
    *reinterpret_cast<u32x2_t*>(h + o + f) = u32x2_t{h01, h23};
    *reinterpret_cast<u32x2_t*>(dab + 2 * o + f) = u32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
    *reinterpret_cast<u32x2_t*>(dab + 2 * o + F + f) = u32x2_t{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
    float v = dg_quad(p, h01, h23);
    v += __shfl_xor(v, 4, kWave);  // the blocks of the chunk: (a0 + a1) + (a2 + a3)
    v += __shfl_xor(v, 8, kWave);
    v += __shfl_xor(v, 1, kWave);  // then the quads
    v += __shfl_xor(v, 2, kWave);
    if ((threadIdx.x & 15) == 0) dgp[(int64_t)(f >> 6) * rows + r] = v;
  }
}

// dg[r] = sum over the 64-column chunks c of dgp[c * rows + r] (nc a multiple of 4): quarter q of
// the chunks (nc/4 consecutive ones) summed in order, then (q0 + q1) + (q2 + q3). A block takes 64
// rows; lane l of a wavefront takes row l % 16 and quarter l / 16.
__global__ __launch_bounds__(256) void dg_sum_kernel(const float* __restrict__ dgp, int nc, int64_t rows,
                                                     float* __restrict__ dg) {
  const int q = (threadIdx.x >> 4) & 3;
  const int64_t r = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (threadIdx.x & 15);
  const int nq = nc / 4;
  float acc = 0.0f;
  if (r < rows) {
    const float* p = dgp + (int64_t)q * nq * rows + r;
#pragma unroll 8
    for (int c = 0; c < nq; ++c) acc += p[c * rows];
  }
  acc += __shfl_xor(acc, 16, kWave);
  acc += __shfl_xor(acc, 32, kWave);
  if (r < rows && q == 0) dg[r] = acc;
}

// Per token: dlogit_{e_k} = g_k (dg_k - sum_j g_j dg_j), zero for the experts not kept.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ dg, const int32_t* __restrict__ token_row,
                                                         const int32_t* __restrict__ topk_idx,
                                                         const float* __restrict__ topk_w, int64_t T, int E, int K,
                                                         float* __restrict__ dlogits) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float gdg = 0.0f;
  for (int k = 0; k < K; ++k) gdg = fmaf(topk_w[t * K + k], dg[token_row[t * K + k]], gdg);
  for (int e = 0; e < E; ++e) dlogits[t * E + e] = 0.0f;
  for (int k = 0; k < K; ++k) {
    const float gk = topk_w[t * K + k];
    dlogits[t * E + topk_idx[t * K + k]] = gk * (dg[token_row[t * K + k]] - gdg);
  }
}

// dx[t] = sum_k dxp[token_row[t][k]] (slot order) + sum_e W_g[:, e] dlogit[t][e] (expert order).
// When the product that wrote dxp was split into k-ranges, a row of dxp is first rebuilt as the
// sum of its range partials in range order (part + p*part_stride, p < nparts).
// One block per kDxTokens tokens (the gate weights of a column are read once for all of them),
// 4 columns per thread.
constexpr int kDxTokens = 4;
template <int EMAX>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dxp, const float* __restrict__ part,
                                                 int nparts, int64_t part_stride, const int32_t* __restrict__ token_row,
                                                 const float* __restrict__ dlogits, const bf16_t* __restrict__ w_gate,
                                                 int64_t T, int d, int E, int K, float* __restrict__ dx) {
  const int64_t tb = (int64_t)blockIdx.x * kDxTokens;
  const int nt = (int)min<int64_t>(kDxTokens, T - tb);
  float dl[kDxTokens][EMAX];
#pragma unroll
  for (int i = 0; i < kDxTokens; ++i)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) dl[i][e] = (i < nt && e < E) ? dlogits[(tb + i) * E + e] : 0.0f;
  auto row = [&](int64_t t, int k, int c) {
    const int64_t off = (int64_t)token_row[t * K + k] * d + c;
    f32x4_t o = *reinterpret_cast<const f32x4_t*>(dxp + off);
    for (int p = 0; p < nparts; ++p) o = o + *reinterpret_cast<const f32x4_t*>(part + p * part_stride + off);
    return o;
  };
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float wg[4][EMAX];  // W_g[c + q][e]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (EMAX == 8) {
        if (E == 8) {
          const u32x4_t wr = load16(w_gate + (int64_t)(c + q) * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) wg[q][e] = (e & 1) ? bf16_hi(wr[e >> 1]) : bf16_lo(wr[e >> 1]);
          continue;
        }
      }
#pragma unroll
      for (int e = 0; e < EMAX; ++e) wg[q][e] = e < E ? Elem<bf16_t>::to_f32(w_gate[(int64_t)(c + q) * E + e]) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kDxTokens; ++i) {
      if (i >= nt) break;
      const int64_t t = tb + i;
      f32x4_t acc = row(t, 0, c);
      for (int k = 1; k < K; ++k) acc = acc + row(t, k, c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float rsum = 0.0f;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < E) rsum = fmaf(wg[q][e], dl[i][e], rsum);
        acc[q] += rsum;
      }
      *reinterpret_cast<f32x4_t*>(dx + t * d + c) = acc;
    }
  }
}

// The same dx for E = 8, K <= 2 and at most one k-range partial, with K and the partial count known
// at compile time: a column chunk's loads (the four W_g rows, every token's K rows of dxp and their
// partials) are issued together before its arithmetic; the generic loop waits out a memory round trip
// per load behind its run-time slot, partial and expert checks. Same arithmetic in the same order.
template <int KT, int NP>
__global__ __launch_bounds__(256) void dx_fast_kernel(const float* __restrict__ dxp, const float* __restrict__ part,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ dlogits, const bf16_t* __restrict__ w_gate,
                                                      int64_t T, int d, float* __restrict__ dx) {
  const int64_t tb = (int64_t)blockIdx.x * kDxTokens;
  const int nt = (int)min<int64_t>(kDxTokens, T - tb);
  float dl[kDxTokens][8];
  int64_t base[kDxTokens][KT];
#pragma unroll
  for (int i = 0; i < kDxTokens; ++i) {
    const int64_t t = tb + (i < nt ? i : 0);  // tokens past the end read token tb and are not stored
#pragma unroll
    for (int e = 0; e < 8; ++e) dl[i][e] = dlogits[t * 8 + e];
#pragma unroll
    for (int k = 0; k < KT; ++k) base[i][k] = (int64_t)token_row[t * KT + k] * d;
  }
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    u32x4_t wr[4];
    f32x4_t o[kDxTokens][KT], pp[kDxTokens][NP > 0 ? KT : 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) wr[q] = load16(w_gate + (int64_t)(c + q) * 8);
#pragma unroll
    for (int i = 0; i < kDxTokens; ++i)
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        o[i][k] = *reinterpret_cast<const f32x4_t*>(dxp + base[i][k] + c);
        if constexpr (NP > 0) pp[i][k] = *reinterpret_cast<const f32x4_t*>(part + base[i][k] + c);
      }
    float wg[4][8];  // W_g[c + q][e]
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) wg[q][e] = (e & 1) ? bf16_hi(wr[q][e >> 1]) : bf16_lo(wr[q][e >> 1]);
#pragma unroll
    for (int i = 0; i < kDxTokens; ++i) {
      if (i >= nt) break;
      f32x4_t acc = o[i][0];
      if constexpr (NP > 0) acc = acc + pp[i][0];
#pragma unroll
      for (int k = 1; k < KT; ++k) {
        f32x4_t r = o[i][k];
        if constexpr (NP > 0) r = r + pp[i][k];
        acc = acc + r;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float rsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) rsum = fmaf(wg[q][e], dl[i][e], rsum);
        acc[q] += rsum;
      }
      *reinterpret_cast<f32x4_t*>(dx + (tb + i) * d + c) = acc;
    }
  }
}

// dW_g partials: chunk c of kDwgChunk tokens, part[c][j][e] = sum over its tokens t (ascending) of
// x[t][j] * dlogit[t][e]. A thread takes C consecutive columns (4 with up to 8 experts: one 8-byte
// load per token; 2 beyond) and its token loop is unrolled so that U loads are in flight; the
// chunks' partials are then added in chunk order by dwgate_sum_kernel.
constexpr int kDwgChunk = 64;
// EXACT: E == EMAX, so the expert loops carry no bound test (with one, every expert of every token
// became a branch and a wait for its LDS read).
template <int EMAX, int C, bool EXACT>
__global__ __launch_bounds__(64) void dwgate_part_kernel(const bf16_t* __restrict__ x, const float* __restrict__ dlogits,
                                                         int64_t T, int d, int E_, float* __restrict__ part) {
  static_assert(C == 4 || C == 2, "columns per thread");
  const int E = EXACT ? EMAX : E_;
  const int j0 = (blockIdx.x * 64 + threadIdx.x) * C;
  const int ch = blockIdx.y;
  // the chunk's logit gradients, staged once (per token, every lane needs the same E values)
  __shared__ __attribute__((aligned(16))) float sdl[kDwgChunk * EMAX];
  const int64_t t0 = (int64_t)ch * kDwgChunk, t1 = min<int64_t>(T, t0 + kDwgChunk);
  if constexpr (EXACT) {
    // 16-byte pieces, all of a thread's loads in flight together
    constexpr int kPer = kDwgChunk * EMAX / 4 / 64;
    const int n16 = (int)(t1 - t0) * EMAX / 4;
    f32x4_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + 64 * k;
      if (i < n16) v[k] = reinterpret_cast<const f32x4_t*>(dlogits + t0 * EMAX)[i];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + 64 * k;
      if (i < n16) reinterpret_cast<f32x4_t*>(sdl)[i] = v[k];
    }
  } else {
    for (int i = threadIdx.x; i < (int)(t1 - t0) * E; i += 64) sdl[i] = dlogits[t0 * E + i];
  }
  __syncthreads();
  if (j0 >= d) return;
  float acc[C][EMAX];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[c][e] = 0.0f;
  constexpr int U = 16;  // tokens whose loads are issued together
  for (int64_t tb = t0; tb < t1; tb += U) {
    uint32_t xv[U][C / 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (C == 4) {
        const u32x2_t v = tb + u < t1 ? *reinterpret_cast<const u32x2_t*>(x + (tb + u) * d + j0) : u32x2_t{0u, 0u};
        xv[u][0] = v[0];
        xv[u][1] = v[1];
      } else {
        xv[u][0] = tb + u < t1 ? *reinterpret_cast<const uint32_t*>(x + (tb + u) * d + j0) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t1) break;
      const float* dl = sdl + (tb + u - t0) * E;
      float xf[C];
#pragma unroll
      for (int q = 0; q < C / 2; ++q) {
        xf[2 * q] = bf16_lo(xv[u][q]);
        xf[2 * q + 1] = bf16_hi(xv[u][q]);
      }
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e < E) {
          const float g = dl[e];
#pragma unroll
          for (int c = 0; c < C; ++c) acc[c][e] = fmaf(xf[c], g, acc[c][e]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) part[((int64_t)ch * d + j0 + c) * E + e] = acc[c][e];
}

__global__ __launch_bounds__(256) void dwgate_sum_kernel(const float* __restrict__ part, int nch, int d, int E,
                                                         float* __restrict__ dwg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * E) return;
  float s = 0.0f;
#pragma unroll 16
  for (int ch = 0; ch < nch; ++ch) s += part[(int64_t)ch * d * E + i];  // loads in flight together, sums in order
  dwg[i] = s;
}

}  // namespace

int dwgate_chunks(int64_t T) { return (int)((T + kDwgChunk - 1) / kDwgChunk); }

void launch_gather_dy(const float* dy, const int32_t* row_token, const int32_t* token_row, const float* topk_w, int K,
                      int64_t rows, int d, void* dy_perm, void* do_perm, float* row_g, hipStream_t s) {
  (void)row_token;
  launch_kernel(gather_dy_kernel, dim3((unsigned)(rows / K)), dim3(256), 0, s, dy, token_row, topk_w, K, d,
                static_cast<bf16_t*>(dy_perm), static_cast<bf16_t*>(do_perm), row_g);
}

void launch_swiglu_bwd(const float* A, const float* B, const float* DHP, const int32_t* row_token,
                       const int32_t* token_row, const float* topk_w, int K, int64_t rows, int F, void* h, void* dab,
                       float* dgp, hipStream_t s) {
  launch_kernel(swiglu_bwd_kernel, dim3((unsigned)rows), dim3(256), 0, s, A, B, DHP, row_token, token_row, topk_w, K,
                F, rows, static_cast<bf16_t*>(h), static_cast<bf16_t*>(dab), dgp);
}

void launch_dg_sum(const float* dgp, int F, int64_t rows, float* dg, hipStream_t s) {
  launch_kernel(dg_sum_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, s, dgp, F / 64, rows, dg);
}

void launch_router_bwd(const float* dg, const int32_t* token_row, const int32_t* topk_idx, const float* topk_w,
                       int64_t T, int E, int K, float* dlogits, hipStream_t s) {
  launch_kernel(router_bwd_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, dg, token_row, topk_idx, topk_w,
                T, E, K, dlogits);
}

void launch_dx(const float* dxp, const float* part, int nparts, const int32_t* token_row, const float* dlogits,
               const void* w_gate, int64_t T, int d, int E, int K, float* dx, hipStream_t s) {
  const bf16_t* wg = static_cast<const bf16_t*>(w_gate);
  const int64_t stride = T * K * (int64_t)d;
  const unsigned blocks = (unsigned)((T + kDxTokens - 1) / kDxTokens);
  if (E == 8 && (K == 1 || K == 2) && nparts <= 1) {
    auto go = [&](auto kernel) {
      launch_kernel(kernel, dim3(blocks), dim3(256), 0, s, dxp, part, token_row, dlogits, wg, T, d, dx);
    };
    if (K == 2)
      nparts ? go(dx_fast_kernel<2, 1>) : go(dx_fast_kernel<2, 0>);
    else
      nparts ? go(dx_fast_kernel<1, 1>) : go(dx_fast_kernel<1, 0>);
    return;
  }
  if (E <= 8)
    launch_kernel(dx_kernel<8>, dim3((unsigned)((T + kDxTokens - 1) / kDxTokens)), dim3(256), 0, s, dxp, part, nparts,
                  stride, token_row, dlogits, wg, T, d, E, K, dx);
  else
    launch_kernel(dx_kernel<kMaxExperts>, dim3((unsigned)((T + kDxTokens - 1) / kDxTokens)), dim3(256), 0, s, dxp, part,
                  nparts, stride, token_row, dlogits, wg, T, d, E, K, dx);
}

void launch_dwgate(const void* x, const float* dlogits, int64_t T, int d, int E, float* part, float* dwg, hipStream_t s) {
  const int nch = dwgate_chunks(T);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  if (E == 8)
    launch_kernel(dwgate_part_kernel<8, 4, true>, dim3((unsigned)((d + 255) / 256), (unsigned)nch), dim3(64), 0, s,
                  xb, dlogits, T, d, E, part);
  else if (E < 8)
    launch_kernel(dwgate_part_kernel<8, 4, false>, dim3((unsigned)((d + 255) / 256), (unsigned)nch), dim3(64), 0, s,
                  xb, dlogits, T, d, E, part);
  else
    launch_kernel(dwgate_part_kernel<kMaxExperts, 2, false>, dim3((unsigned)((d + 127) / 128), (unsigned)nch), dim3(64), 0, s,
                  xb, dlogits, T, d, E, part);
  launch_kernel(dwgate_sum_kernel, dim3((unsigned)(((int64_t)d * E + 255) / 256)), dim3(256), 0, s, part, nch, d, E, dwg);
}

}  // namespace moe
