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

__device__ inline float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ inline float dsilu_f(float z) {
  const float s = 1.0f / (1.0f + expf(-z));
  return s * (1.0f + z * (1.0f - s));
}

// Slot k of row r (row_token[r] = t and token_row[t*K + k] = r) and its gate weight.
__device__ inline float row_gate(const int32_t* row_token, const int32_t* token_row, const float* topk_w, int K,
                                 int r, int& t_out) {
  const int t = row_token[r];
  float g = 0.0f;
  for (int k = 0; k < K; ++k)
    if (token_row[(int64_t)t * K + k] == r) g = topk_w[(int64_t)t * K + k];
  t_out = t;
  return g;
}

// Per row r = (t, k): dy_perm[r] = bf16(dy[t]), do_perm[r] = bf16(g_k dy[t]). One block per row.
__global__ __launch_bounds__(256) void gather_dy_kernel(const float* __restrict__ dy, const int32_t* __restrict__ row_token,
                                                        const int32_t* __restrict__ token_row,
                                                        const float* __restrict__ topk_w, int K, int d,
                                                        bf16_t* __restrict__ dy_perm, bf16_t* __restrict__ do_perm) {
  const int r = blockIdx.x;
  int t;
  const float g = row_gate(row_token, token_row, topk_w, K, r, t);
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(dy + (int64_t)t * d + c);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(dy + (int64_t)t * d + c + 4);
    store16(dy_perm + (int64_t)r * d + c,
            u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
    store16(do_perm + (int64_t)r * d + c,
            u32x4_t{pack_bf16x2(g * a[0], g * a[1]), pack_bf16x2(g * a[2], g * a[3]), pack_bf16x2(g * b[0], g * b[1]),
                    pack_bf16x2(g * b[2], g * b[3])});
  }
}

// Per row r: from the recomputed pre-activations a = A[r], b = B[r] and dh' = DHP[r] (fp32):
// h = bf16(silu(a) b) (as the forward stores it), dg[r] = sum_f dh'_f h_f (fixed order),
// dab[r] = [bf16(da) | bf16(db)] with da = g dh' b silu'(a), db = g dh' silu(a). One block per row.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                         const float* __restrict__ DHP,
                                                         const int32_t* __restrict__ row_token,
                                                         const int32_t* __restrict__ token_row,
                                                         const float* __restrict__ topk_w, int K, int F,
                                                         bf16_t* __restrict__ h, bf16_t* __restrict__ dab,
                                                         float* __restrict__ dg) {
  __shared__ float part[256 / kWave];
  const int r = blockIdx.x;
  int t;
  const float g = row_gate(row_token, token_row, topk_w, K, r, t);
  const int64_t o = (int64_t)r * F;
  float acc = 0.0f;
  for (int f = threadIdx.x * 4; f < F; f += 256 * 4) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(A + o + f);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(B + o + f);
    const f32x4_t p = *reinterpret_cast<const f32x4_t*>(DHP + o + f);
    float hv[4], da[4], db[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s = silu_f(a[q]);
      hv[q] = s * b[q];
      const float dh = g * p[q];
      da[q] = dh * b[q] * dsilu_f(a[q]);
      db[q] = dh * s;
    }
    const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
    *reinterpret_cast<u32x2_t*>(h + o + f) = u32x2_t{h01, h23};
    acc = fmaf(p[0], bf16_lo(h01), acc);
    acc = fmaf(p[1], bf16_hi(h01), acc);
    acc = fmaf(p[2], bf16_lo(h23), acc);
    acc = fmaf(p[3], bf16_hi(h23), acc);
    *reinterpret_cast<u32x2_t*>(dab + 2 * o + f) = u32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
    *reinterpret_cast<u32x2_t*>(dab + 2 * o + F + f) = u32x2_t{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) dg[r] = ((part[0] + part[1]) + part[2]) + part[3];
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
// One block per token, 4 columns per thread.
template <int EMAX>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dxp, const float* __restrict__ part,
                                                 int nparts, int64_t part_stride, const int32_t* __restrict__ token_row,
                                                 const float* __restrict__ dlogits, const bf16_t* __restrict__ w_gate,
                                                 int d, int E, int K, float* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  float dl[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) dl[e] = e < E ? dlogits[t * E + e] : 0.0f;
  auto row = [&](int k, int c) {
    const int64_t off = (int64_t)token_row[t * K + k] * d + c;
    f32x4_t o = *reinterpret_cast<const f32x4_t*>(dxp + off);
    for (int p = 0; p < nparts; ++p) o = o + *reinterpret_cast<const f32x4_t*>(part + p * part_stride + off);
    return o;
  };
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    f32x4_t s = row(0, c);
    for (int k = 1; k < K; ++k) s = s + row(k, c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float rsum = 0.0f;
      if (EMAX == 8 && E == 8) {
        // the row's 8 gate weights in one 16-byte load; same order of products as below
        const u32x4_t wr = load16(w_gate + (int64_t)(c + q) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          rsum = fmaf((e & 1) ? bf16_hi(wr[e >> 1]) : bf16_lo(wr[e >> 1]), dl[e], rsum);
      } else {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
          if (e < E) rsum = fmaf(Elem<bf16_t>::to_f32(w_gate[(int64_t)(c + q) * E + e]), dl[e], rsum);
      }
      s[q] += rsum;
    }
    *reinterpret_cast<f32x4_t*>(dx + t * d + c) = s;
  }
}

// dW_g = x^T dlogit in two passes: part[ch][j][e] = sum over the tokens of chunk ch (ascending),
// then dW_g[j][e] = sum over chunks (ascending). One thread per column j.
constexpr int kDwgChunk = 128;
template <int EMAX>
__global__ __launch_bounds__(256) void dwgate_part_kernel(const bf16_t* __restrict__ x, const float* __restrict__ dlogits,
                                                          int64_t T, int d, int E, float* __restrict__ part) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int ch = blockIdx.y;
  if (j >= d) return;
  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0f;
  const int64_t t1 = min<int64_t>(T, (int64_t)(ch + 1) * kDwgChunk);
  for (int64_t t = (int64_t)ch * kDwgChunk; t < t1; ++t) {
    const float xv = Elem<bf16_t>::to_f32(x[t * d + j]);
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) acc[e] = fmaf(xv, dlogits[t * E + e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) part[((int64_t)ch * d + j) * E + e] = acc[e];
}

__global__ __launch_bounds__(256) void dwgate_sum_kernel(const float* __restrict__ part, int nch, int d, int E,
                                                         float* __restrict__ dwg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * E) return;
  float s = 0.0f;
  for (int ch = 0; ch < nch; ++ch) s += part[(int64_t)ch * d * E + i];
  dwg[i] = s;
}

}  // namespace

int dwgate_chunks(int64_t T) { return (int)((T + kDwgChunk - 1) / kDwgChunk); }

void launch_gather_dy(const float* dy, const int32_t* row_token, const int32_t* token_row, const float* topk_w, int K,
                      int64_t rows, int d, void* dy_perm, void* do_perm, hipStream_t s) {
  launch_kernel(gather_dy_kernel, dim3((unsigned)rows), dim3(256), 0, s, dy, row_token, token_row, topk_w, K, d,
                static_cast<bf16_t*>(dy_perm), static_cast<bf16_t*>(do_perm));
}

void launch_swiglu_bwd(const float* A, const float* B, const float* DHP, const int32_t* row_token,
                       const int32_t* token_row, const float* topk_w, int K, int64_t rows, int F, void* h, void* dab,
                       float* dg, hipStream_t s) {
  launch_kernel(swiglu_bwd_kernel, dim3((unsigned)rows), dim3(256), 0, s, A, B, DHP, row_token, token_row, topk_w, K,
                F, static_cast<bf16_t*>(h), static_cast<bf16_t*>(dab), dg);
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
  if (E <= 8)
    launch_kernel(dx_kernel<8>, dim3((unsigned)T), dim3(256), 0, s, dxp, part, nparts, stride, token_row, dlogits, wg,
                  d, E, K, dx);
  else
    launch_kernel(dx_kernel<kMaxExperts>, dim3((unsigned)T), dim3(256), 0, s, dxp, part, nparts, stride, token_row,
                  dlogits, wg, d, E, K, dx);
}

void launch_dwgate(const void* x, const float* dlogits, int64_t T, int d, int E, float* part, float* dwg, hipStream_t s) {
  const int nch = dwgate_chunks(T);
  const dim3 g1((unsigned)((d + 255) / 256), (unsigned)nch);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  if (E <= 8)
    launch_kernel(dwgate_part_kernel<8>, g1, dim3(256), 0, s, xb, dlogits, T, d, E, part);
  else
    launch_kernel(dwgate_part_kernel<kMaxExperts>, g1, dim3(256), 0, s, xb, dlogits, T, d, E, part);
  launch_kernel(dwgate_sum_kernel, dim3((unsigned)(((int64_t)d * E + 255) / 256)), dim3(256), 0, s, part, nch, d, E, dwg);
}

}  // namespace moe
