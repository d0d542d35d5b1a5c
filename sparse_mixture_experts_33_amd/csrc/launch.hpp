// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI is in moe.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Dispatch timing. A caller arms a pair of events; the next kernel launched by the same host
// thread records them as its own start and end timestamps (hipExtLaunchKernel), so timing adds
// no packet to the queue (an hipEventRecord between two kernels holds the next dispatch back by
// several microseconds). The launch disarms them.
struct DispatchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
DispatchEvents& pending_dispatch_events();  // per host thread

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  DispatchEvents& ev = pending_dispatch_events();
  if (ev.start || ev.stop) {
    const DispatchEvents e = ev;
    ev = DispatchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e.start, e.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kRowMajor = 0;
constexpr int kPacked = 1;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 64;
constexpr int kMaxKSplit = 4;  // k-ranges of the down projection in moe_forward

void launch_route(int dtype, const void* x, const void* w_gate, const float* bias, int64_t T, int d, int E, int K,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream);

void launch_permute_index(const int32_t* topk_idx, int64_t T, int E, int K, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t stream);

void launch_gather_rows(const void* x, const int32_t* row_token, int64_t rows, int64_t row_bytes, void* x_perm,
                        hipStream_t stream);

// Expert FFN over expert-contiguous rows, as two grouped GEMMs.
// up:   h[r] = silu(act[src(r)] . w1[e]^T) * (act[src(r)] . w3[e]^T), src(r) = row_src ? row_src[r] : r
//       (row_src carries the permutation's gather into the first matmul)
// down: y_perm[r] = h[r] . w2[e]^T
// rows = T*K; the tile shape is chosen from rows/E, and any routing is handled correctly.
// layout: kRowMajor or kPacked (fragment-packed weights, see moe_pack_weights in moe.h).
// hpk (tiled path only): h is kept fragment-packed between the two products, each group starting a
// new 16-row block (tile_gemm.hip, HPK); it then needs (rows + 15 E) x F elements and is read only by
// launch_expert_down with the same flag. The streaming path ignores it (h row-major).
void launch_expert_up(int dtype, int layout, const void* act, const int32_t* row_src, const int32_t* offsets,
                      int64_t rows, int d, int F, int E, const void* w1, const void* w3, void* h, hipStream_t stream,
                      bool hpk = false);
// ksplit > 1 (moe_forward only, tiled path only): k-range p > 0 writes its partial sums to
// y_part + (p-1)*rows*d; y_perm then holds only range 0 and the combine adds the rest.
void launch_expert_down(int dtype, int layout, const void* h, const int32_t* offsets, int64_t rows, int d, int F,
                        int E, const void* w2, float* y_perm, int ksplit, float* y_part, hipStream_t stream,
                        bool hpk = false);

// Tiled (LDS-staged, 256 x 256) grouped GEMMs for large groups; tile_gemm_applies says when
// they are used instead of the streaming kernels.
bool tile_gemm_applies(int dtype, int64_t rows, int E, int d, int F);
// k-ranges the down projection of moe_forward is split into (1 = no split).
int tile_down_ksplit(int dtype, int64_t rows, int E, int d, int F);
void launch_tile_up(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows, int d,
                    int F, int E, const void* w1, const void* w3, void* h, hipStream_t stream, bool hpk = false);
// Grouped product with transposed weights (backward pass): out[r][n] = sum_k act[r][k] W_e[k][n] for the
// rows r of group e, W_e [K][N] row-major (kRowMajor) or fragment-packed as [K][N] (kPacked); wa holds
// k < K/2 and wb the rest when wb is given (wb NULL: wa holds all K). fp32 out, split into ksplit
// k-ranges as launch_tile_down. N multiple of 256, K of 64 (of 128 with wb).
void launch_tile_wt(int layout, const void* act, const int32_t* offsets, int64_t rows, int N, int K, int E,
                    const void* wa, const void* wb, float* out, int ksplit, float* part, hipStream_t stream);
// The two pre-activations a = x.w1^T, b = x.w3^T (fp32) in one pass of the up tile, and, if h is
// not null, h = bf16(silu(a) b) as the fused product forms it (the forward keeping activations).
void launch_tile_up_pair(int layout, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                         int d, int F, int E, const void* w1, const void* w3, float* a, float* b, hipStream_t stream,
                         void* h = nullptr, bool hpk = false);
// Backward pass: the same pair product finishing the SwiGLU derivative in its epilogue, given
// dh' = w2^T dy of every row (fp32 [rows][F]): h = bf16(silu(a) b) [rows][F], dab = [bf16(da) |
// bf16(db)] [rows][2F] and the gate-gradient partials dgp [F/64][rows] (launch_dg_sum adds them up),
// the same bits as launch_swiglu_bwd forms from stored a, b. row_token gathers the rows of x, row_g
// holds each row's gate (launch_gather_dy); sink is 16 bytes of device memory whose contents are
// never used (it takes the stores of the rows past a tile's end).
void launch_tile_up_pair_bwd(int layout, const void* act, const int32_t* row_token, const int32_t* offsets,
                             int64_t rows, int d, int F, int E, const void* w1, const void* w3, const float* dhp,
                             const float* row_g, void* h, void* dab, float* dgp, void* sink, hipStream_t stream);
void launch_tile_down(int layout, const void* h, const int32_t* offsets, int64_t rows, int d, int F, int E,
                      const void* w2, float* y_perm, int ksplit, float* y_part, hipStream_t stream, bool hpk = false);

// Weight-gradient products of the backward pass (bf16 operands, fp32 out): for each expert e,
// out[e][m][n] = sum over the rows r of e's group of p[r][m] * q[r][n], p and q group-sorted rows of
// strides ldp and ldq. M and N multiples of 256. packed_out: out[e] in the fragment-packed element
// order of an [M][N] weight instead of row-major.
void launch_tile_wgrad(const void* p, int M, int ldp, const void* q, int N, int ldq, const int32_t* offsets, int E,
                       float* out, hipStream_t stream, bool packed_out = false);

// Rearranges W[E][N][K] (row-major) into the fragment-packed layout.
void launch_pack_weights(int dtype, const void* w, int E, int N, int K, void* w_packed, hipStream_t stream);

// nparts extra partial-sum buffers (y_part, each rows*d) are added to y_perm in order first.
void launch_combine(const float* y_perm, const float* y_part, int nparts, const int32_t* token_row, const float* topk_w,
                    int64_t T, int d, int K, int y_dtype, int accumulate, void* y, hipStream_t stream);

void launch_rmsnorm(const float* h, int64_t T, int d, float eps, void* x_bf16, hipStream_t stream);

// Backward pass (bf16 operands, fp32 sums; see backward.hip).
// dy_perm[r] = bf16(dy[t]), do_perm[r] = bf16(g dy[t]), row_g[r] = g for row r = (t, k) with gate g.
void launch_gather_dy(const float* dy, const int32_t* row_token, const int32_t* token_row, const float* topk_w, int K,
                      int64_t rows, int d, void* dy_perm, void* do_perm, float* row_g, hipStream_t stream);
// h = bf16(silu(A) B), dab = [bf16(g dh' B silu'(A)) | bf16(g dh' silu(A))] per row, and the partials
// dgp [F/64][rows] of dg = dh' . h per 64-column chunk (F a multiple of 256).
void launch_swiglu_bwd(const float* A, const float* B, const float* DHP, const int32_t* row_token,
                       const int32_t* token_row, const float* topk_w, int K, int64_t rows, int F, void* h, void* dab,
                       float* dgp, hipStream_t stream);
// dg[r] = sum of the F/64 partials of row r in chunk order.
void launch_dg_sum(const float* dgp, int F, int64_t rows, float* dg, hipStream_t stream);
void launch_router_bwd(const float* dg, const int32_t* token_row, const int32_t* topk_idx, const float* topk_w,
                       int64_t T, int E, int K, float* dlogits, hipStream_t stream);
// dxp rows are rebuilt from nparts extra k-range partials (part, each T*K*d) before the sum.
void launch_dx(const float* dxp, const float* part, int nparts, const int32_t* token_row, const float* dlogits,
               const void* w_gate, int64_t T, int d, int E, int K, float* dx, hipStream_t stream);
// dW_g = x^T dlogits; part holds dwgate_chunks(T) * d * E floats.
int dwgate_chunks(int64_t T);
void launch_dwgate(const void* x, const float* dlogits, int64_t T, int d, int E, float* part, float* dwg,
                   hipStream_t stream);

// Decoder block (attention.hip). Head width 128; a key-value head serves a multiple of 4 query heads.
// qkv [T][(Hq + 2 Hkv) * 128] fp32 -> q [Hq][T][128], k, v [Hkv][T][128] bf16, rotary embedding on q, k.
void launch_rope_qkv(const float* qkv, int64_t T, int Hq, int Hkv, double base, void* q, void* k, void* v,
                     hipStream_t stream);
// Causal grouped-query attention: q [Hq][T][128], k, v [Hkv][T][128] -> o [T][Hq * 128], all bf16.
void launch_attention(const void* q, const void* k, const void* v, void* o, int64_t T, int Hq, int Hkv,
                      hipStream_t stream);
// h += a (fp32), x = bf16(rmsnorm(h)) (unit weight).
void launch_residual_norm(float* h, const float* a, int64_t T, int d, float eps, void* x, hipStream_t stream);
// off = {0, T}: one group holding every row (dense products through the grouped kernels).
void launch_set_offsets(int32_t* off, int64_t T, hipStream_t stream);

}  // namespace moe
