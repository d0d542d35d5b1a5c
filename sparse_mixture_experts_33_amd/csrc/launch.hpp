// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI is in moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 64;

void launch_route(int dtype, const void* x, const void* w_gate, const float* bias, int64_t T, int d, int E, int K,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream);

void launch_permute_index(const int32_t* topk_idx, int64_t T, int E, int K, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t stream);

void launch_gather_rows(const void* x, const int32_t* row_token, int64_t rows, int64_t row_bytes, void* x_perm,
                        hipStream_t stream);

// Expert FFN over expert-contiguous rows. row_src == nullptr: activation row r is act[r];
// otherwise act[row_src[r]] (the gather of the permutation fused into the first matmul).
// expected_rows_per_expert (T*K/E) picks the tile shape; any routing is handled correctly.
void launch_expert_ffn(int dtype, const void* act, const int32_t* row_src, const int32_t* offsets, int64_t rows,
                       int d, int F, int E, const void* w1, const void* w3, const void* w2, void* h, float* y_perm,
                       hipStream_t stream);

void launch_combine(const float* y_perm, const int32_t* token_row, const float* topk_w, int64_t T, int d, int K,
                    int y_dtype, int accumulate, void* y, hipStream_t stream);

void launch_rmsnorm(const float* h, int64_t T, int d, float eps, void* x_bf16, hipStream_t stream);

}  // namespace moe
