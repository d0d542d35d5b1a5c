// Token permutation into expert-contiguous order: per-expert histogram, exclusive scan, stable
// scatter (tokens per expert vary from call to call: zh.newsflash.city article, section on the
// mixture-of-experts layer; ja.news.hada.io summary on MegaBlocks-style grouping).
//
// permute_index_kernel runs as ONE workgroup: T*K slot ids are tiny (C4: 128 KB) and a single
// workgroup makes the result deterministic without atomics. Thread i owns a contiguous chunk of
// slots s = t*K + k. (1) It counts its chunk per expert into an LDS table cnt[e][i].
// (2) An exclusive scan over that table in (expert, thread) order turns each entry into the
// first row thread i writes for expert e. (3) Thread i walks its chunk again in slot order and
// hands out consecutive rows. Rows of one expert therefore follow ascending token index.
//
// gather_rows_kernel copies whole rows x[row_token[r]] -> x_perm[r] with 16-byte accesses
// (HBM-bound: 2 * T*K*d*elem bytes).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <int NT>
__global__ __launch_bounds__(NT) void permute_index_kernel(const int32_t* __restrict__ topk_idx, int64_t S, int K,
                                                           int E, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ token_row) {
  extern __shared__ int32_t cnt[];  // [E][NT]
  __shared__ int32_t wave_tot[NT / kWave];
  const int i = threadIdx.x;
  const int64_t chunk = (S + NT - 1) / NT;
  const int64_t s0 = min<int64_t>(S, (int64_t)i * chunk);
  const int64_t s1 = min<int64_t>(S, s0 + chunk);

  for (int e = 0; e < E; ++e) cnt[e * NT + i] = 0;
  // unrolled so that the chunk's loads are in flight together rather than one latency each
#pragma unroll 8
  for (int64_t s = s0; s < s1; ++s) cnt[topk_idx[s] * NT + i] += 1;
  __syncthreads();

  // Exclusive scan of the flattened table (index e*NT + i); thread j owns entries [j*E, (j+1)*E).
  int run = 0;
  for (int q = 0; q < E; ++q) run += cnt[i * E + q];
  const int lane = i & (kWave - 1), w = i / kWave;
  int incl = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int excl = incl - run;
  for (int q = 0; q < w; ++q) excl += wave_tot[q];
  for (int q = 0; q < E; ++q) {
    int v = cnt[i * E + q];
    cnt[i * E + q] = excl;
    excl += v;
  }
  __syncthreads();

  if (i < E) {
    const int lo = cnt[i * NT];
    const int hi = (i + 1 < E) ? cnt[(i + 1) * NT] : (int)S;
    offsets[i] = lo;
    counts[i] = hi - lo;
  }
  if (i == 0) offsets[E] = (int)S;
  __syncthreads();

  // eight slot ids loaded together, then handed out in slot order
  for (int64_t s = s0; s < s1; s += 8) {
    int e8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) e8[u] = topk_idx[min(s + u, s1 - 1)];  // clamped: loads need no branch
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s + u < s1) {
        const int row = cnt[e8[u] * NT + i]++;
        row_token[row] = (int32_t)((s + u) / K);
        token_row[s + u] = row;
      }
    }
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token, int64_t rows,
                                                          int64_t row_bytes, uint8_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= rows) return;
  const int64_t src = row_token[r];
  const uint8_t* in = x + src * row_bytes;
  uint8_t* out = x_perm + r * row_bytes;
  for (int64_t off = (int64_t)lane * 16; off < row_bytes; off += kWave * 16) store16(out + off, load16(in + off));
}

template <int NT>
void launch_index(const int32_t* idx, int64_t S, int K, int E, int32_t* counts, int32_t* offsets,
                  int32_t* row_token, int32_t* token_row, hipStream_t s) {
  launch_kernel((permute_index_kernel<NT>), dim3(1), dim3(NT), (size_t)E * NT * sizeof(int32_t), s, idx, S, K,
                     E, counts, offsets, row_token, token_row);
}

}  // namespace

void launch_permute_index(const int32_t* topk_idx, int64_t T, int E, int K, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t stream) {
  const int64_t S = T * K;
  // the LDS table holds E*NT int32 (at most 32 KB); a single wavefront for few slots (decode)
  if (S <= 512)
    launch_index<64>(topk_idx, S, K, E, counts, offsets, row_token, token_row, stream);
  else if (E <= 8)
    launch_index<1024>(topk_idx, S, K, E, counts, offsets, row_token, token_row, stream);
  else if (E <= 16)
    launch_index<512>(topk_idx, S, K, E, counts, offsets, row_token, token_row, stream);
  else if (E <= 32)
    launch_index<256>(topk_idx, S, K, E, counts, offsets, row_token, token_row, stream);
  else
    launch_index<128>(topk_idx, S, K, E, counts, offsets, row_token, token_row, stream);
}

void launch_gather_rows(const void* x, const int32_t* row_token, int64_t rows, int64_t row_bytes, void* x_perm,
                        hipStream_t stream) {
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  launch_kernel(gather_rows_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint8_t*>(x),
                     row_token, rows, row_bytes, static_cast<uint8_t*>(x_perm));
}

}  // namespace moe
