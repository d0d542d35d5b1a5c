// Token permutation into expert-contiguous order: per-expert histogram, exclusive scan, stable
// scatter (tokens per expert vary from call to call: zh.newsflash.city article, section on the
// mixture-of-experts layer; ja.news.hada.io summary on MegaBlocks-style grouping).
//
// permute_index_kernel runs as ONE workgroup (few slots, or more than 8 experts): a single
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

// Many slots, E <= 8: one workgroup per window of 1024 consecutive slots (4 per thread), so the
// scatter runs on many CUs instead of one. Each workgroup counts every slot's expert itself (S int32
// loads from L2, all of a thread's loads of a batch in flight), taking the counts of the windows
// before its own as its starting rows; the windows are aligned with the threads' loads, so a
// thread's count before its own window is a running total at the window's start. Its own slots are
// then ranked as in permute_index_kernel (per-thread counts, a scan in thread order), which gives
// the same rows: every expert's rows in ascending slot order. No workgroup reads what another
// writes. Per call, with launch (T tokens, K = 2): T = 2048 11.1 -> 8.3 us, T = 4096 17.6 -> 9.2 us,
// T = 16384 64.7 -> 17.1 us against the single workgroup.
constexpr int kPermWin = 1024;
__global__ __launch_bounds__(256) void permute_window_kernel(const int32_t* __restrict__ topk_idx, int64_t S, int K,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_token,
                                                             int32_t* __restrict__ token_row) {
  __shared__ int32_t red[4][16];   // per-wave [before | total] per expert
  __shared__ int32_t wtot[4][8];   // per-wave totals of the own-window counts
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  const int64_t win = blockIdx.x;
  // per-thread counts in 16-bit fields: expert e in field e % 2 of register e / 2 (a thread sees at
  // most S / 256 slots of one expert; S < 2^24 keeps that below 2^16)
  uint32_t tot[4] = {0u, 0u, 0u, 0u}, bef[4] = {0u, 0u, 0u, 0u};
  int mine[4] = {-1, -1, -1, -1};
  auto add = [](uint32_t (&c)[4], int e) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] += (e >> 1) == r ? (1u << (16 * (e & 1))) : 0u;
  };
  constexpr int U = 8;  // windows per batch of loads
  const int64_t nwin = (S + kPermWin - 1) / kPermWin;
  for (int64_t w0 = 0; w0 < nwin; w0 += U) {
    int v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t sl = (w0 + u) * kPermWin + 4 * i + j;
        v[u][j] = topk_idx[sl < S ? sl : S - 1];  // clamped: the loads need no branch
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (w0 + u == win) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bef[r] = tot[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) mine[j] = (win * kPermWin + 4 * i + j < S) ? v[u][j] : -1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((w0 + u) * kPermWin + 4 * i + j < S) add(tot, v[u][j]);
    }
  }
  // workgroup sums of bef and tot per expert (fixed order: butterfly, then the four waves)
  int bsum[8], tsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bsum[e] = (int)((bef[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    tsum[e] = (int)((tot[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      bsum[e] += __shfl_xor(bsum[e], m, kWave);
      tsum[e] += __shfl_xor(tsum[e], m, kWave);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[w][e] = bsum[e];
      red[w][8 + e] = tsum[e];
    }
  }
  // own window: this thread's counts per expert and their inclusive scan over the wave
  int own[8], incl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    own[e] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) own[e] += mine[j] == e ? 1 : 0;
    incl[e] = own[e];
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = __shfl_up(incl[e], o, kWave);
      if (lane >= o) incl[e] += n;
    }
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wtot[w][e] = incl[e];
  }
  __syncthreads();
  int next[8];  // next row of each expert for this thread
  int start = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int before = red[0][e] + red[1][e] + red[2][e] + red[3][e];
    const int total = red[0][8 + e] + red[1][8 + e] + red[2][8 + e] + red[3][8 + e];
    int wave_before = 0;
    for (int q = 0; q < w; ++q) wave_before += wtot[q][e];
    next[e] = start + before + wave_before + incl[e] - own[e];
    if (win == 0 && i == 0 && e < E) {
      offsets[e] = start;
      counts[e] = total;
    }
    start += e < E ? total : 0;
  }
  if (win == 0 && i == 0) offsets[E] = (int)S;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = mine[j];
    if (e < 0) continue;
    int row = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      row = e == q ? next[q] : row;
      next[q] += e == q ? 1 : 0;
    }
    const int64_t sl = win * kPermWin + 4 * i + j;
    row_token[row] = (int32_t)(sl / K);
    token_row[sl] = row;
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
  if (S > 2048 && E <= 8 && S < (1 << 24)) {
    launch_kernel(permute_window_kernel, dim3((unsigned)((S + kPermWin - 1) / kPermWin)), dim3(256), 0, stream, topk_idx,
                  S, K, E, counts, offsets, row_token, token_row);
    return;
  }
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
