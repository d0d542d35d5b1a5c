// One-time rearrangement of expert weights W[E][N][K] (row-major) into the fragment-packed
// layout read by the grouped expert GEMMs (layout defined next to moe_pack_weights in moe.h):
// 16 rows x 4V columns per 1 KB fragment, lane order, fragments of a 16-row block adjacent.
// One thread writes one 16-byte piece; writes are fully coalesced, each read is 16 contiguous
// bytes of a row.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ w, int64_t pieces, int N, int K,
                                                   T* __restrict__ wp) {
  constexpr int V = 16 / sizeof(T);
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte piece of the output
  if (o >= pieces) return;
  const int lane = (int)(o & 63);
  const int64_t frag = o >> 6;
  const int64_t frags_per_block = K / (4 * V);
  const int64_t blk = frag / frags_per_block;  // e*(N/16) + n/16
  const int q = (int)(frag - blk * frags_per_block);
  const int64_t row = blk * 16 + (lane & 15);  // e*N + n
  const int64_t k0 = (int64_t)q * 4 * V + (lane >> 4) * V;
  store16(wp + o * V, load16(w + row * K + k0));
}

}  // namespace

void launch_pack_weights(int dtype, const void* w, int E, int N, int K, void* w_packed, hipStream_t stream) {
  const int V = dtype == kBF16 ? 8 : 4;
  const int64_t pieces = (int64_t)E * N * K / V;
  const unsigned blocks = (unsigned)((pieces + 255) / 256);
  if (dtype == kBF16)
    launch_kernel(pack_kernel<bf16_t>, dim3(blocks), dim3(256), 0, stream, static_cast<const bf16_t*>(w), pieces,
                       N, K, static_cast<bf16_t*>(w_packed));
  else
    launch_kernel(pack_kernel<float>, dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(w), pieces,
                       N, K, static_cast<float*>(w_packed));
}

}  // namespace moe
