// Device-side helpers shared by the gfx950 kernels of the mixture-of-experts library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 stored as its 16-bit pattern

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;  // MFMA bf16 operand (8 values per lane)
typedef __attribute__((ext_vector_type(4))) float f32x4_t;    // 16x16 MFMA accumulator fragment
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t; // one 16-byte global/LDS access
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static inline float to_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
  __device__ static inline float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ inline u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ inline u32x4_t load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ inline void store16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16x16 output tile, 32-deep bf16 contraction on the matrix cores:
// D[i][j] += sum_k A[i][k] B[k][j]; lane l supplies row i = l%16 of A and column j = l%16 of B,
// 8 consecutive k values each; lane l receives D rows 4*(l/16)..+3 of column l%16.
__device__ inline f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// Same 16x16 tile with a 4-deep fp32 contraction: one k value per lane.
__device__ inline f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T> __device__ inline T wave_bcast0(T v) { return __shfl(v, 0, kWave); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Maps a linear tile index to (expert, first row, rows) for expert groups of
// `tile` rows: expert e owns ceil(n_e / tile) consecutive tile indices. Returns
// false when the index lies past the last tile (the grid is sized for the
// worst case because the group sizes live only on the device).
__device__ inline bool find_tile(const int32_t* offsets, int E, int tile, int idx, int& e_out, int& r0,
                                 int& nrows) {
  for (int e = 0; e < E; ++e) {
    int lo = offsets[e], hi = offsets[e + 1];
    int nt = (hi - lo + tile - 1) / tile;
    if (idx < nt) {
      e_out = e;
      r0 = lo + idx * tile;
      nrows = min(tile, hi - r0);
      return true;
    }
    idx -= nt;
  }
  return false;
}

// SwiGLU expert activation (xyznot.com summary, "Método": silu(x w1) * (x w3)) and its derivative.
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

// Backward of one SwiGLU element of a routed row with gate g, pre-activations a, b and
// dh' = (w2^T dy)_f = p: h = silu(a) b, da = g p b silu'(a), db = g p silu(a). The kernel that reads
// stored pre-activations and the pre-activation product's epilogue both call this, so the two give
// the same bits.
__device__ inline void swiglu_bwd_elem(float a, float b, float p, float g, float& h, float& da, float& db) {
  const float s = silu_f(a);
  h = s * b;
  const float dh = g * p;
  da = dh * b * dsilu_f(a);
  db = dh * s;
}

// Gate-gradient partial of 4 consecutive columns: sum over q of p_q h_q in q order, h_q as stored
// (bf16). The gate gradient of a row is summed in a fixed order from these: the four quads of a
// 16-column block and the four blocks of a 64-column chunk as two pairwise trees
// ((q0 + q1) + (q2 + q3) over blocks, then over quads), then the chunks in column order.
__device__ inline float dg_quad(f32x4_t p, uint32_t h01, uint32_t h23) {
  float v = 0.0f;
  v = fmaf(p[0], bf16_lo(h01), v);
  v = fmaf(p[1], bf16_hi(h01), v);
  v = fmaf(p[2], bf16_lo(h23), v);
  v = fmaf(p[3], bf16_hi(h23), v);
  return v;
}

}  // namespace moe
