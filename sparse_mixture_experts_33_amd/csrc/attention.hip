// Decoder block around the mixture-of-experts layer: rotary embedding, causal grouped-query
// attention and the residual + norm step. The pages give the block by its numbers only (xyznot.com
// summary, "Método": 32 attention heads, 8 key-value heads, width 4096, the Mistral 7B layout with
// the MoE layer in place of the feed-forward sub-block, a full 32k context); head width 128 and
// the rotary form are readings (no position encoding is named on the pages).
//
// Attention (flash form, one pass over the keys with a running softmax): a workgroup takes 64
// query positions of the 4 query heads that share one key-value head (group size Hq/Hkv a
// multiple of 4), two wavefronts per head, so every 64-key tile staged in LDS serves 4 heads.
// Per wavefront and key tile, on 16x16x32 bf16 MFMAs with fp32 sums:
//   S^T = K Q^T       (K from LDS, the wavefront's Q fragments held in registers all along)
//   running max / sum per query, P = exp(S - max) rounded to bf16
//   O^T += V^T P^T    (V^T assembled by transposing LDS reads, P^T straight from the S^T
//                      accumulators: the contraction order over keys is chosen to match the
//                      layout in which the accumulators hold them)
// Query positions are the output columns of both products, so every softmax statistic lives in
// the four lanes that hold one column (two cross-lane steps). Query blocks are launched longest
// first (a block at position p visits p/64 + 1 key tiles).
#include "common.hpp"
#include "launch.hpp"

#include <cmath>

namespace moe {
namespace {

constexpr int kHD = 128;         // head width
constexpr int kQB = 64;          // query positions per workgroup (per wavefront)
constexpr int kKB = 64;          // keys per tile
// LDS rows of the K and V tiles (elements): 288 B. Measured on gfx950 with the bank-conflict
// counter, this stride leaves both the 16-byte K-fragment reads and the transposing V reads free
// of conflicts; 272 B, conflict-free for the K reads under a plain 32-bank model, doubles their
// LDS cycles.
constexpr int kKRow = kHD + 16;
constexpr int kVRow = kHD + 16;

// qkv [T][(Hq + 2 Hkv) * 128] fp32 -> q [Hq][T][128], k [Hkv][T][128], v [Hkv][T][128] bf16, with the
// rotary embedding on q and k: in each head the pair (i, i + 64) of position t turns by the angle
// t * base^(-i/64). One workgroup per position: thread (i = tid % 64, h0 = tid / 64) owns the pair i
// of heads h0, h0 + 4, ..., so the angle's sine and cosine are computed once per pair and position.
__global__ __launch_bounds__(256) void rope_qkv_kernel(const float* __restrict__ qkv, int64_t T, int Hq, int Hkv,
                                                       double log_base, bf16_t* __restrict__ q,
                                                       bf16_t* __restrict__ k, bf16_t* __restrict__ v) {
  const int64_t t = blockIdx.x;
  const int i = threadIdx.x & 63, h0 = threadIdx.x >> 6;
  const int H = Hq + 2 * Hkv;
  // angle in double, reduced to [-pi, pi] before the fp32 sine and cosine
  const double ang = (double)t * exp(-(double)i / 64.0 * log_base);
  const double red = ang - 6.283185307179586 * rint(ang / 6.283185307179586);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  const float* src = qkv + t * (int64_t)H * kHD;
#pragma unroll 4
  for (int h = h0; h < H; h += 4) {
    float a = src[h * kHD + i], b = src[h * kHD + i + 64];
    bf16_t* dst;
    if (h < Hq + Hkv) {
      const float ra = a * cs - b * sn, rb = a * sn + b * cs;
      a = ra;
      b = rb;
      dst = h < Hq ? q + ((int64_t)h * T + t) * kHD : k + ((int64_t)(h - Hq) * T + t) * kHD;
    } else {
      dst = v + ((int64_t)(h - Hq - Hkv) * T + t) * kHD;
    }
    dst[i] = (bf16_t)f32_to_bf16_rne(a);
    dst[i + 64] = (bf16_t)f32_to_bf16_rne(b);
  }
}

__device__ inline float max4(f32x4_t v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

// Two fp32 values to a bf16 pair (round to nearest even) with the hardware conversion.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ inline uint32_t cvt_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 2^x with the hardware instruction alone. exp2f wraps it in a rescaling that keeps subnormal
// results; here a result below 2^-126 comes out as zero instead, i.e. a key whose weight is under
// 2^-126 of the running maximum's drops out of the sums, far below the bf16 rounding of the weights.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The running maximum of a query moves only when a tile's maximum exceeds it by more than this
// (in units of log2 after scaling): the exponentials then stay below 2^8, and the rescaling of the
// output accumulators, which every lane of the wavefront skips together, is rare after the first tiles.
constexpr float kLazyMax = 8.0f;

// q [Hq][T][128], k, v [Hkv][T][128] bf16 -> o [T][Hq*128] bf16. Grid: (T/64 rounded up) * (Hq/4)
// workgroups of 8 wavefronts: wavefront w takes query head 4 (group) + w/2 and the query positions
// q0 + 32 (w%2) .. +31 (two 16-position blocks).
//
// Two phases. Wavefronts w and w + 4 share a SIMD; those below 4 (phase 0) run each key tile
// straight through (scores, softmax, second product), those from 4 up (phase 1) run half a tile
// behind: between two barriers they finish the previous tile (exponentials, second product) and
// start this one (scores, the running-max check). So while one wavefront of a SIMD is in its
// softmax, the other issues MFMAs. Each phase stages its half of the next tile's rows, at its own
// point between barriers; three LDS buffers keep a tile resident until the later phase is done
// with it (tile n+1 is written while phase 1 may still read tile n-1).
__global__ __launch_bounds__(512, 1) void attention_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                           const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                                           int64_t T, int Hq, int Hkv, float scale_log2) {
  constexpr int QJ = 2;  // 16-position query blocks per wavefront
  constexpr int NB = 3;  // LDS tile buffers
  __shared__ __attribute__((aligned(16))) bf16_t ks[NB][kKB * kKRow];
  __shared__ __attribute__((aligned(16))) bf16_t vs[NB][kKB * kVRow];

  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int phase = wave >> 2;
  const int nqb = (int)((T + kQB - 1) / kQB), nhg = Hq / 4;
  const int qb = nqb - 1 - (int)(blockIdx.x / nhg);  // longest blocks first
  const int hq = (int)(blockIdx.x % nhg) * 4 + (wave >> 1);
  const int hk = hq / (Hq / Hkv);  // the 4 heads of a workgroup share it (group size % 4 == 0)
  const int64_t q0 = (int64_t)qb * kQB;
  const int qw = 32 * (wave & 1);  // first query of this wavefront within the block
  const int nsteps = qb + 1;       // key tiles 0..qb; the last one is the diagonal tile

  // Q fragments as the B operand of S^T = K Q^T: query block j, k-chunk c (32 dims); lane: query
  // q0 + qw + 16 j + li, dims 32 c + 8 g .. +7. Rows past T load the last row (never stored).
  u32x4_t qf[QJ][4];
#pragma unroll
  for (int j = 0; j < QJ; ++j) {
    const int64_t t = min(q0 + qw + 16 * j + li, T - 1);
    const bf16_t* row = q + ((int64_t)hq * T + t) * kHD;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[j][c] = load16(row + 32 * c + 8 * g);
  }

  // K/V tile rows: a phase stages rows 32 phase .. +31 of a tile (16 B per thread per row block)
  const bf16_t* kbase = k + (int64_t)hk * T * kHD;
  const bf16_t* vbase = v + (int64_t)hk * T * kHD;
  const int tid = (wave & 3) * kWave + lane;  // thread index within the phase
  const int lr = 32 * phase + (tid >> 4), lc = (tid & 15) * 8;  // first row and column of this thread
  u32x4_t kreg[2], vreg[2];
  auto gload = [&](int tile) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t key = min((int64_t)tile * kKB + lr + 16 * r, T - 1);  // keys past T are masked
      kreg[r] = load16(kbase + key * kHD + lc);
      vreg[r] = load16(vbase + key * kHD + lc);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      store16(&ks[buf][(lr + 16 * r) * kKRow + lc], kreg[r]);
      store16(&vs[buf][(lr + 16 * r) * kVRow + lc], vreg[r]);
    }
  };
  // LDS-only barrier: the global loads in flight (the next tiles) are not waited for
  auto barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  f32x4_t oacc[8][QJ];  // O^T: dim block d (16 dims) x query block j
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int j = 0; j < QJ; ++j) oacc[d][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // running max per query in exponent units (max * scale_log2; all four lanes of a query agree)
  float mrun[QJ];
  // running sum of the weights per query: a 16-row block of the second product whose A operand
  // is all ones, so every row of it holds sum_k P[k][q] over the bf16 weights that the output
  // itself is formed from (on the matrix cores, instead of 32 dependent additions per step)
  f32x4_t lacc[QJ];
  const u32x4_t ones = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
#pragma unroll
  for (int j = 0; j < QJ; ++j) {
    mrun[j] = 0.f;
    lacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Scores and the running-max step of tile st (in LDS buffer buf): t = exponents of the weights,
  // t = S * scale_log2 - running max. They are formed in place of the scores, and their maximum
  // decides whether the running max must move: being results of arithmetic, they take the max
  // instructions without the NaN-quieting each raw MFMA output would need. The first tile always
  // sets the running max (to its own maximum).
  float t[QJ][4][4];
  auto scores = [&](int st, int buf) {
    // S^T = K Q^T: key block i (A operand rows = keys, from LDS), query block j
    f32x4_t s[4][QJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < QJ; ++j) s[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4_t kf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = load16(&ks[buf][(16 * i + li) * kKRow + 32 * c + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < QJ; ++j) s[i][j] = mfma_bf16(kf[i], qf[j][c], s[i][j]);
    }
    // causal mask on the diagonal tile (k0 == q0), which also holds every key past T
    if (st == nsteps - 1) {
      const int64_t k0 = (int64_t)st * kKB;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < QJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kk = 16 * i + 4 * g + r, qq = qw + 16 * j + li;
            if (kk > qq || k0 + kk >= T) s[i][j][r] = -INFINITY;
          }
    }
    float m[QJ];
    bool grow = st == 0;
#pragma unroll
    for (int j = 0; j < QJ; ++j) {
      m[j] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          t[j][i][r] = fmaf(s[i][j][r], scale_log2, -mrun[j]);
          m[j] = fmaxf(m[j], t[j][i][r]);
        }
      grow |= m[j] > kLazyMax;
    }
    if (__any(grow)) {
#pragma unroll
      for (int j = 0; j < QJ; ++j) {
        float mx = fmaxf(m[j], __shfl_xor(m[j], 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        // the running max moves up by dm (to the tile's max on the first tile)
        const float dm = st == 0 ? mx : fmaxf(mx, 0.f);
        const float alpha = st == 0 ? 0.f : exp2_hw(-dm);
        mrun[j] += dm;
        lacc[j] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][j] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[j][i][r] -= dm;
      }
    }
  };

  // Weights P = 2^t rounded to bf16 and O^T += V^T P^T with the V tile in buffer buf. P^T is the B
  // operand: key chunk kc (32 keys = key blocks 2kc, 2kc+1), lane slots 0-3 = keys 4g..4g+3 of
  // block 2kc, slots 4-7 the same of block 2kc+1. The A operand (dims x keys) comes from
  // transposing reads of the V tile: in each group of 16 lanes, lanes 4a..4a+3 address row a's 16
  // columns and lane i receives column i of the 4 rows, so lane (g, i) gets dim 16 d + i at keys
  // 4g..4g+3 of key blocks 2kc and 2kc+1.
  auto weigh = [&](int buf) {
    u32x4_t pf[2][QJ];
#pragma unroll
    for (int j = 0; j < QJ; ++j) {
      float p[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[i][r] = exp2_hw(t[j][i][r]);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        pf[kc][j] = u32x4_t{cvt_bf16x2(p[2 * kc][0], p[2 * kc][1]), cvt_bf16x2(p[2 * kc][2], p[2 * kc][3]),
                            cvt_bf16x2(p[2 * kc + 1][0], p[2 * kc + 1][1]),
                            cvt_bf16x2(p[2 * kc + 1][2], p[2 * kc + 1][3])};
    }
    typedef __attribute__((ext_vector_type(4))) short v4s;
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const int ta = (lane >> 2) & 3, tc = lane & 3;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16_t* p0 = &vs[buf][(32 * kc + 4 * g + ta) * kVRow + 16 * d + 4 * tc];
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p0));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p0 + 16 * kVRow));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t vf = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
        for (int j = 0; j < QJ; ++j) oacc[d][j] = mfma_bf16(vf, pf[kc][j], oacc[d][j]);
      }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int j = 0; j < QJ; ++j) lacc[j] = mfma_bf16(ones, pf[kc][j], lacc[j]);
  };

  // tile 0 in buffer 0 (both phases' rows)
  gload(0);
  lstore(0);
  // The Q fragments must have landed before the loop. Left alone, the compiler sinks their loads
  // to the loop entry; the wait for them, merged over the back edge, then counts the next tile's
  // K/V prefetch too and stalls every step's first product on it. An empty asm that reads them
  // pins the loads here and makes the wait happen once.
#pragma unroll
  for (int j = 0; j < QJ; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(qf[j][c]));
  barrier();
  // Between barriers st-1 and st, tile st+1 is staged by both phases into buffer (st+1) % 3, whose
  // previous tile st-2 both phases finished before barrier st-1.
  if (phase == 0) {
    int buf = 0;
    for (int st = 0; st < nsteps; ++st) {
      const int nbuf = buf == NB - 1 ? 0 : buf + 1;
      if (st + 1 < nsteps) gload(st + 1);
      scores(st, buf);
      weigh(buf);
      if (st + 1 < nsteps) lstore(nbuf);
      barrier();
      buf = nbuf;
    }
  } else {
    if (nsteps > 1) gload(1);
    int buf = 0, pbuf = NB - 1;
    for (int st = 0; st < nsteps; ++st) {
      const int nbuf = buf == NB - 1 ? 0 : buf + 1;
      if (st > 0) weigh(pbuf);  // tile st-1, staged before barrier st-2
      if (st + 1 < nsteps) {
        lstore(nbuf);
        if (st + 2 < nsteps) gload(st + 2);
      }
      scores(st, buf);
      barrier();
      pbuf = buf;
      buf = nbuf;
    }
    weigh(pbuf);
  }

  // O = O^T / sum, rounded to bf16; lane: query q0 + qw + 16 j + li, dims 16 d + 4 g .. +3
#pragma unroll
  for (int j = 0; j < QJ; ++j) {
    const float inv = 1.0f / lacc[j][0];
    const int64_t t = q0 + qw + 16 * j + li;
    if (t >= T) continue;
    bf16_t* dst = o + t * (int64_t)Hq * kHD + (int64_t)hq * kHD + 4 * g;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<u32x2_t*>(dst + 16 * d) =
          u32x2_t{cvt_bf16x2(oacc[d][j][0] * inv, oacc[d][j][1] * inv),
                  cvt_bf16x2(oacc[d][j][2] * inv, oacc[d][j][3] * inv)};
  }
}

// h[t] += a[t] (fp32), then x[t] = bf16(h[t] / sqrt(mean(h[t]^2) + eps)); one wavefront per row.
// Rows of up to kResNormRegD values stay in registers between the two.
constexpr int kResNormRegD = 4096;
__global__ __launch_bounds__(256) void residual_norm_kernel(float* __restrict__ h, const float* __restrict__ a,
                                                            int64_t T, int d, float eps, bf16_t* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  float* row = h + t * d;
  const float* add = a + t * d;
  float ss = 0.0f;
  auto sum_in = [&](int c) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + c);
    v += *reinterpret_cast<const f32x4_t*>(add + c);
    *reinterpret_cast<f32x4_t*>(row + c) = v;
    return v;
  };
  auto sq = [&](const f32x4_t& v) {
    ss = fmaf(v[0], v[0], ss);
    ss = fmaf(v[1], v[1], ss);
    ss = fmaf(v[2], v[2], ss);
    ss = fmaf(v[3], v[3], ss);
  };
  auto put = [&](int c, const f32x4_t& v, float inv) {
    *reinterpret_cast<u32x2_t*>(x + t * d + c) = u32x2_t{pack_bf16x2(v[0] * inv, v[1] * inv),
                                                         pack_bf16x2(v[2] * inv, v[3] * inv)};
  };
  if (d <= kResNormRegD) {
    // the updated row stays in registers for the scaling (h is read once)
    constexpr int kPer = kResNormRegD / (kWave * 4);
    f32x4_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * 4 + kWave * 4 * i;
      if (c < d) {
        v[i] = sum_in(c);
        sq(v[i]);
      }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * 4 + kWave * 4 * i;
      if (c < d) put(c, v[i], inv);
    }
    return;
  }
  for (int c = lane * 4; c < d; c += kWave * 4) sq(sum_in(c));
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane * 4; c < d; c += kWave * 4) put(c, *reinterpret_cast<const f32x4_t*>(row + c), inv);
}

__global__ void set_offsets_kernel(int32_t* off, int32_t T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

}  // namespace

void launch_rope_qkv(const float* qkv, int64_t T, int Hq, int Hkv, double base, void* q, void* k, void* v,
                     hipStream_t s) {
  launch_kernel(rope_qkv_kernel, dim3((unsigned)T), dim3(256), 0, s, qkv, T, Hq, Hkv, std::log(base),
                static_cast<bf16_t*>(q), static_cast<bf16_t*>(k), static_cast<bf16_t*>(v));
}

void launch_attention(const void* q, const void* k, const void* v, void* o, int64_t T, int Hq, int Hkv,
                      hipStream_t s) {
  const int64_t nqb = (T + kQB - 1) / kQB;
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kHD));
  launch_kernel(attention_kernel, dim3((unsigned)(nqb * (Hq / 4))), dim3(512), 0, s, static_cast<const bf16_t*>(q),
                static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), static_cast<bf16_t*>(o), T, Hq, Hkv,
                scale_log2);
}

void launch_residual_norm(float* h, const float* a, int64_t T, int d, float eps, void* x, hipStream_t s) {
  launch_kernel(residual_norm_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, h, a, T, d, eps,
                static_cast<bf16_t*>(x));
}

void launch_set_offsets(int32_t* off, int64_t T, hipStream_t s) {
  launch_kernel(set_offsets_kernel, dim3(1), dim3(64), 0, s, off, (int32_t)T);
}

}  // namespace moe
