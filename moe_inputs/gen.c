/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module produces the input tensors that both the HIP library and the
 * CPU oracle consume. It holds none of the mixture-of-experts arithmetic:
 * it only turns (key, element index) into a Gaussian sample and stores it in
 * the requested storage type.
 *
 * Definitions (each element is independent of every other, so any slice of a
 * tensor can be regenerated on its own and the result does not depend on the
 * thread count):
 *   mix(z)        SplitMix64 output function (Steele, Lea and Flood, "Fast
 *                 splittable pseudorandom number generators", OOPSLA 2014).
 *   r_j           mix(key + (2i + j + 1) * 0x9E3779B97F4A7C15), j = 0, 1.
 *   u1            ((r_0 >> 11) + 0.5) * 2^-53        in (0, 1)
 *   u2            (r_1 >> 11) * 2^-53                in [0, 1)
 *   n_i           sqrt(-2 ln u1) * cos(2 pi u2)      (Box and Muller, 1958)
 *   value_i       sigma * n_i in double, rounded to fp32 (round to nearest
 *                 even); for bf16 storage the fp32 value is then rounded to
 *                 bf16 (round to nearest even).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t gen_mix64(uint64_t z) { return mix64(z); }

/* Key of tensor `tensor` in layer `layer` of the workload seeded by `seed`. */
uint64_t gen_key(uint64_t seed, uint64_t layer, uint64_t tensor) {
  uint64_t k = mix64(seed + GOLDEN);
  k = mix64(k ^ (layer * 0xD1B54A32D192ED03ULL + 0x2545F4914F6CDD1DULL));
  k = mix64(k ^ (tensor * 0x8CB92BA72F3D8DD7ULL + 0x632BE59BD9B4E019ULL));
  return k;
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t r0 = mix64(key + (2 * i + 1) * GOLDEN);
  uint64_t r1 = mix64(key + (2 * i + 2) * GOLDEN);
  double u1 = ((double)(r0 >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  double u2 = (double)(r1 >> 11) * (1.0 / 9007199254740992.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40); /* NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float* out) {
  #pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = (float)(sigma * normal_at(key, start + (uint64_t)j));
}

void gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t* out) {
  #pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = f32_to_bf16_rne((float)(sigma * normal_at(key, start + (uint64_t)j)));
}

/* Uniform integers in [0, m) from the same counter stream (used for synthetic
 * routings and token samples): floor(u * m) with u = (r >> 11) * 2^-53. */
void gen_uniform_int(uint64_t key, uint64_t start, uint64_t n, uint64_t m, int64_t* out) {
  for (uint64_t j = 0; j < n; ++j) {
    uint64_t r = mix64(key + (start + j + 1) * GOLDEN);
    double u = (double)(r >> 11) * (1.0 / 9007199254740992.0);
    uint64_t v = (uint64_t)(u * (double)m);
    out[j] = (int64_t)(v < m ? v : m - 1);
  }
}
