/*
 * Seeded, counter-based synthetic tensors shared by the CPU oracle and the GPU path.
 *
 * This module holds none of the method's arithmetic. It only draws numbers:
 *   value(seed, tag, i) is a pure function of its arguments, so any row of any tensor can be
 *   regenerated on its own (the oracle regenerates only the query rows it samples), and the
 *   bytes do not depend on thread count or order.
 *
 * Definitions (all published generators, restated here):
 *   - mix64: the SplitMix64 output function of Steele, Lea and Flood, "Fast splittable
 *     pseudorandom number generators", OOPSLA 2014 (constants as in that generator).
 *   - stream(seed, tag): base = mix64(seed * GAMMA ^ mix64(tag + 1)); word i = mix64(base + (i + 1) * GAMMA).
 *   - uniform double in [0, 1): top 53 bits of the word times 2^-53.
 *   - standard normal: Box and Muller (1958). Element i uses the pair p = i / 2:
 *     u1 = U(2p), u2 = U(2p + 1), r = sqrt(-2 ln(1 - u1)), z = r cos(2 pi u2) for even i,
 *     r sin(2 pi u2) for odd i, computed in double.
 *   - bf16: the float32 value (double rounded to float) rounded to the upper 16 bits with
 *     round-to-nearest-even.
 *   - row RMS normalisation (input preparation for latent rows): x / sqrt(mean(x^2) + eps) in
 *     float32, rounded to bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define TG_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t tg_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t tg_base(uint64_t seed, uint64_t tag) {
  return tg_mix64(seed * TG_GAMMA ^ tg_mix64(tag + 1));
}

static inline uint64_t tg_word(uint64_t base, uint64_t i) { return tg_mix64(base + (i + 1) * TG_GAMMA); }

static inline double tg_u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

static inline uint16_t tg_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static inline float tg_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static inline double tg_normal_at(uint64_t base, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = tg_u01(tg_word(base, 2 * p));
  double u2 = tg_u01(tg_word(base, 2 * p + 1));
  double r = sqrt(-2.0 * log(1.0 - u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* out[j] = bf16(scale * N(0,1)[start + j]) for j < n. */
void tg_normal_bf16(uint64_t seed, uint64_t tag, int64_t start, int64_t n, double scale, uint16_t* out) {
  uint64_t base = tg_base(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = tg_bf16_rne((float)(scale * tg_normal_at(base, (uint64_t)(start + j))));
}

/* out[j] = bf16(scale * U[0,1)[start + j]) for j < n. */
void tg_uniform_bf16(uint64_t seed, uint64_t tag, int64_t start, int64_t n, double scale, uint16_t* out) {
  uint64_t base = tg_base(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = tg_bf16_rne((float)(scale * tg_u01(tg_word(base, (uint64_t)(start + j)))));
}

/* out[j] = lo + floor(U[0,1)[j] * (hi - lo + 1)) for j < n: integers uniform on [lo, hi]. */
void tg_uniform_int(uint64_t seed, uint64_t tag, int64_t n, int64_t lo, int64_t hi, int64_t* out) {
  uint64_t base = tg_base(seed, tag);
  for (int64_t j = 0; j < n; ++j) {
    int64_t v = lo + (int64_t)(tg_u01(tg_word(base, (uint64_t)j)) * (double)(hi - lo + 1));
    out[j] = v > hi ? hi : v;
  }
}

/* In place: each of n_rows rows of dim bf16 values becomes bf16(x / sqrt(mean(x^2) + eps)), float32 math. */
void tg_rms_rows_bf16(uint16_t* rows, int64_t n_rows, int64_t dim, float eps) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    uint16_t* x = rows + r * dim;
    float ss = 0.0f;
    for (int64_t i = 0; i < dim; ++i) {
      float v = tg_bf16_to_f32(x[i]);
      ss += v * v;
    }
    float inv = 1.0f / sqrtf(ss / (float)dim + eps);
    for (int64_t i = 0; i < dim; ++i) x[i] = tg_bf16_rne(tg_bf16_to_f32(x[i]) * inv);
  }
}

/* Raw words, for the generator's own self-test. */
void tg_words(uint64_t seed, uint64_t tag, int64_t start, int64_t n, uint64_t* out) {
  uint64_t base = tg_base(seed, tag);
  for (int64_t j = 0; j < n; ++j) out[j] = tg_word(base, (uint64_t)(start + j));
}

uint64_t tg_mix64_public(uint64_t z) { return tg_mix64(z); }
