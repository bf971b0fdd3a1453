/*
 * Seeded synthetic input generator shared by the oracle tests, the GPU tests and the bench.
 *
 * It holds none of the frame step's arithmetic: it only turns (master seed, stream name,
 * element index) into numbers.  Every value is addressable by its index (counter-based), so the
 * result does not depend on the thread count or on how a tensor is chunked.
 *
 *   key(seed, name)  = mix64(mix64(seed) ^ fnv1a64(name))
 *   raw(key, i)      = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)      -- the i-th SplitMix64 output
 *   u(key, i)        = ((raw >> 11) + 1) * 2^-53                       -- uniform on (0, 1]
 *   normal pair j    = Box-Muller on u(key, 2j), u(key, 2j + 1), in double:
 *                      r = sqrt(-2 ln u1); z[2j] = r cos(2 pi u2); z[2j+1] = r sin(2 pi u2)
 *   weight value     = (float)(std * z)        (then optionally bf16 round-to-nearest-even)
 *   token            = floor(u * n)            (uniform on {0 .. n-1})
 *
 * mix64 is the SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014); FNV-1a 64 is the Fowler-Noll-Vo hash; Box-Muller is the 1958
 * transform.  Built with gcc -O2 -fopenmp (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t fnv1a64(const char *s) {
  uint64_t h = 0xCBF29CE484222325ULL;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001B3ULL;
  }
  return h;
}

uint64_t rqgen_key(uint64_t seed, const char *name) { return mix64(mix64(seed) ^ fnv1a64(name)); }

static inline uint64_t raw_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double u01_at(uint64_t key, uint64_t i) {
  return (double)((raw_at(key, i) >> 11) + 1) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}


/* One Box-Muller pair: z[2j] and z[2j+1] of stream `key`. */
static inline void normal_pair(uint64_t key, uint64_t j, double *z0, double *z1) {
  const double u1 = u01_at(key, 2 * j), u2 = u01_at(key, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925 * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
}

/* Fill out[0..n) with N(0, std^2) values of stream `key`, elements [start, start + n).
   Iterates over Box-Muller pairs; each pair is computed once. */
#define RQGEN_NORMAL_FILL(STORE)                                                   \
  const uint64_t j_lo = start >> 1, j_hi = (start + (uint64_t)n + 1) >> 1;        \
  _Pragma("omp parallel for schedule(static)")                                    \
  for (int64_t jj = (int64_t)j_lo; jj < (int64_t)j_hi; ++jj) {                    \
    double z[2];                                                                  \
    normal_pair(key, (uint64_t)jj, &z[0], &z[1]);                                 \
    for (int t = 0; t < 2; ++t) {                                                 \
      const uint64_t idx = 2 * (uint64_t)jj + (uint64_t)t;                        \
      if (idx < start || idx >= start + (uint64_t)n) continue;                    \
      STORE(out[idx - start], (float)(std * z[t]));                               \
    }                                                                             \
  }

#define STORE_F32(dst, v) (dst) = (v)
#define STORE_BF16(dst, v) (dst) = f32_to_bf16_rne(v)

void rqgen_normal_f32(uint64_t key, uint64_t start, int64_t n, double std, float *out) {
  RQGEN_NORMAL_FILL(STORE_F32)
}

/* Same values as rqgen_normal_f32, each rounded to bfloat16 (round-to-nearest-even), as raw bits. */
void rqgen_normal_bf16(uint64_t key, uint64_t start, int64_t n, double std, uint16_t *out) {
  RQGEN_NORMAL_FILL(STORE_BF16)
}

/* Uniform integers in [0, card): element i of stream `key`. */
void rqgen_uniform_int(uint64_t key, uint64_t start, int64_t n, int64_t card, int32_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t v = (int64_t)floor(u01_at(key, start + (uint64_t)i) * (double)card);
    if (v >= card) v = card - 1; /* u = 1 exactly */
    out[i] = (int32_t)v;
  }
}

/* Uniform doubles on (0, 1]: element i of stream `key` (exposed for tests of the generator). */
void rqgen_uniform_f64(uint64_t key, uint64_t start, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = u01_at(key, start + (uint64_t)i);
}

/* bf16 round-to-nearest-even of an f32 array (input preparation for bf16-stored configs). */
void rqgen_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
