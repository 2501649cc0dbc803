/*
 * Seeded, counter-based synthetic input generator.
 *
 * Shared by the CPU oracle's tests and by the GPU path's tests and benchmark.
 * It holds none of the attention method's arithmetic: it only draws numbers.
 *
 * Definitions (stable; every value is a pure function of (seed, stream, counter)):
 *   mix64(z)      = the SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable
 *                   pseudorandom number generators", OOPSLA 2014):
 *                     z ^= z >> 30; z *= 0xbf58476d1ce4e5b9;
 *                     z ^= z >> 27; z *= 0x94d049bb133111eb; z ^= z >> 31
 *   key(s, st)    = mix64(mix64(s) ^ (st * 0x9e3779b97f4a7c15))
 *   u64(s,st,c)   = mix64(key(s, st) + (c + 1) * 0x9e3779b97f4a7c15)
 *   normal(s,st,i)= Box-Muller on u1 = ((u64(s,st,2i) >> 11) + 1) * 2^-53  (0, 1]
 *                                  u2 =  (u64(s,st,2i+1) >> 11)    * 2^-53  [0, 1)
 *                   z = sqrt(-2 ln u1) * cos(2 pi u2), evaluated in double, then
 *                   rounded once to float (round-to-nearest-even).
 *   bf16 storage  = float -> bf16 by round-to-nearest-even on the bit pattern
 *                   (inputs are finite by construction).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xbf58476d1ce4e5b9ULL;
  z ^= z >> 27;
  z *= 0x94d049bb133111ebULL;
  z ^= z >> 31;
  return z;
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * 0x9e3779b97f4a7c15ULL));
}

static inline uint64_t draw_u64(uint64_t key, uint64_t counter) {
  return mix64(key + (counter + 1) * 0x9e3779b97f4a7c15ULL);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t counter) {
  return draw_u64(stream_key(seed, stream), counter);
}

static inline float draw_normal(uint64_t key, uint64_t i) {
  const double two_m53 = 1.0 / 9007199254740992.0;
  double u1 = (double)((draw_u64(key, 2 * i) >> 11) + 1) * two_m53;
  double u2 = (double)(draw_u64(key, 2 * i + 1) >> 11) * two_m53;
  double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
  return (float)z;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[k] = normal(seed, stream, offset + k) for k in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      float* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) out[k] = draw_normal(key, offset + (uint64_t)k);
}

/* Same draws as synth_normal_f32, times `mult`, stored as bf16 bit patterns.
 * `mult` is applied in float before storage rounding (callers pass powers of 2
 * or 1, so the product is exact). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       float mult, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k)
    out[k] = f32_to_bf16_rne(draw_normal(key, offset + (uint64_t)k) * mult);
}

/* Seeded Fisher-Yates permutation of [0, n): draw j uniformly in [0, i] from
 * counter (n - 1 - i) for i = n-1 .. 1 (modulo reduction; the bias is far below
 * anything a synthetic input cares about). */
void synth_permutation(uint64_t seed, uint64_t stream, int64_t n, int32_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    uint64_t j = draw_u64(key, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* k distinct values from [0, n), in draw order: the first k slots of a partial
 * Fisher-Yates shuffle driven by the same counters as synth_permutation.
 * `scratch` holds n int32. */
void synth_sample(uint64_t seed, uint64_t stream, int64_t n, int64_t k,
                  int32_t* scratch, int32_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) scratch[i] = (int32_t)i;
  for (int64_t i = 0; i < k; ++i) {
    uint64_t j = (uint64_t)i + draw_u64(key, (uint64_t)i) % (uint64_t)(n - i);
    int32_t t = scratch[i];
    scratch[i] = scratch[j];
    scratch[j] = t;
    out[i] = scratch[i];
  }
}
