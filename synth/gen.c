/*
 * gen.c -- seeded synthetic inputs shared by the tests, the bench and the smoke check.
 * It holds none of the attention arithmetic: only a counter-based generator.
 *
 * Generator (published definitions):
 *   splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 *   OOPSLA 2014; the finaliser constants as in Vigna's public-domain splitmix64.c):
 *     x_n = seed + (n + 1) * 0x9E3779B97F4A7C15 (mod 2^64), u64_n = mix(x_n);
 *   uniform double u_n = (u64_n >> 11) * 2^-53 in [0, 1);
 *   Box-Muller (1958) on the pair (u_{2k}, u_{2k+1}):
 *     r = sqrt(-2 ln(1 - u_{2k})), element 2k = r cos(2 pi u_{2k+1}), element 2k+1 = r sin(...);
 *   fp32 values are the fp64 result rounded to nearest even (a C cast); bf16 values are the
 *   fp32 values rounded to nearest even on the top 16 bits.
 * Element n of a stream depends only on (seed, n), so any slice can be generated alone.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static double sm_uniform(uint64_t seed, uint64_t n) {
  uint64_t x = seed + (n + 1) * 0x9E3779B97F4A7C15ULL;
  return (double)(sm_mix(x) >> 11) * (1.0 / 9007199254740992.0);
}

static double sm_normal(uint64_t seed, uint64_t e) {
  uint64_t k = e >> 1;
  double u1 = sm_uniform(seed, 2 * k), u2 = sm_uniform(seed, 2 * k + 1);
  double r = sqrt(-2.0 * log(1.0 - u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (e & 1) ? r * sin(a) : r * cos(a);
}

void synth_uniform_f64(uint64_t seed, int64_t start, int64_t n, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sm_uniform(seed, (uint64_t)(start + i));
}

void synth_normal_f32(uint64_t seed, int64_t start, int64_t n, float mean, float std, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)((double)mean + (double)std * sm_normal(seed, (uint64_t)(start + i)));
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet). */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
      out[i] = (uint16_t)((u >> 16) | 0x0040u);
    } else {
      uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
      out[i] = (uint16_t)((u + bias) >> 16);
    }
  }
}

/* Bernoulli(p) mask of 0 / -inf, element n of stream seed. */
void synth_neg_inf_mask_f32(uint64_t seed, int64_t start, int64_t n, double p, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = sm_uniform(seed, (uint64_t)(start + i)) < p ? -INFINITY : 0.0f;
}
