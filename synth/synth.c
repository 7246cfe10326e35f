/*
 * Seeded synthetic inputs for the ternary group-scaled matmul.
 *
 * This module only draws random numbers. It knows nothing about packing,
 * scales, rotation or matrix products: it hands out ternary codes in
 * {-1, 0, +1}, standard normal doubles and random signs. The same bytes it
 * produces feed both the GPU library and the CPU oracle.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014), used in counter form:
 * value i of a stream is mix64(base + (i + 1) * GAMMA), where base is
 * derived from (seed, stream id). Any element can be computed on its own,
 * so the fills below split over threads without changing a single value.
 * Normals come from the Box-Muller transform on two uniforms per pair.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ mix64(stream + 0x1B873593ULL);
}

/* uniform double in [0, 1) with 53 random bits */
static inline double uniform(uint64_t base, uint64_t i) {
  return (double)(mix64(base + (i + 1) * GAMMA) >> 11) * (1.0 / 9007199254740992.0);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return mix64(stream_base(seed, stream) + (i + 1) * GAMMA);
}

/* codes: u < p_neg -> -1, u < p_neg + p_zero -> 0, otherwise +1 */
void synth_trits(uint64_t seed, uint64_t stream, int64_t count, double p_zero, int8_t* out) {
  const uint64_t base = stream_base(seed, stream);
  const double p_neg = 0.5 * (1.0 - p_zero);
  const double p_le0 = p_neg + p_zero;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    double u = uniform(base, (uint64_t)i);
    out[i] = (int8_t)(u < p_neg ? -1 : (u < p_le0 ? 0 : 1));
  }
}

/* standard normals via Box-Muller: element 2j uses cos, 2j+1 uses sin */
void synth_normal(uint64_t seed, uint64_t stream, int64_t count, double* out) {
  const uint64_t base = stream_base(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (count + 1) / 2; ++j) {
    double u1 = uniform(base, (uint64_t)(2 * j));
    double u2 = uniform(base, (uint64_t)(2 * j + 1));
    double r = sqrt(-2.0 * log(1.0 - u1)); /* 1-u1 in (0, 1] */
    double a = two_pi * u2;
    out[2 * j] = r * cos(a);
    if (2 * j + 1 < count) out[2 * j + 1] = r * sin(a);
  }
}

/* random signs in {-1, +1}, one bit of each draw */
void synth_signs(uint64_t seed, uint64_t stream, int64_t count, int8_t* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    out[i] = (int8_t)((mix64(base + ((uint64_t)i + 1) * GAMMA) >> 63) ? -1 : 1);
  }
}
