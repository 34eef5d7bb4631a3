/*
 * Seeded, counter-based input generator (host side).
 *
 * This file is input plumbing only: it holds none of the MoE sublayer's
 * arithmetic. Both the CPU oracle's inputs and the GPU path's inputs are drawn
 * from the same definition; the device twin lives in synth_gpu.hip and is
 * written separately from the same definition below.
 *
 * Definition (SplitMix64, Steele/Lea/Flood 2014, as published with
 * java.util.SplittableRandom):
 *   mix(z)  = z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *             z *= 0x94D049BB133111EB; z ^= z>>31
 *   base(seed, tensor) = mix(mix(seed) + tensor)
 *   draw(seed, tensor, i) = mix(base + (i+1) * 0x9E3779B97F4A7C15)
 * i.e. element i of a tensor is the (i+1)-th output of a SplitMix64 stream
 * whose state starts at base. Any element can be drawn on its own, so the
 * values do not depend on how the work is split across threads.
 *
 *   uniform(i) = (draw(i) >> 11) * 2^-53                       in [0, 1)
 *   normal(i)  : Box-Muller on the pair p = i >> 1:
 *                u1 = ((draw(2p) >> 11) + 1) * 2^-53            in (0, 1]
 *                u2 = (draw(2p+1) >> 11) * 2^-53
 *                r = sqrt(-2 ln u1), t = 2 pi u2
 *                even i -> r cos t, odd i -> r sin t
 * Values are formed in double as mean + std * normal (or lo + (hi-lo) * u),
 * rounded once to float (round to nearest even), and, for BF16 outputs,
 * that float is rounded to BF16 with round to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ull

static uint64_t synth_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

static uint64_t synth_base(uint64_t seed, uint64_t tensor) {
  return synth_mix(synth_mix(seed) + tensor);
}

static uint64_t synth_draw(uint64_t base, uint64_t i) {
  return synth_mix(base + (i + 1ull) * SYNTH_GOLDEN);
}

static double synth_uniform_at(uint64_t base, uint64_t i) {
  return (double)(synth_draw(base, i) >> 11) * 0x1.0p-53;
}

static double synth_normal_at(uint64_t base, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = (double)((synth_draw(base, 2 * p) >> 11) + 1ull) * 0x1.0p-53;
  double u2 = (double)(synth_draw(base, 2 * p + 1) >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static uint16_t synth_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet nan */
    return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                      double mean, double stdv, float* out) {
  uint64_t b = synth_base(seed, tensor);
  for (int64_t j = 0; j < n; ++j)
    out[j] = (float)(mean + stdv * synth_normal_at(b, start + (uint64_t)j));
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                       double mean, double stdv, uint16_t* out) {
  uint64_t b = synth_base(seed, tensor);
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_f32_to_bf16((float)(mean + stdv * synth_normal_at(b, start + (uint64_t)j)));
}

void synth_uniform_f32(uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                       double lo, double hi, float* out) {
  uint64_t b = synth_base(seed, tensor);
  for (int64_t j = 0; j < n; ++j)
    out[j] = (float)(lo + (hi - lo) * synth_uniform_at(b, start + (uint64_t)j));
}

void synth_uniform_bf16(uint64_t seed, uint64_t tensor, uint64_t start, int64_t n,
                        double lo, double hi, uint16_t* out) {
  uint64_t b = synth_base(seed, tensor);
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_f32_to_bf16((float)(lo + (hi - lo) * synth_uniform_at(b, start + (uint64_t)j)));
}

/* raw 64-bit draws, for tests of the generator itself */
void synth_raw_u64(uint64_t seed, uint64_t tensor, uint64_t start, int64_t n, uint64_t* out) {
  uint64_t b = synth_base(seed, tensor);
  for (int64_t j = 0; j < n; ++j) out[j] = synth_draw(b, start + (uint64_t)j);
}
