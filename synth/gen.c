/*
 * Seeded synthetic tensors for the MoE layer workloads.
 *
 * This file holds no arithmetic of the MoE method itself: it only turns a
 * (seed, element index) pair into a normally distributed number, rounded to
 * the storage type.  Both the GPU path's tests and the CPU oracle consume the
 * bytes it writes, so the two sides always see identical inputs.
 *
 * Generator (counter-based, so any element can be produced independently and
 * the work splits over threads without changing a single output bit):
 *   mix(z)  : the SplitMix64 finaliser (Steele, Lea and Flood, "Fast
 *             splittable pseudorandom number generators", OOPSLA 2014):
 *             z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *             z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
 *   draw(s, c) = mix(s + (c + 1) * 0x9E3779B97F4A7C15), i.e. the c-th output
 *             of a SplitMix64 stream started at state s.
 *   element i of a stream with state s:
 *             u1 = ((draw(s, 2i) >> 11) + 1) * 2^-53      in (0, 1]
 *             u2 =  (draw(s, 2i+1) >> 11)    * 2^-53      in [0, 1)
 *             z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, cosine branch)
 *             v  = mean + std * z, in double, then rounded to fp32
 *             (round to nearest even), then for bf16 storage rounded again
 *             from the fp32 bits to bf16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t sm_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

static inline uint64_t sm_draw(uint64_t state, uint64_t counter) {
  return sm_mix(state + (counter + 1ULL) * 0x9E3779B97F4A7C15ULL);
}

static inline double normal_at(uint64_t state, uint64_t i) {
  const double two_m53 = 1.0 / 9007199254740992.0; /* 2^-53 */
  double u1 = (double)((sm_draw(state, 2 * i) >> 11) + 1ULL) * two_m53;
  double u2 = (double)(sm_draw(state, 2 * i + 1) >> 11) * two_m53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite here). */
static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t lsb = (v.u >> 16) & 1u;
  uint32_t rounded = v.u + 0x7FFFu + lsb;
  return (uint16_t)(rounded >> 16);
}

/* The stream state of a tensor is mix(seed) so that nearby seeds give
 * unrelated streams. */
uint64_t synth_stream_state(uint64_t seed) { return sm_mix(seed); }

void synth_normal_f32(uint64_t seed, int64_t first, int64_t n, double mean,
                      double std, float* out) {
  uint64_t st = sm_mix(seed);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(mean + std * normal_at(st, (uint64_t)(first + i)));
}

void synth_normal_bf16(uint64_t seed, int64_t first, int64_t n, double mean,
                       double std, uint16_t* out) {
  uint64_t st = sm_mix(seed);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne(
        (float)(mean + std * normal_at(st, (uint64_t)(first + i))));
}
