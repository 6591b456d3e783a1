/*
 * Seeded synthetic inputs: counter-based random tensors for the decode-step
 * workloads (weights, scales, prompts).  This file holds no arithmetic of the
 * decoder itself; it only turns (seed, stream, index) into numbers.
 *
 * Generator: SplitMix64 finaliser (Steele, Lea, Flood 2014; the public-domain
 * constants published by Vigna) applied to seed ^ stream-hash + index * golden
 * ratio.  Every element depends only on (seed, stream, index), so the output is
 * identical for any thread count and any generation order.
 *
 * Normal deviates: Box-Muller on two uniforms drawn at indices 2j and 2j+1;
 * element 2j takes the cosine branch and 2j+1 the sine branch.
 * bf16 outputs are rounded to nearest-even from fp32.
 */
#include <stdint.h>
#include <math.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

/* uniform in (0, 1]: never 0, so log() below is finite */
static inline double unit_open0(uint64_t x) {
  return ((double)(x >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf/nan: not produced here */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * 0xD1B54A32D192ED03ULL ^ mix64(stream + 0x632BE59BD9B4E019ULL));
}

/* out[i] = bf16(mean + std * N(0,1)), i in [0, n) */
void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t key, float mean, float std) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (n + 1) / 2; ++j) {
    double u1 = unit_open0(draw(key, 2 * (uint64_t)j));
    double u2 = unit_open0(draw(key, 2 * (uint64_t)j + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = two_pi * u2;
    int64_t i0 = 2 * j, i1 = 2 * j + 1;
    out[i0] = f32_to_bf16_rne((float)(mean + std * r * cos(a)));
    if (i1 < n) out[i1] = f32_to_bf16_rne((float)(mean + std * r * sin(a)));
  }
}

/* out[i] = bf16(U(lo, hi)) */
void synth_uniform_bf16(uint16_t* out, int64_t n, uint64_t key, float lo, float hi) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = unit_open0(draw(key, (uint64_t)i)) - 0x1p-53; /* [0, 1) */
    out[i] = f32_to_bf16_rne((float)(lo + (hi - lo) * u));
  }
}

/* n 32-bit words, each eight independent uniform 4-bit codes (all 32 bits uniform) */
void synth_bits32(uint32_t* out, int64_t n, uint64_t key) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint32_t)(draw(key, (uint64_t)i) >> 32);
}

/* token ids uniform in [0, vocab) */
void synth_tokens(int32_t* out, int64_t n, uint64_t key, int32_t vocab) {
  for (int64_t i = 0; i < n; ++i) {
    uint64_t x = draw(key, (uint64_t)i);
    out[i] = (int32_t)((x >> 32) % (uint64_t)vocab);
  }
}
