/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no arithmetic of the decoder transition. It only turns
 * (seed, stream, element index) into numbers, so that the CPU oracle and the
 * GPU library can be fed bit-identical weights, encoder representations,
 * encoder memory, sequence lengths and sampling uniforms without either side
 * generating them itself.
 *
 * Draw for element i of stream `stream` under `seed`:
 *   key = mix(mix(seed + G) ^ (stream * C2))
 *   h   = mix(key + (i + 1) * G)
 * where mix() is the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) and
 * G = 0x9E3779B97F4A7C15 is its Weyl increment.
 *
 * "Normal" values are an Irwin-Hall(4) stand-in for N(0,1): the four 16-bit
 * lanes of h are summed as integers, centred and scaled to unit variance in
 * two correctly rounded fp32 multiplications (support +-2*sqrt(3)). No
 * transcendental function is involved, so any implementation of these few
 * integer steps reproduces the values exactly.
 */
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define STREAM_MUL 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ (stream * STREAM_MUL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN);
}

/* unit-variance Irwin-Hall(4) value from one 64-bit draw */
static inline float ih4(uint64_t h) {
  const float scale = (float)(1.7320508075688772 / 131072.0); /* sqrt(3)/2^17 */
  int32_t s = (int32_t)(h & 0xffffu) + (int32_t)((h >> 16) & 0xffffu) +
              (int32_t)((h >> 32) & 0xffffu) + (int32_t)(h >> 48);
  float x = (float)(2 * s - 4 * 65535); /* exact: |x| < 2^19 */
  return x * scale;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out_kind: 0 = fp32, 1 = bf16 bit patterns (round to nearest even).
 * value = offset + sigma * ih4(h), each step one fp32 rounding. */
void synth_normal(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                  float sigma, float offset, int out_kind, void* out,
                  int nthreads) {
  const uint64_t key = stream_key(seed, stream);
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    float v = ih4(draw(key, start + (uint64_t)j)) * sigma;
    v = v + offset;
    if (out_kind == 0)
      ((float*)out)[j] = v;
    else
      ((uint16_t*)out)[j] = f32_to_bf16_rne(v);
  }
}

/* integers uniform on [lo, hi] (modulo reduction of the 64-bit draw) */
void synth_uniform_int(uint64_t seed, uint64_t stream, uint64_t start,
                       uint64_t n, int64_t lo, int64_t hi, int32_t* out) {
  const uint64_t key = stream_key(seed, stream);
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (uint64_t j = 0; j < n; ++j)
    out[j] = (int32_t)(lo + (int64_t)(draw(key, start + j) % span));
}

/* floats uniform on [0, 1): top 24 bits of the draw times 2^-24 (exact) */
void synth_uniform01(uint64_t seed, uint64_t stream, uint64_t start,
                     uint64_t n, float* out) {
  const uint64_t key = stream_key(seed, stream);
  for (uint64_t j = 0; j < n; ++j)
    out[j] = (float)(draw(key, start + j) >> 40) * (1.0f / 16777216.0f);
}
