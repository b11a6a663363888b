/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU path.
 *
 * This module holds no arithmetic of the decode step itself.  It only draws
 * numbers: every value is a pure function of (seed, tensor id, element index),
 * so any slice of any tensor can be regenerated anywhere, in any order, by any
 * number of threads.
 *
 *   splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014; constants as published by Vigna) turns a 64-bit
 *   counter into a 64-bit hash.  A normal deviate is one Box-Muller draw
 *   (Box and Muller 1958) from two such hashes.
 *
 * Weight recipe for the int4 configuration: symmetric quantisation over
 * groups of 64 consecutive input elements of one output row, scale
 * s = bf16(absmax / 7), code q = clamp(rne(w / s), -8, 7), stored as the
 * unsigned nibble q + 8, element 2j in the low nibble of byte j.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid) {
  return splitmix64(seed ^ splitmix64(tid ^ 0xD1B54A32D192ED03ull));
}

/* Standard normal deviate number i of the stream `key` (single-precision Box-Muller). */
static inline float normal_at(uint64_t key, uint64_t i) {
  uint64_t h1 = splitmix64(key + 2 * i), h2 = splitmix64(key + 2 * i + 1);
  float u1 = ((float)(h1 >> 40) + 1.0f) * (1.0f / 16777216.0f); /* (0, 1] */
  float u2 = (float)(h2 >> 40) * (1.0f / 16777216.0f);          /* [0, 1) */
  return sqrtf(-2.0f * logf(u1)) * cosf(6.2831853f * u2);
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint64_t synth_splitmix64(uint64_t x) { return splitmix64(x); }

/* out[i] = fp32(sigma * N_i), elements [off, off + n) of the stream. */
void synth_normal_f32(uint64_t seed, uint64_t tid, double sigma, int64_t off, int64_t n, float* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)sigma * normal_at(key, (uint64_t)(off + i));
}

/* out[i] = bf16(fp32(sigma * N_i)) as raw bits. */
void synth_normal_bf16(uint64_t seed, uint64_t tid, double sigma, int64_t off, int64_t n, uint16_t* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16((float)sigma * normal_at(key, (uint64_t)(off + i)));
}

/*
 * Rows [row0, row0 + nrows) of a [rows][cols] weight drawn as fp32(sigma * N)
 * (element index r * cols + c of the stream) and quantised to int4 group-64.
 * codes: [nrows][cols / 2] bytes, scales: [nrows][cols / 64] bf16 bits.
 */
void synth_int4g64(uint64_t seed, uint64_t tid, double sigma, int64_t cols, int64_t row0, int64_t nrows,
                   uint8_t* codes, uint16_t* scales) {
  uint64_t key = stream_key(seed, tid);
  int64_t ngroups = cols / 64;
#pragma omp parallel for schedule(static)
  for (int64_t rg = 0; rg < nrows * ngroups; ++rg) {
    int64_t r = rg / ngroups, g = rg % ngroups;
    float w[64];
    float amax = 0.0f;
    uint64_t base = (uint64_t)((row0 + r) * cols + g * 64);
    for (int j = 0; j < 64; ++j) {
      w[j] = (float)sigma * normal_at(key, base + (uint64_t)j);
      float a = fabsf(w[j]);
      if (a > amax) amax = a;
    }
    uint16_t sb = f32_to_bf16(amax / 7.0f);
    float s = bf16_to_f32(sb);
    scales[r * ngroups + g] = sb;
    uint8_t* dst = codes + r * (cols / 2) + g * 32;
    for (int j = 0; j < 64; j += 2) {
      int q0 = 0, q1 = 0;
      if (s != 0.0f) {
        q0 = (int)rintf(w[j] / s);
        q1 = (int)rintf(w[j + 1] / s);
        q0 = q0 < -8 ? -8 : (q0 > 7 ? 7 : q0);
        q1 = q1 < -8 ? -8 : (q1 > 7 ? 7 : q1);
      }
      dst[j / 2] = (uint8_t)((q0 + 8) | ((q1 + 8) << 4));
    }
  }
}

/* out[i] uniform integer in [lo, hi] (multiply-shift range reduction). */
void synth_uniform_int(uint64_t seed, uint64_t tid, int64_t lo, int64_t hi, int64_t off, int64_t n, int32_t* out) {
  uint64_t key = stream_key(seed, tid);
  uint64_t range = (uint64_t)(hi - lo + 1);
  for (int64_t i = 0; i < n; ++i) {
    uint64_t h = splitmix64(key + (uint64_t)(off + i)) >> 32;
    out[i] = (int32_t)(lo + (int64_t)((h * range) >> 32));
  }
}
