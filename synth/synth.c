/* synth.c -- host implementation of the seeded input generator (definition in synth.h). */
#include "synth.h"

#include <math.h>
#include <string.h>

uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_fnv1a64(const char* s) {
  uint64_t h = 0xCBF29CE484222325ULL;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001B3ULL;
  }
  return h;
}

uint64_t synth_key(uint64_t seed, const char* name) {
  return synth_mix64(synth_fnv1a64(name) ^ synth_mix64(seed + SYNTH_GOLDEN));
}

float synth_scale(double sigma) { return (float)(sigma / sqrt(SYNTH_IH_VAR)); }

static inline int32_t ih_of(uint64_t r) {
  int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) + (int32_t)((r >> 32) & 0xFFFF) +
              (int32_t)((r >> 48) & 0xFFFF);
  return s - SYNTH_IH_MEAN;
}

int32_t synth_ih(uint64_t key, uint64_t i) { return ih_of(synth_mix64(key + (i + 1) * SYNTH_GOLDEN)); }

uint16_t synth_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint64_t key, float scale, uint64_t off, size_t n, uint16_t* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 16))
  for (size_t j = 0; j < n; ++j) {
    float v = (float)synth_ih(key, off + j) * scale;
    out[j] = synth_f32_to_bf16(v);
  }
}

void synth_normal_f32(uint64_t key, float scale, uint64_t off, size_t n, float* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 16))
  for (size_t j = 0; j < n; ++j) out[j] = (float)synth_ih(key, off + j) * scale;
}

void synth_gain_bf16(uint64_t key, float scale, size_t n, uint16_t* out) {
  for (size_t j = 0; j < n; ++j) {
    volatile float t = (float)synth_ih(key, j) * scale; /* keep the two roundings separate */
    float v = 1.0f + t;
    out[j] = synth_f32_to_bf16(v);
  }
}

void synth_sigmoid_normal_f32(uint64_t key, size_t n, float* out) {
  double sd = sqrt(SYNTH_IH_VAR);
  for (size_t j = 0; j < n; ++j) {
    double z = (double)synth_ih(key, j) / sd;
    out[j] = (float)(1.0 / (1.0 + exp(-z)));
  }
}

void synth_tokens(uint64_t key, uint32_t V, size_t n, int32_t* out) {
  for (size_t j = 0; j < n; ++j) {
    uint64_t r = synth_mix64(key + (j + 1) * SYNTH_GOLDEN);
    out[j] = (int32_t)(((r >> 32) * (uint64_t)V) >> 32);
  }
}
