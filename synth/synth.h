/*
 * synth.h -- seeded synthetic inputs (weights, caches, recurrent state, tokens).
 *
 * This module holds no arithmetic of the decode step. It only turns
 * (seed, tensor name, element index) into numbers, so that the oracle and the
 * HIP path can be fed identical inputs. A device implementation of the same
 * definition lives in synth_dev.hip; both produce bit-identical outputs.
 *
 * Definition (every step is integer arithmetic or one correctly rounded IEEE
 * operation, so CPU and GPU agree bit for bit):
 *
 *   mix64(z)      SplitMix64 output function (Steele, Lea and Flood,
 *                 "Fast splittable pseudorandom number generators", OOPSLA
 *                 2014; constants as in Vigna's public splitmix64.c):
 *                   z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *                   z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *                   return z ^ (z >> 31)
 *   key(seed, name) = mix64(FNV1a64(name) ^ mix64(seed + G)),  G = 0x9E3779B97F4A7C15
 *   r_i           = mix64(key + (i + 1) * G)   (the SplitMix64 stream from state key)
 *   s_i           = sum of the four 16-bit fields of r_i        (Irwin-Hall, n = 4)
 *   z_i           = s_i - 131070                               (integer, |z| <= 131070)
 *   normal(i)     = (float)z_i * scale,  scale = (float)(sigma / sqrt(4 * (65536^2 - 1) / 12))
 *                   i.e. an approximately normal variate with standard deviation sigma
 *   bf16(v)       = round-to-nearest-even of the fp32 v to bfloat16
 *   gain(i)       = bf16(1.0f + (float)z_i * scale)   (two separately rounded fp32 ops)
 *   token(i)      = (uint32)(((r_i >> 32) * V) >> 32)  (uniform over [0, V))
 *   sigmoid_normal(i) = (float)(1 / (1 + exp(-z_i / IH_STD)))  (host only, double precision)
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL
#define SYNTH_IH_MEAN 131070
/* sqrt(4 * (65536^2 - 1) / 12): standard deviation of the sum of four uniform 16-bit integers */
#define SYNTH_IH_VAR 1431655765.0

uint64_t synth_mix64(uint64_t z);
uint64_t synth_fnv1a64(const char* s);
uint64_t synth_key(uint64_t seed, const char* name);
/* scale such that (float)z * scale has standard deviation sigma */
float synth_scale(double sigma);
/* integer Irwin-Hall deviate z_i of stream `key` (exposed for tests) */
int32_t synth_ih(uint64_t key, uint64_t i);

/* out[j] = bf16((float)z_{off+j} * scale), j < n */
void synth_normal_bf16(uint64_t key, float scale, uint64_t off, size_t n, uint16_t* out);
/* out[j] = (float)z_{off+j} * scale */
void synth_normal_f32(uint64_t key, float scale, uint64_t off, size_t n, float* out);
/* out[j] = bf16(1.0f + (float)z_j * scale) */
void synth_gain_bf16(uint64_t key, float scale, size_t n, uint16_t* out);
/* out[j] = (float)sigmoid(z_j / IH_STD) computed in double */
void synth_sigmoid_normal_f32(uint64_t key, size_t n, float* out);
/* out[j] = token in [0, V) */
void synth_tokens(uint64_t key, uint32_t V, size_t n, int32_t* out);
/* fp32 -> bf16 round-to-nearest-even (NaN kept quiet) */
uint16_t synth_f32_to_bf16(float f);

#ifdef __cplusplus
}
#endif
#endif
