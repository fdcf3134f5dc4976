/*
 * Seeded synthetic inputs for the MoE layer forward.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic
 * (no routing, no softmax, no matrix products), so both the oracle side and
 * the GPU side can take their inputs from it without sharing any step of the
 * method. Every value is a pure function of (seed, tensor id, expert, index):
 * any split of the index range, any thread count, gives identical bytes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based hash; two 53-bit
 * uniforms per pair of elements; the Box-Muller transform (Box and Muller,
 * 1958) in double; the double result is rounded to float (round to nearest
 * even), and for bf16 tensors the float is rounded to bf16 with round to
 * nearest even on its bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint32_t tensor, uint32_t expert) {
  return mix64(mix64(mix64(seed) ^ (uint64_t)tensor) ^ (uint64_t)expert);
}

/* Standard normal number number `i` of the stream `key`. */
static double normal_at(uint64_t key, int64_t i) {
  uint64_t q = (uint64_t)i >> 1;
  uint64_t a = mix64(key + 2u * q);
  uint64_t b = mix64(key + 2u * q + 1u);
  double u1 = ((double)((a >> 11) + 1u)) * 0x1.0p-53; /* (0, 1] */
  double u2 = ((double)(b >> 11)) * 0x1.0p-53;        /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(ang) : r * cos(ang);
}

/* Uniform 64-bit word number `i` of the stream `key`. */
static uint64_t word_at(uint64_t key, int64_t i) { return mix64(key ^ mix64((uint64_t)i)); }

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_normal_f32(uint64_t seed, uint32_t tensor, uint32_t expert, int64_t n, double sigma,
                      float* out) {
  uint64_t key = stream_key(seed, tensor, expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, i));
}

/* n_per_expert values for each of num_experts experts, expert ids starting at
 * first_expert; expert e's values land at out[(e - first_expert) * n_per_expert]. */
void synth_normal_bf16(uint64_t seed, uint32_t tensor, uint32_t first_expert, uint32_t num_experts,
                       int64_t n_per_expert, double sigma, uint16_t* out) {
  const int64_t chunk = 1 << 16;
  int64_t chunks_per_expert = (n_per_expert + chunk - 1) / chunk;
  int64_t total = chunks_per_expert * (int64_t)num_experts;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t c = 0; c < total; ++c) {
    uint32_t le = (uint32_t)(c / chunks_per_expert);
    int64_t i0 = (c % chunks_per_expert) * chunk;
    int64_t i1 = i0 + chunk < n_per_expert ? i0 + chunk : n_per_expert;
    uint64_t key = stream_key(seed, tensor, first_expert + le);
    uint16_t* dst = out + (int64_t)le * n_per_expert;
    for (int64_t i = i0; i < i1; ++i) dst[i] = f32_to_bf16_rne((float)(sigma * normal_at(key, i)));
  }
}

/* Logits quantised to eight exactly representable levels (+-0.25 ... +-1.75):
 * level = clamp(floor(z / 0.5) + 4, 0, 7), value = (level - 3.5) * 0.5, z ~ N(0,1). */
void synth_tie_levels_f32(uint64_t seed, uint32_t tensor, uint32_t expert, int64_t n, float* out) {
  uint64_t key = stream_key(seed, tensor, expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double z = normal_at(key, i);
    double lv = floor(z / 0.5) + 4.0;
    if (lv < 0.0) lv = 0.0;
    if (lv > 7.0) lv = 7.0;
    out[i] = (float)((lv - 3.5) * 0.5);
  }
}

/* k distinct expert ids in [0, E) per token, uniformly drawn by rejection,
 * in draw order (not sorted). Requires k <= E. */
void synth_topk_ids(uint64_t seed, uint32_t tensor, int32_t T, int32_t E, int32_t k, int32_t* out) {
  uint64_t key = stream_key(seed, tensor, 0);
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    int64_t draw = (int64_t)t << 20;
    for (int32_t j = 0; j < k; ++j) {
      for (;;) {
        int32_t e = (int32_t)(word_at(key, draw++) % (uint64_t)E);
        int dup = 0;
        for (int32_t q = 0; q < j; ++q) dup |= (out[(int64_t)t * k + q] == e);
        if (!dup) {
          out[(int64_t)t * k + j] = e;
          break;
        }
      }
    }
  }
}

/* Uniform integers in [0, m). */
void synth_uniform_int(uint64_t seed, uint32_t tensor, int64_t n, int64_t m, int64_t* out) {
  uint64_t key = stream_key(seed, tensor, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (int64_t)(word_at(key, i) % (uint64_t)m);
}
