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

/* OCP FP8 E4M3 ("e4m3fn": exponent bias 7, three mantissa bits, no
 * infinities, 0x7F and 0xFF are NaN, largest finite value 448; OCP 8-bit
 * Floating Point Specification, 2023). A finite float is rounded to the
 * nearest code with ties to the even code; magnitudes of 448 and above
 * saturate to 448. Input preparation only: it makes the quantised weights
 * that both sides then read. */
static uint8_t f32_to_e4m3(float f) {
  const uint8_t sign = signbit(f) ? 0x80 : 0;
  const double a = fabs((double)f);
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0x1p-6) return sign | (uint8_t)rint(a * 512.0); /* units of 2^-9; 8 is 2^-6 */
  int e;
  const double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
  double m = rint((fr * 2.0 - 1.0) * 8.0);
  int E = e + 6; /* biased exponent: a = (1 + m/8) * 2^(E - 7) */
  if (m == 8.0) {
    m = 0.0;
    E += 1;
  }
  return sign | (uint8_t)(E << 3) | (uint8_t)m;
}

/* Weights quantised per output row: for each of num_experts experts (ids from
 * first_expert) and each of its rows, the fp32 normals sigma * N(0,1) at
 * indices row * cols + c of the expert's stream (the same numbers the bf16
 * generator rounds), scale = max |w| / 448 over the row (1 for an all-zero
 * row), codes q = e4m3(w / scale). q is [num_experts, rows, cols], scale
 * [num_experts, rows]; the weight the layer uses is scale * value(q). */
void synth_fp8_rows(uint64_t seed, uint32_t tensor, uint32_t first_expert, uint32_t num_experts,
                    int64_t rows, int64_t cols, double sigma, uint8_t* q, float* scale) {
  const int64_t total = rows * (int64_t)num_experts;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t g = 0; g < total; ++g) {
    const uint32_t le = (uint32_t)(g / rows);
    const int64_t r = g % rows;
    const uint64_t key = stream_key(seed, tensor, first_expert + le);
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      const float w = (float)(sigma * normal_at(key, r * cols + c));
      if (fabsf(w) > amax) amax = fabsf(w);
    }
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scale[g] = s;
    uint8_t* dst = q + g * cols;
    for (int64_t c = 0; c < cols; ++c) {
      const float w = (float)(sigma * normal_at(key, r * cols + c));
      dst[c] = f32_to_e4m3(w / s);
    }
  }
}
