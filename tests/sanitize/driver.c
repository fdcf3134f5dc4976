/*
 * Runs every oracle and input-generator function once on small, ragged
 * inputs, for a CPU build under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (tests/test_sanitize.py compiles it together with oracle.c and
 * synth.c). Exits 0 when every call returned success; the sanitizers abort
 * on an out-of-bounds access, a leak or undefined behaviour.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_partition(int32_t E, int32_t S, int32_t s, int32_t* first, int32_t* count);
int32_t oracle_owner(int32_t E, int32_t S, int32_t e);
void oracle_router_logits(const uint16_t* x, const float* wg, const float* bias, int32_t T,
                          int32_t H, int32_t E, float* logits);
int oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                 double* weights);
int oracle_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t first, int32_t L,
                   int32_t* counts, int32_t* offsets, int32_t* permuted_rows,
                   int32_t* expanded_to_permuted);
int oracle_grouped_ffn(const uint16_t* x, const int32_t* permuted_rows, const int32_t* offsets,
                       int32_t L, int32_t T, int32_t k, int32_t H, int32_t I, const uint16_t* w1,
                       const uint16_t* w2, double* expert_out);
int oracle_grouped_ffn_fp8(const uint16_t* x, const int32_t* permuted_rows,
                           const int32_t* offsets, int32_t L, int32_t T, int32_t k, int32_t H,
                           int32_t I, const uint8_t* w1q, const float* w1s, const uint8_t* w2q,
                           const float* w2s, double* expert_out);
void oracle_combine(const double* expert_out, const int32_t* e2p, const double* weights, int32_t T,
                    int32_t k, int32_t H, double* y);
int oracle_forward(const uint16_t* x, const float* wg, const float* bias, const uint16_t* w1,
                   const uint16_t* w2, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                   int32_t first, int32_t L, const int32_t* sample, int32_t n_sample,
                   float* logits, int32_t* ids, double* weights, double* y);
void synth_normal_f32(uint64_t seed, uint32_t tensor, uint32_t expert, int64_t n, double sigma,
                      float* out);
void synth_normal_bf16(uint64_t seed, uint32_t tensor, uint32_t first_expert, uint32_t num_experts,
                       int64_t n_per_expert, double sigma, uint16_t* out);
void synth_tie_levels_f32(uint64_t seed, uint32_t tensor, uint32_t expert, int64_t n, float* out);
void synth_topk_ids(uint64_t seed, uint32_t tensor, int32_t T, int32_t E, int32_t k, int32_t* out);
void synth_uniform_int(uint64_t seed, uint32_t tensor, int64_t n, int64_t m, int64_t* out);
void synth_fp8_rows(uint64_t seed, uint32_t tensor, uint32_t first_expert, uint32_t num_experts,
                    int64_t rows, int64_t cols, double sigma, uint8_t* q, float* scale);

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);       \
      return 1;                                                      \
    }                                                                \
  } while (0)

static void* cal(size_t n, size_t s) { return calloc(n ? n : 1, s); }

static int run(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t first, int32_t L) {
  uint16_t* x = cal((size_t)T * H, 2);
  float* wg = cal((size_t)E * H, 4);
  float* bias = cal((size_t)E, 4);
  uint16_t* w1 = cal((size_t)L * 2 * I * H, 2);
  uint16_t* w2 = cal((size_t)L * H * I, 2);
  uint8_t* w1q = cal((size_t)L * 2 * I * H, 1);
  uint8_t* w2q = cal((size_t)L * H * I, 1);
  float* w1s = cal((size_t)L * 2 * I, 4);
  float* w2s = cal((size_t)L * H, 4);
  float* logits = cal((size_t)T * E, 4);
  float* ties = cal((size_t)T * E, 4);
  int32_t* ids = cal((size_t)T * k, 4);
  int32_t* ids2 = cal((size_t)T * k, 4);
  double* w = cal((size_t)T * k, 8);
  int32_t* counts = cal(E, 4);
  int32_t* offsets = cal((size_t)L + 1, 4);
  int32_t* perm = cal((size_t)T * k, 4);
  int32_t* e2p = cal((size_t)T * k, 4);
  double* eo = cal((size_t)T * k * H, 8);
  double* y = cal((size_t)T * H, 8);
  int32_t sample[2] = {0, T - 1};
  int64_t ints[16];
  int rc = 0;
  synth_normal_bf16(7, 1, 0, 1, (int64_t)T * H, 1.0, x);
  synth_normal_f32(7, 2, 0, (int64_t)E * H, 0.1, wg);
  synth_normal_f32(7, 5, 0, E, 1.0, bias);
  synth_normal_bf16(7, 3, first, L, (int64_t)2 * I * H, 0.02, w1);
  synth_normal_bf16(7, 4, first, L, (int64_t)H * I, 0.02, w2);
  synth_fp8_rows(7, 3, first, L, 2 * I, H, 0.02, w1q, w1s);
  synth_fp8_rows(7, 4, first, L, H, I, 0.02, w2q, w2s);
  synth_tie_levels_f32(7, 106, 0, (int64_t)T * E, ties);
  synth_topk_ids(7, 7, T, E, k, ids2);
  synth_uniform_int(7, 8, 16, 5, ints);
  oracle_router_logits(x, wg, bias, T, H, E, logits);
  if (oracle_route(logits, T, E, k, ids, w) != 0) rc = 1;
  if (oracle_route(ties, T, E, k, ids, w) != 0) rc = 1;
  if (oracle_route(logits, T, E, k, ids, w) != 0) rc = 1;
  if (oracle_permute(ids, T, k, E, first, L, counts, offsets, perm, e2p) != 0) rc = 1;
  if (oracle_grouped_ffn(x, perm, offsets, L, T, k, H, I, w1, w2, eo) != 0) rc = 1;
  if (oracle_grouped_ffn_fp8(x, perm, offsets, L, T, k, H, I, w1q, w1s, w2q, w2s, eo) != 0) rc = 1;
  oracle_combine(eo, e2p, w, T, k, H, y);
  if (oracle_forward(x, wg, bias, w1, w2, T, H, I, E, k, first, L, sample, 2, logits, ids, w, y) != 0)
    rc = 1;
  if (oracle_permute(ids2, T, k, E, first, L, counts, offsets, perm, e2p) != 0) rc = 1;
  free(x); free(wg); free(bias); free(w1); free(w2); free(w1q); free(w2q); free(w1s); free(w2s);
  free(logits); free(ties); free(ids); free(ids2); free(w); free(counts); free(offsets); free(perm);
  free(e2p); free(eo); free(y);
  return rc;
}

int main(void) {
  int32_t f, c;
  for (int32_t E = 1; E <= 40; ++E)
    for (int32_t S = 1; S <= 7; ++S)
      for (int32_t s = 0; s < S; ++s) {
        CHECK(oracle_partition(E, S, s, &f, &c) == 0);
        for (int32_t e = f; e < f + c; ++e) CHECK(oracle_owner(E, S, e) == s);
      }
  CHECK(run(5, 24, 16, 6, 2, 0, 6) == 0);
  CHECK(run(9, 13, 7, 11, 3, 4, 5) == 0);
  CHECK(run(3, 8, 8, 4, 4, 1, 0) == 0);
  CHECK(run(17, 32, 24, 40, 8, 10, 20) == 0);
  printf("sanitized oracle and generator: ok\n");
  return 0;
}
