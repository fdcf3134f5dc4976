/*
 * ORACLE for the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the GPU path
 * computes. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the library path never calls it and shares no code,
 * header, table or helper with it. Floating point is carried in double
 * (fp64) except where the definition itself is fp32 (router logits are fp32
 * values; the top-k decision is taken on them).
 *
 * Pages cited (all are analyses of merged flashinfer pull requests):
 *  [P-ACT]   "FlashInfer MoE optimisation: overlapping grouped activation
 *            staging on Ampere and Hopper" (flashinfer PR #7368).
 *  [P-ROUTE] "TRTLLM-Gen MoE routing optimisation in FlashInfer: relieving
 *            register pressure" (flashinfer PR #3751).
 *  [P-A2A]   "FlashInfer MoE all-to-all optimisation: TRT-LLM's one-sided A2A"
 *            (flashinfer PR #3697).
 *  [P-VSA]   "Attention optimisation for Hopper (SM90): FlashInfer 'Cake'
 *            backend" (flashinfer PR #5586).
 *
 * The pages describe kernels, not the full layer; where they are silent the
 * plainest reading is taken and stated next to the function that uses it.
 *
 * OpenMP pragmas split only independent outer loops (tokens, entries); the
 * arithmetic of every output is the sequential loop written below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

static double bf16_val(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Expert partition across shares.
 * [P-A2A] section 1, "Flexible expert-to-rank mapping": with base = E / S and
 * rem = E % S, the shares are contiguous ranges of expert ids; the first rem
 * shares hold base + 1 experts and the others hold base. Share s therefore
 * starts after s full shares of base experts plus one extra expert for every
 * earlier share that holds base + 1.
 * Reading: E < S is legal (base = 0), later shares are then empty. */
int oracle_partition(int32_t E, int32_t S, int32_t s, int32_t* first, int32_t* count) {
  if (E < 1 || S < 1 || s < 0 || s >= S) return ORC_BAD;
  int32_t base = E / S, rem = E % S;
  int32_t f = 0;
  for (int32_t q = 0; q < s; ++q) f += base + (q < rem ? 1 : 0);
  *first = f;
  *count = base + (s < rem ? 1 : 0);
  return ORC_OK;
}

/* The share whose range holds expert e (the plain definition: search). */
int32_t oracle_owner(int32_t E, int32_t S, int32_t e) {
  for (int32_t s = 0; s < S; ++s) {
    int32_t f, c;
    oracle_partition(E, S, s, &f, &c);
    if (e >= f && e < f + c) return s;
  }
  return -1;
}

/* ------------------------------------------------------------------------ */
/* Router logits: logits[t, e] = x[t, :] . W_g[e, :] (+ b[e]).
 * The pages do not state the router; the logit is read as the fp32 value of
 * the exact affine map. x is bf16 and W_g fp32, so every product is exact in
 * double; the sum runs in double over h ascending, the bias is added in
 * double, and the result is rounded once to fp32. */
void oracle_router_logits(const uint16_t* x, const float* wg, const float* bias, int32_t T,
                          int32_t H, int32_t E, float* logits) {
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
      for (int32_t h = 0; h < H; ++h) xr[h] = bf16_val(x[(int64_t)t * H + h]);
      for (int32_t e = 0; e < E; ++e) {
        const float* w = wg + (int64_t)e * H;
        double acc = 0.0;
        for (int32_t h = 0; h < H; ++h) acc += xr[h] * (double)w[h];
        if (bias) acc += (double)bias[e];
        logits[(int64_t)t * E + e] = (float)acc;
      }
    }
    free(xr);
  }
}

/* ------------------------------------------------------------------------ */
/* Routing: softmax over the E logits, top-k, renormalise over the k chosen.
 * [P-ROUTE] names the routing method ("softmax_sum") and says the kernel
 * emits routing indices; the steps themselves come from the layer statement.
 * Readings:
 *  - the selection is taken on the fp32 logits (softmax is strictly
 *    increasing, so the order is the same as on probabilities, and no ties
 *    are created by rounding exp); equal logits go to the lower expert id;
 *    -0 and +0 compare equal;
 *  - slot j holds the j-th largest logit (ties: lower id first);
 *  - weights: p = softmax(l) over all E in double, w_j = p[id_j] / sum_i p[id_i]
 *    over the k chosen ids, always renormalised (k = 1 gives w = 1).
 * Non-finite logits are outside the domain: returns ORC_BAD. */
int oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                 double* weights) {
  if (T < 0 || E < 1 || k < 1 || k > E) return ORC_BAD;
  for (int64_t i = 0; i < (int64_t)T * E; ++i)
    if (!isfinite(logits[i])) return ORC_BAD;
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      const float* l = logits + (int64_t)t * E;
      memset(taken, 0, (size_t)E);
      for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (best < 0 || l[e] > l[best]) best = e; /* strict: keeps the lower id on equality */
        }
        taken[best] = 1;
        ids[(int64_t)t * k + j] = best;
      }
      double m = (double)l[0];
      for (int32_t e = 1; e < E; ++e)
        if ((double)l[e] > m) m = (double)l[e];
      double z = 0.0;
      for (int32_t e = 0; e < E; ++e) {
        p[e] = exp((double)l[e] - m);
        z += p[e];
      }
      for (int32_t e = 0; e < E; ++e) p[e] /= z;
      double s = 0.0;
      for (int32_t j = 0; j < k; ++j) s += p[ids[(int64_t)t * k + j]];
      for (int32_t j = 0; j < k; ++j)
        weights[(int64_t)t * k + j] = p[ids[(int64_t)t * k + j]] / s;
    }
    free(taken);
    free(p);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Histogram, prefix scan and permutation.
 * Entries are the expanded indices r = t*k + j. counts[e] counts the entries
 * routed to e, over all E experts. The local share is [first, first + L);
 * offsets[i] is where local expert first + i starts, offsets[L] = N_L.
 * Reading (the pages leave the order inside an expert open): a stable
 * counting sort by expert, so within an expert the entries keep ascending r.
 * permuted_rows[p] = r of the entry placed at p; expanded_to_permuted[r] = p,
 * or -1 for an entry whose expert is outside the share ([P-ACT] section 1
 * marks an absent group member by a negative index). */
int oracle_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t first, int32_t L,
                   int32_t* counts, int32_t* offsets, int32_t* permuted_rows,
                   int32_t* expanded_to_permuted) {
  if (T < 0 || k < 1 || E < 1 || first < 0 || L < 0 || first + L > E) return ORC_BAD;
  int64_t n = (int64_t)T * k;
  for (int64_t r = 0; r < n; ++r)
    if (ids[r] < 0 || ids[r] >= E) return ORC_BAD;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r = 0; r < n; ++r) counts[ids[r]] += 1;
  offsets[0] = 0;
  for (int32_t i = 0; i < L; ++i) offsets[i + 1] = offsets[i] + counts[first + i];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(L > 0 ? L : 1));
  for (int32_t i = 0; i < L; ++i) cursor[i] = offsets[i];
  for (int64_t r = 0; r < n; ++r) {
    int32_t e = ids[r];
    if (e >= first && e < first + L) {
      int32_t p = cursor[e - first]++;
      permuted_rows[p] = (int32_t)r;
      expanded_to_permuted[r] = p;
    } else {
      expanded_to_permuted[r] = -1;
    }
  }
  free(cursor);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* One expert applied to one activation row.
 * W1 of the expert is [2I, H]: rows [0, I) are the gate projection and rows
 * [I, 2I) the up projection (reading of the gate/up split that [P-ACT]
 * section 2 mentions; concatenated halves, not interleaved rows). W2 is [H, I].
 *   g_i = W1[i, :] . x,  u_i = W1[I + i, :] . x,  a_i = silu(g_i) * u_i,
 *   silu(g) = g / (1 + exp(-g)),  out[c] = W2[c, :] . a.
 * No biases. Everything in double; the intermediate a is never rounded. */
void oracle_expert_row(const uint16_t* xrow, const uint16_t* w1e, const uint16_t* w2e, int32_t H,
                       int32_t I, double* out) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  for (int32_t h = 0; h < H; ++h) xv[h] = bf16_val(xrow[h]);
  for (int32_t i = 0; i < I; ++i) {
    const uint16_t* wg = w1e + (int64_t)i * H;
    const uint16_t* wu = w1e + (int64_t)(I + i) * H;
    double g = 0.0, u = 0.0;
    for (int32_t h = 0; h < H; ++h) g += bf16_val(wg[h]) * xv[h];
    for (int32_t h = 0; h < H; ++h) u += bf16_val(wu[h]) * xv[h];
    a[i] = g / (1.0 + exp(-g)) * u;
  }
  for (int32_t c = 0; c < H; ++c) {
    const uint16_t* w = w2e + (int64_t)c * I;
    double acc = 0.0;
    for (int32_t i = 0; i < I; ++i) acc += bf16_val(w[i]) * a[i];
    out[c] = acc;
  }
  free(xv);
  free(a);
}

/* Grouped FFN over the permuted entries of the local share.
 * The row gathered for entry p is x[permuted_rows[p] / k] ([P-ACT] section 1
 * divides the route index by an input-route divisor to find the input row;
 * read here as k because the route indices are expanded indices t*k + j).
 * Local expert i uses w1 + i*2I*H and w2 + i*H*I. expert_out is [N_L, H]. */
int oracle_grouped_ffn(const uint16_t* x, const int32_t* permuted_rows, const int32_t* offsets,
                       int32_t L, int32_t T, int32_t k, int32_t H, int32_t I, const uint16_t* w1,
                       const uint16_t* w2, double* expert_out) {
  if (L < 0 || T < 0 || k < 1 || H < 1 || I < 1) return ORC_BAD;
  int32_t n = L > 0 ? offsets[L] : 0;
  for (int32_t p = 0; p < n; ++p) {
    int32_t r = permuted_rows[p];
    if (r < 0 || r >= T * k) return ORC_BAD;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t p = 0; p < n; ++p) {
    int32_t i = 0;
    while (offsets[i + 1] <= p) ++i;
    int32_t tok = permuted_rows[p] / k;
    oracle_expert_row(x + (int64_t)tok * H, w1 + (int64_t)i * 2 * I * H, w2 + (int64_t)i * H * I, H,
                      I, expert_out + (int64_t)p * H);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* FP8 expert weights (the FP8 path the [P-ACT] page mentions beside bf16 and
 * fp16, section 2: FP8 E4M3 operands). Reading: the OCP "e4m3fn" encoding
 * (sign bit, 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 holds
 * the subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; no
 * infinities), weights only (activations stay bf16), one fp32 scale per
 * weight row: W[r, c] = scale[r] * value(q[r, c]). */
double oracle_e4m3_value(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* The expert FFN of oracle_expert_row with dequantised weights: W1 rows
 * [0, I) gate and [I, 2I) up, W2 [H, I], each element scale[row] * value. */
void oracle_expert_row_fp8(const uint16_t* xrow, const uint8_t* w1q, const float* w1s,
                           const uint8_t* w2q, const float* w2s, int32_t H, int32_t I,
                           double* out) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  for (int32_t h = 0; h < H; ++h) xv[h] = bf16_val(xrow[h]);
  for (int32_t i = 0; i < I; ++i) {
    const uint8_t* qg = w1q + (int64_t)i * H;
    const uint8_t* qu = w1q + (int64_t)(I + i) * H;
    const double sg = (double)w1s[i], su = (double)w1s[I + i];
    double g = 0.0, u = 0.0;
    for (int32_t h = 0; h < H; ++h) g += sg * oracle_e4m3_value(qg[h]) * xv[h];
    for (int32_t h = 0; h < H; ++h) u += su * oracle_e4m3_value(qu[h]) * xv[h];
    const double silu_g = g / (1.0 + exp(-g));
    a[i] = silu_g * u;
  }
  for (int32_t c = 0; c < H; ++c) {
    const uint8_t* q = w2q + (int64_t)c * I;
    const double sc = (double)w2s[c];
    double acc = 0.0;
    for (int32_t i = 0; i < I; ++i) acc += sc * oracle_e4m3_value(q[i]) * a[i];
    out[c] = acc;
  }
  free(xv);
  free(a);
}

/* oracle_grouped_ffn with FP8 weights: w1q [L, 2I, H] codes, w1s [L, 2I],
 * w2q [L, H, I] codes, w2s [L, H]. */
int oracle_grouped_ffn_fp8(const uint16_t* x, const int32_t* permuted_rows,
                           const int32_t* offsets, int32_t L, int32_t T, int32_t k, int32_t H,
                           int32_t I, const uint8_t* w1q, const float* w1s, const uint8_t* w2q,
                           const float* w2s, double* expert_out) {
  if (L < 0 || T < 0 || k < 1 || H < 1 || I < 1) return ORC_BAD;
  int32_t n = L > 0 ? offsets[L] : 0;
  for (int32_t p = 0; p < n; ++p) {
    int32_t r = permuted_rows[p];
    if (r < 0 || r >= T * k) return ORC_BAD;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t p = 0; p < n; ++p) {
    int32_t i = 0;
    while (offsets[i + 1] <= p) ++i;
    int32_t row_tok = permuted_rows[p] / k;
    oracle_expert_row_fp8(x + (int64_t)row_tok * H, w1q + (int64_t)i * 2 * I * H,
                          w1s + (int64_t)i * 2 * I, w2q + (int64_t)i * H * I,
                          w2s + (int64_t)i * H, H, I, expert_out + (int64_t)p * H);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Routing-weighted combine back to token order:
 *   y[t, c] = sum over j = 0 .. k-1 of w[t, j] * expert_out[e2p[t*k + j], c],
 * skipping entries with e2p = -1 (experts outside the share), j ascending.
 * Reading: the weights were renormalised over all k before masking, so the
 * outputs of all shares add up to the full layer. [P-VSA] section 3 keeps the
 * partial results in fp32 to the end; here they are double, and the single
 * rounding to bf16 is left to the caller. */
void oracle_combine(const double* expert_out, const int32_t* e2p, const double* weights, int32_t T,
                    int32_t k, int32_t H, double* y) {
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t p = e2p[(int64_t)t * k + j];
        if (p >= 0) acc += weights[(int64_t)t * k + j] * expert_out[(int64_t)p * H + c];
      }
      y[(int64_t)t * H + c] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Whole layer for a sample of tokens: router logits and routing for all T
 * tokens, then for each sampled token t
 *   y[t] = sum_j [first <= id_j < first + L] * w_j * expert_{id_j}(x[t]),
 * j ascending, in double. bias may be NULL. sample lists n_sample token
 * indices; y is [n_sample, H]. logits [T, E], ids [T, k], weights [T, k]. */
int oracle_forward(const uint16_t* x, const float* wg, const float* bias, const uint16_t* w1,
                   const uint16_t* w2, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                   int32_t first, int32_t L, const int32_t* sample, int32_t n_sample,
                   float* logits, int32_t* ids, double* weights, double* y) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || k > E || first < 0 || L < 0 || first + L > E)
    return ORC_BAD;
  for (int32_t s = 0; s < n_sample; ++s)
    if (sample[s] < 0 || sample[s] >= T) return ORC_BAD;
  oracle_router_logits(x, wg, bias, T, H, E, logits);
  if (oracle_route(logits, T, E, k, ids, weights) != ORC_OK) return ORC_BAD;
  double* part = (double*)calloc((size_t)n_sample * k * H, sizeof(double));
  if (!part) return ORC_BAD;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < (int64_t)n_sample * k; ++q) {
    int32_t t = sample[q / k];
    int32_t e = ids[(int64_t)t * k + q % k];
    if (e < first || e >= first + L) continue;
    int32_t i = e - first;
    oracle_expert_row(x + (int64_t)t * H, w1 + (int64_t)i * 2 * I * H, w2 + (int64_t)i * H * I, H, I,
                      part + q * H);
  }
  for (int32_t s = 0; s < n_sample; ++s) {
    int32_t t = sample[s];
    for (int32_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = ids[(int64_t)t * k + j];
        if (e < first || e >= first + L) continue;
        acc += weights[(int64_t)t * k + j] * part[((int64_t)s * k + j) * H + c];
      }
      y[(int64_t)s * H + c] = acc;
    }
  }
  free(part);
  return ORC_OK;
}
