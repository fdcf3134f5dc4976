/*
 * moe.h -- C ABI of libmoe.so, a single-GPU Mixture-of-Experts layer forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The layer: router logits -> softmax / top-k / renormalise -> per-expert
 * histogram, prefix scan and stable token permutation -> gather of each
 * expert's activation rows -> grouped expert FFN (W1 gate/up, SwiGLU, W2 down)
 * -> routing-weighted combine back to token order. One GPU runs either all
 * experts or one contiguous share of them.
 *
 * Pages cited (analyses of merged flashinfer pull requests):
 *  [P-ACT]   "FlashInfer MoE optimisation: overlapping grouped activation
 *            staging on Ampere and Hopper" (PR #7368).
 *  [P-ROUTE] "TRTLLM-Gen MoE routing optimisation in FlashInfer: relieving
 *            register pressure" (PR #3751).
 *  [P-A2A]   "FlashInfer MoE all-to-all optimisation: TRT-LLM's one-sided A2A"
 *            (PR #3697).
 *  [P-FP4]   "Beyond the limits of NVFP4 GEMM: pipeline optimisation with L2
 *            weight prefetch" (PR #7424).
 *  [P-VSA]   "Attention optimisation for Hopper (SM90): FlashInfer 'Cake'
 *            backend" (PR #5586).
 *
 * Conventions shared by every call:
 *  - Pointers are caller-owned DEVICE pointers unless a parameter says
 *    "host". The library never allocates, frees or keeps memory, and keeps
 *    no state between calls ([P-FP4] section 2: workspace and outputs are
 *    handed in by the caller).
 *  - bf16 tensors are passed as uint16_t bit patterns. All tensors are dense
 *    row-major with the shapes written next to each parameter.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Calls enqueue work and return; nothing waits for the GPU, and no call
 *    copies data to the host.
 *  - Errors: every argument the host can see is checked before anything is
 *    launched; on any error nothing is launched and no output is written
 *    (checked launches that report failure, [P-A2A] section 2). A failed
 *    launch returns MOE_ERROR_LAUNCH. Nothing throws across the ABI.
 *  - T = 0 is valid and launches nothing.
 *  - Limits: 1 <= E <= 4096, 1 <= k <= min(E, 32), H >= 1, I >= 1,
 *    T * k < 2^31, T * k * max(H, I) < 2^31 elements.
 *  - Fast path: 16-byte aligned x / w1 / w2 / expert_out / workspace and H, I
 *    multiples of 128. Any other shape or alignment runs a correct
 *    element-wise path instead of failing ([P-ACT] section 1: the 128-bit
 *    vector gather keeps a scalar fallback for unaligned inputs).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_SUCCESS = 0,
  MOE_ERROR_INVALID_VALUE = 1, /* bad size, null pointer, share out of range */
  MOE_ERROR_UNSUPPORTED = 2,   /* outside the limits above */
  MOE_ERROR_WORKSPACE = 3,     /* workspace missing, too small or misaligned */
  MOE_ERROR_LAUNCH = 4         /* a kernel launch failed */
} moe_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* moe_status_string(moe_status status);

/* Name of the HIP error behind the last MOE_ERROR_LAUNCH returned on the
 * calling host thread ("hipSuccess" if there was none). Diagnostic only. */
const char* moe_last_launch_error(void);

/*
 * moe_partition -- contiguous ceil/floor split of E experts over S shares.
 * [P-A2A] section 1, "Flexible expert-to-rank mapping": base = E / S,
 * rem = E % S; shares 0 .. rem-1 hold base + 1 experts, the others base, in
 * expert order. Pure host function; first_expert and num_local are HOST
 * pointers. E < S is allowed (the last shares are then empty).
 * Errors: E < 1, S < 1, share outside [0, S), null output pointer.
 */
moe_status moe_partition(int32_t num_experts, int32_t num_shares, int32_t share,
                         int32_t* first_expert, int32_t* num_local);

/*
 * moe_workspace_size -- bytes of device workspace that moe_forward needs
 * (*bytes, HOST pointer); the caller allocates it and passes it in ([P-FP4]
 * section 2: the caller provides the workspace and output buffers).
 * moe_router_logits, moe_permute, moe_route_permute and moe_grouped_ffn need
 * no more than this for the same sizes, so one workspace serves every call.
 * The workspace must be 256-byte aligned. Its contents need no
 * initialisation and are scratch after the call.
 */
moe_status moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                              int32_t num_local, size_t* bytes);

/*
 * moe_router_logits -- logits[t, e] = x[t, :] . w_gate[e, :] + bias[e].
 * The pages leave the router unstated; the logit is the fp32 value of the
 * exact affine map: the products (bf16 x fp32) are exact in fp64, the sum is
 * carried in fp64 and rounded once to fp32.
 *   x       [T, H] bf16;  w_gate [E, H] fp32;  bias [E] fp32 or NULL
 *   logits  [T, E] fp32 (output)
 *   ws / ws_bytes  workspace (moe_workspace_size with the same T, H, E; it
 *                  holds fp64 partial sums when T > 64, unused otherwise)
 */
moe_status moe_router_logits(const uint16_t* x, const float* w_gate, const float* bias, int32_t T,
                             int32_t H, int32_t E, float* logits, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * moe_route -- softmax over the E logits, top-k, renormalise over the k.
 * [P-ROUTE] (routing kernel emitting routing indices; "softmax_sum" method).
 * Selection on the fp32 logits, larger first, equal logits to the lower
 * expert id (-0 equals +0); slot j holds the j-th selection. Weights:
 * w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected logits,
 * which equals the full softmax renormalised over the selection.
 *   logits       [T, E] fp32, finite (NaN / inf give unspecified ids/weights)
 *   topk_ids     [T, k] int32 (output), distinct within a token
 *   topk_weights [T, k] fp32 (output), sum to 1 per token
 */
moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_weights, void* stream);

/*
 * moe_permute -- per-expert histogram, prefix scan and stable permutation.
 * Entries are expanded indices r = t * k + j. The local share is experts
 * [first_expert, first_expert + num_local).
 *   topk_ids             [T, k] int32 in [0, E), distinct within a token.
 *                        Ids outside [0, E) are skipped (not counted,
 *                        expanded_to_permuted = -1); repeated ids within a
 *                        token give an unspecified permutation but never an
 *                        out-of-range write.
 *   expert_counts        [E] int32 (output): entries per expert, all E.
 *   expert_offsets       [num_local + 1] int32 (output): exclusive scan of
 *                        the local counts; offsets[num_local] = N_L.
 *   permuted_rows        [T * k] int32 (output): permuted_rows[p] = r of the
 *                        p-th local entry, experts in order and ascending r
 *                        within an expert; positions >= N_L are not written.
 *   expanded_to_permuted [T * k] int32 (output): p of entry r, or -1 when
 *                        r's expert is outside the share ([P-ACT] section 1
 *                        marks absent group members with a negative index).
 *   ws / ws_bytes        workspace (moe_workspace_size).
 */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t first_expert, int32_t num_local, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* permuted_rows,
                       int32_t* expanded_to_permuted, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_permute -- moe_route, then moe_permute on its topk_ids: the
 * routing steps of the layer in one call (the routing kernel of [P-ROUTE]
 * emits the routing indices that the permutation consumes), in the variant
 * moe_routing_plan names for these sizes. Arguments, outputs and errors are
 * those of moe_route and moe_permute; the workspace is moe_permute's
 * (moe_workspace_size covers it). Every variant gives identical outputs.
 */
moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t first_expert, int32_t num_local, int32_t* topk_ids,
                             float* topk_weights, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* permuted_rows, int32_t* expanded_to_permuted, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Routing variants: how the selection and the permutation are split into
 * kernels ([P-ROUTE] section 1: the launch shape follows the token count;
 * section 2: the valid shapes are fixed ahead of time).
 *   MOE_ROUTING_ONE_BLOCK   T <= 64: one single-block kernel selects and
 *                           permutes in on-chip memory (one launch; the
 *                           selection runs on one compute unit).
 *   MOE_ROUTING_TWO_KERNELS a selection kernel (one wave per token), then a
 *                           single-block permutation; while every 64-token
 *                           tile's masks and bases fit in one block's LDS.
 *   MOE_ROUTING_TILED       the selection kernel also writes per-tile token
 *                           masks, then a scan kernel and a scatter kernel;
 *                           any T.
 */
typedef enum moe_routing_variant {
  MOE_ROUTING_AUTO = 0,
  MOE_ROUTING_ONE_BLOCK = 1,
  MOE_ROUTING_TWO_KERNELS = 2,
  MOE_ROUTING_TILED = 3
} moe_routing_variant;

/*
 * moe_routing_plan -- the variant moe_route_permute and moe_forward run for
 * T tokens, E experts, top-k and a share of num_local experts (*variant,
 * HOST pointer): the applicable variant with the smallest time predicted by
 * a cost model fitted to the variants' measured times ([P-VSA]'s planner
 * likewise picks a kernel configuration from a cost estimate). Pure host
 * function. Errors as moe_route.
 */
moe_status moe_routing_plan(int32_t T, int32_t E, int32_t k, int32_t num_local,
                            int32_t* variant);

/*
 * moe_route_permute_variant -- moe_route_permute in a given variant (a
 * moe_routing_variant; MOE_ROUTING_AUTO = the plan), for measurement and
 * testing. MOE_ERROR_UNSUPPORTED when the variant does not apply to these
 * sizes; otherwise as moe_route_permute.
 */
moe_status moe_route_permute_variant(const float* logits, int32_t T, int32_t E, int32_t k,
                                     int32_t first_expert, int32_t num_local, int32_t* topk_ids,
                                     float* topk_weights, int32_t* expert_counts,
                                     int32_t* expert_offsets, int32_t* permuted_rows,
                                     int32_t* expanded_to_permuted, void* ws, size_t ws_bytes,
                                     int32_t variant, void* stream);

/*
 * moe_grouped_ffn -- for every local entry p of local expert i:
 *   x_g   = x[permuted_rows[p] / k]   (gather; [P-ACT] section 1 divides the
 *                                      route index by the route divisor)
 *   g, u  = W1[i][0:I] . x_g, W1[i][I:2I] . x_g   (gate rows first, then up;
 *                                      the gate/up split of [P-ACT] section 2)
 *   a     = silu(g) * u                (kept in fp32, never rounded to bf16)
 *   out_p = W2[i] . a
 * bf16 MFMA with fp32 accumulation; a enters W2's product as the exact sum of
 * two bf16 parts (hi + lo), so only the final output is ever rounded.
 *   x              [T, H] bf16
 *   permuted_rows  [T * k] int32, entries of [0, N_L) read; values outside
 *                  [0, T * k) gather a zero row
 *   expert_offsets [num_local + 1] int32, non-decreasing from 0, last <= T*k
 *   w1             [num_local, 2I, H] bf16 (local experts only)
 *   w2             [num_local, H, I] bf16
 *   expert_out     [T * k, H] fp32 (output): rows [0, N_L) written
 *   ws / ws_bytes  workspace (moe_workspace_size)
 */
moe_status moe_grouped_ffn(const uint16_t* x, const int32_t* permuted_rows,
                           const int32_t* expert_offsets, int32_t num_local, int32_t T, int32_t k,
                           int32_t H, int32_t I, const uint16_t* w1, const uint16_t* w2,
                           float* expert_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn_fp8 -- moe_grouped_ffn with FP8 expert weights: the same
 * gather, gate/up split, SwiGLU and down projection, with each weight row
 * stored as FP8 E4M3 codes and one fp32 scale ([P-ACT] section 2 runs the
 * grouped projection on FP8 E4M3 operands beside bf16 / fp16). Reading: the
 * OCP "e4m3fn" encoding (bias 7, no infinities, 0x7F / 0xFF NaN), weights
 * only (x stays bf16), W[r, c] = scale[r] * value(code[r, c]). Codes are
 * widened to bf16 exactly, multiplied on bf16 MFMA with fp32 accumulation,
 * and each finished row sum is multiplied by its row's scale.
 *   w1q  [num_local, 2I, H] uint8 codes     w1s  [num_local, 2I] fp32 scales
 *   w2q  [num_local, H, I] uint8 codes      w2s  [num_local, H] fp32 scales
 * Every other argument, the workspace and the errors are as for
 * moe_grouped_ffn; w1s and w2s must not be NULL.
 */
moe_status moe_grouped_ffn_fp8(const uint16_t* x, const int32_t* permuted_rows,
                               const int32_t* expert_offsets, int32_t num_local, int32_t T,
                               int32_t k, int32_t H, int32_t I, const uint8_t* w1q,
                               const float* w1s, const uint8_t* w2q, const float* w2s,
                               float* expert_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- y[t, :] = sum over j ascending of topk_weights[t, j] *
 * expert_out[expanded_to_permuted[t*k + j], :], skipping -1 entries; fp32
 * accumulation and one round-to-nearest-even to bf16 ([P-VSA] section 3
 * keeps fp32 partials until the end). A token with no local entry gets 0.
 *   expert_out           [T * k, H] fp32 (rows indexed by permuted position)
 *   expanded_to_permuted [T * k] int32, values in [-1, T * k)
 *   topk_weights         [T, k] fp32
 *   y                    [T, H] bf16 (output)
 */
moe_status moe_combine(const float* expert_out, const int32_t* expanded_to_permuted,
                       const float* topk_weights, int32_t T, int32_t k, int32_t H, uint16_t* y,
                       void* stream);

/*
 * moe_forward -- the whole layer on one GPU for one expert share:
 * moe_router_logits -> moe_route_permute -> moe_grouped_ffn -> moe_combine,
 * stream-ordered, with no host synchronisation in between. The share is the
 * contiguous expert range of the ceil/floor partition ([P-A2A] section 1;
 * moe_partition); selections of experts outside it are masked after
 * renormalisation (the non-local members of [P-ACT] section 1 carry a
 * negative index), so the outputs of all shares add up to the whole layer.
 *   x [T, H] bf16; w_gate [E, H] fp32; router_bias [E] fp32 or NULL;
 *   w1 [num_local, 2I, H] bf16; w2 [num_local, H, I] bf16 (local experts)
 *   y [T, H] bf16 (output)
 *   logits_out [T, E] fp32, topk_ids_out [T, k] int32,
 *   topk_weights_out [T, k] fp32: optional outputs (NULL = kept in ws)
 *   ws / ws_bytes: workspace of at least moe_workspace_size bytes.
 */
moe_status moe_forward(const uint16_t* x, const float* w_gate, const float* router_bias,
                       const uint16_t* w1, const uint16_t* w2, int32_t T, int32_t H, int32_t I,
                       int32_t E, int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                       float* logits_out, int32_t* topk_ids_out, float* topk_weights_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_fp8 -- moe_forward with the FP8 expert weights of
 * moe_grouped_ffn_fp8 (E4M3 codes and one fp32 scale per row, [P-ACT]
 * section 2): router, route, permute and combine as in moe_forward, the
 * grouped FFN as in moe_grouped_ffn_fp8.
 *   w1q [num_local, 2I, H] uint8, w1s [num_local, 2I] fp32,
 *   w2q [num_local, H, I] uint8, w2s [num_local, H] fp32 (local experts)
 * Every other argument, the workspace (moe_workspace_size) and the errors
 * are as for moe_forward.
 */
moe_status moe_forward_fp8(const uint16_t* x, const float* w_gate, const float* router_bias,
                           const uint8_t* w1q, const float* w1s, const uint8_t* w2q,
                           const float* w2s, int32_t T, int32_t H, int32_t I, int32_t E,
                           int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                           float* logits_out, int32_t* topk_ids_out, float* topk_weights_out,
                           void* ws, size_t ws_bytes, void* stream);

/* Size of the device scratch array behind moe_forward_no_alloc (bytes). */
#define MOE_NO_ALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * moe_forward_no_alloc -- moe_forward without a workspace argument, for
 * callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, hosts that forbid allocation). The workspace is a
 * device array of MOE_NO_ALLOC_SCRATCH_BYTES inside the library; each GPU
 * holds its own copy from the first call on it until the process ends. No
 * call allocates or frees memory.
 *   Every argument, output and error is as for moe_forward, plus:
 *   MOE_ERROR_WORKSPACE when moe_workspace_size for these sizes exceeds
 *   MOE_NO_ALLOC_SCRATCH_BYTES (128 MiB): decode-shaped layers (8.5 MiB at
 *   T 32, H 4096, I 14336, 8 experts, top-2) fit; shapes with more than
 *   about 16 entries per expert, whose FFN stages token rows in LDS and keeps
 *   ~130 MiB of cross-block partial sums, do not.
 *   MOE_ERROR_LAUNCH when the array's device address cannot be obtained.
 * Every call on one GPU uses that GPU's one array: calls that overlap on the
 * same GPU (concurrent streams or host threads) race and must be ordered by
 * the caller. The array keeps the last call's contents; every value a call
 * reads from it is written earlier in the same call.
 */
moe_status moe_forward_no_alloc(const uint16_t* x, const float* w_gate,
                                const float* router_bias, const uint16_t* w1,
                                const uint16_t* w2, int32_t T, int32_t H, int32_t I, int32_t E,
                                int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                                float* logits_out, int32_t* topk_ids_out,
                                float* topk_weights_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
