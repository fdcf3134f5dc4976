// C ABI of libmoe.so (declared in include/moe.h): argument checks on the
// host, workspace carving, and the stream-ordered launch chain. No call
// allocates, synchronises or copies to the host.
#include "moe.h"

#include <hip/hip_runtime.h>

#include "plan.h"

#include <cstdint>
#include <mutex>

namespace moe {
size_t router_workspace_bytes(int T, int H, int E);
hipError_t launch_router_logits(const uint16_t* x, const float* wg, const float* bias, int T, int H,
                                int E, float* logits, void* ws, hipStream_t stream);
hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t stream);
size_t permute_workspace_bytes(int T, int E, int L);
hipError_t launch_permute(const int* ids, int T, int k, int E, int first, int L, int* counts,
                          int* offsets, int* perm, int* e2p, void* ws, hipStream_t stream);
hipError_t launch_route_permute(int variant, const float* logits, int T, int E, int k, int first,
                                int L, int* ids, float* w, int* counts, int* offsets, int* perm,
                                int* e2p, void* ws, const PlanOut& po, hipStream_t stream);
int routing_plan(int T, int E, int k, int L);
bool routing_variant_applies(int variant, int T, int E, int L);
size_t ffn_workspace_bytes(int T, int k, int I, int L);
hipError_t launch_grouped_ffn(const uint16_t* x, const int* perm, const int* offsets, int L, int T,
                              int k, int H, int I, const uint16_t* w1, const uint16_t* w2,
                              float* out, void* ws, bool plan_ready, hipStream_t stream);
hipError_t launch_grouped_ffn_fp8(const uint16_t* x, const int* perm, const int* offsets, int L,
                                  int T, int k, int H, int I, const uint8_t* w1q,
                                  const float* w1s, const uint8_t* w2q, const float* w2s,
                                  float* out, void* ws, bool plan_ready, hipStream_t stream);
bool ffn_plan_target(const void* x, const void* w1, const void* w2, const void* out, int T, int k,
                     int L, int H, int I, bool f8, void* ws, PlanOut* po);
hipError_t launch_combine(const float* eo, const int* e2p, const float* w, int T, int k, int H,
                          uint16_t* y, hipStream_t stream);
}  // namespace moe

namespace {

constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 32;
constexpr int64_t kMaxIndex = (int64_t)1 << 31;

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// HIP error of the last failed launch on this host thread (for diagnostics).
thread_local hipError_t t_last_launch_error = hipSuccess;

// hipGetLastError reports the last failing HIP call of the thread, whoever
// made it (a query that returned hipErrorNotReady counts). Clear it before a
// call's launches so the status reflects this call's launches only.
void clear_stale_error() { (void)hipGetLastError(); }

moe_status launched(hipError_t e) {
  if (e == hipSuccess) return MOE_SUCCESS;
  t_last_launch_error = e;
  return MOE_ERROR_LAUNCH;
}

// Sizes shared by every call; returns the status for invalid/unsupported.
moe_status check_common(int64_t T, int64_t E, int64_t k) {
  if (T < 0 || E < 1 || k < 1) return MOE_ERROR_INVALID_VALUE;
  if (k > E) return MOE_ERROR_INVALID_VALUE;
  if (E > kMaxExperts || k > kMaxTopK) return MOE_ERROR_UNSUPPORTED;
  if (T * k >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

moe_status check_share(int64_t E, int64_t first, int64_t L) {
  if (first < 0 || L < 0 || first + L > E) return MOE_ERROR_INVALID_VALUE;
  return MOE_SUCCESS;
}

moe_status check_dims(int64_t T, int64_t k, int64_t H, int64_t I) {
  if (H < 1 || I < 1) return MOE_ERROR_INVALID_VALUE;
  const int64_t m = H > I ? H : I;
  if (T * k * m >= kMaxIndex || 2 * I * H >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

// Workspace layout of moe_forward; every region starts 256-byte aligned.
struct Layout {
  size_t logits, ids, weights, counts, offsets, perm, e2p, router_ws, permute_ws, ffn_ws, expert_out,
      total;
};

Layout layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t L) {
  Layout o{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    size_t here = at;
    at += align256(bytes > 0 ? bytes : 1);
    return here;
  };
  const size_t n = (size_t)T * k;
  o.logits = take((size_t)T * E * 4);
  o.ids = take(n * 4);
  o.weights = take(n * 4);
  o.counts = take((size_t)E * 4);
  o.offsets = take((size_t)(L + 1) * 4);
  o.perm = take(n * 4);
  o.e2p = take(n * 4);
  o.router_ws = take(moe::router_workspace_bytes((int)T, (int)H, (int)E));
  o.permute_ws = take(moe::permute_workspace_bytes((int)T, (int)E, (int)L));
  o.ffn_ws = take(moe::ffn_workspace_bytes((int)T, (int)k, (int)I, (int)L));
  o.expert_out = take(n * (size_t)H * 4);
  o.total = at;
  return o;
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// The layer for one expert share: router logits, route, permute, the grouped
// FFN that `ffn` launches (bf16 or FP8 weights, w1 / w2 the code or value
// arrays), combine. Arguments are checked before any launch; weights_given
// says whether the FFN's weight pointers are all non-NULL. When the
// persistent FFN kernels run, the routing's permutation kernel writes their
// pass plan (one launch fewer: the FFN is told plan_ready).
template <class Ffn>
moe_status forward_layer(const uint16_t* x, const float* w_gate, const float* router_bias,
                         int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                         int32_t first_expert, int32_t num_local, uint16_t* y, float* logits_out,
                         int32_t* topk_ids_out, float* topk_weights_out, void* ws,
                         size_t ws_bytes, void* stream, bool weights_given, const void* w1,
                         const void* w2, bool f8, Ffn ffn) {
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, first_expert, num_local);
  if (st == MOE_SUCCESS) st = check_dims(T, k, H, I);
  if (st != MOE_SUCCESS) return st;
  if ((int64_t)T * E >= kMaxIndex || (int64_t)E * H >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !w_gate || !y || (num_local > 0 && !weights_given)) return MOE_ERROR_INVALID_VALUE;
  const Layout lo = layout(T, H, I, E, k, num_local);
  if (!ws || ws_bytes < lo.total || !aligned256(ws)) return MOE_ERROR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(base + lo.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + lo.ids);
  float* wts = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(base + lo.weights);
  int32_t* counts = reinterpret_cast<int32_t*>(base + lo.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + lo.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(base + lo.perm);
  int32_t* e2p = reinterpret_cast<int32_t*>(base + lo.e2p);
  float* eo = reinterpret_cast<float*>(base + lo.expert_out);
  hipStream_t s = as_stream(stream);

  moe::PlanOut po{};
  const bool plan_ready = num_local > 0 && moe::ffn_plan_target(x, w1, w2, eo, T, k, num_local, H,
                                                                I, f8, base + lo.ffn_ws, &po);

  clear_stale_error();
  hipError_t err =
      moe::launch_router_logits(x, w_gate, router_bias, T, H, E, logits, base + lo.router_ws, s);
  if (err == hipSuccess)
    err = moe::launch_route_permute(moe::routing_plan(T, E, k, num_local), logits, T, E, k,
                                    first_expert, num_local, ids, wts, counts, offsets, perm, e2p,
                                    base + lo.permute_ws, po, s);
  if (err == hipSuccess && num_local > 0)
    err = ffn(perm, offsets, eo, base + lo.ffn_ws, plan_ready, s);
  if (err == hipSuccess) err = moe::launch_combine(eo, e2p, wts, T, k, H, y, s);
  return launched(err);
}

// ---- scratch for moe_forward_no_alloc ---------------------------------
// A file-scope device array that stands in for the workspace of callers that
// cannot allocate. Each GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure;
// *err then holds the HIP error).
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_SUCCESS: return "MOE_SUCCESS";
    case MOE_ERROR_INVALID_VALUE: return "MOE_ERROR_INVALID_VALUE";
    case MOE_ERROR_UNSUPPORTED: return "MOE_ERROR_UNSUPPORTED";
    case MOE_ERROR_WORKSPACE: return "MOE_ERROR_WORKSPACE";
    case MOE_ERROR_LAUNCH: return "MOE_ERROR_LAUNCH";
  }
  return "MOE_ERROR_UNKNOWN";
}

const char* moe_last_launch_error(void) { return hipGetErrorName(t_last_launch_error); }

moe_status moe_partition(int32_t E, int32_t S, int32_t s, int32_t* first_expert,
                         int32_t* num_local) {
  if (!first_expert || !num_local || E < 1 || S < 1 || s < 0 || s >= S)
    return MOE_ERROR_INVALID_VALUE;
  const int32_t base = E / S, rem = E % S;
  // Shares before s: every one holds base experts, and the first min(s, rem)
  // of them one more.
  *first_expert = s * base + (s < rem ? s : rem);
  *num_local = base + (s < rem ? 1 : 0);
  return MOE_SUCCESS;
}

moe_status moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                              int32_t num_local, size_t* bytes) {
  if (!bytes) return MOE_ERROR_INVALID_VALUE;
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, 0, num_local);
  if (st == MOE_SUCCESS) st = check_dims(T, k, H, I);
  if (st != MOE_SUCCESS) return st;
  *bytes = layout(T, H, I, E, k, num_local).total;
  return MOE_SUCCESS;
}

moe_status moe_router_logits(const uint16_t* x, const float* w_gate, const float* bias, int32_t T,
                             int32_t H, int32_t E, float* logits, void* ws, size_t ws_bytes,
                             void* stream) {
  if (T < 0 || H < 1 || E < 1) return MOE_ERROR_INVALID_VALUE;
  if (E > kMaxExperts || (int64_t)T * H >= kMaxIndex || (int64_t)E * H >= kMaxIndex ||
      (int64_t)T * E >= kMaxIndex)
    return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !w_gate || !logits) return MOE_ERROR_INVALID_VALUE;
  const size_t need = moe::router_workspace_bytes(T, H, E);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return MOE_ERROR_WORKSPACE;
  clear_stale_error();
  return launched(
      moe::launch_router_logits(x, w_gate, bias, T, H, E, logits, ws, as_stream(stream)));
}

moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_weights, void* stream) {
  moe_status st = check_common(T, E, k);
  if (st != MOE_SUCCESS) return st;
  if ((int64_t)T * E >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERROR_INVALID_VALUE;
  clear_stale_error();
  return launched(moe::launch_route(logits, T, E, k, topk_ids, topk_weights, as_stream(stream)));
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t first_expert, int32_t num_local, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* permuted_rows,
                       int32_t* expanded_to_permuted, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, first_expert, num_local);
  if (st != MOE_SUCCESS) return st;
  if (T == 0) return MOE_SUCCESS;
  if (!topk_ids || !expert_counts || !expert_offsets || !permuted_rows || !expanded_to_permuted)
    return MOE_ERROR_INVALID_VALUE;
  const size_t need = moe::permute_workspace_bytes(T, E, num_local);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return MOE_ERROR_WORKSPACE;
  clear_stale_error();
  return launched(moe::launch_permute(topk_ids, T, k, E, first_expert, num_local, expert_counts,
                                      expert_offsets, permuted_rows, expanded_to_permuted, ws,
                                      as_stream(stream)));
}

moe_status moe_routing_plan(int32_t T, int32_t E, int32_t k, int32_t num_local,
                            int32_t* variant) {
  if (!variant) return MOE_ERROR_INVALID_VALUE;
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, 0, num_local);
  if (st != MOE_SUCCESS) return st;
  *variant = moe::routing_plan(T, E, k, num_local);
  return MOE_SUCCESS;
}

moe_status moe_route_permute_variant(const float* logits, int32_t T, int32_t E, int32_t k,
                                     int32_t first_expert, int32_t num_local, int32_t* topk_ids,
                                     float* topk_weights, int32_t* expert_counts,
                                     int32_t* expert_offsets, int32_t* permuted_rows,
                                     int32_t* expanded_to_permuted, void* ws, size_t ws_bytes,
                                     int32_t variant, void* stream) {
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, first_expert, num_local);
  if (st != MOE_SUCCESS) return st;
  if ((int64_t)T * E >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  if (variant < MOE_ROUTING_AUTO || variant > MOE_ROUTING_TILED) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!logits || !topk_ids || !topk_weights || !expert_counts || !expert_offsets ||
      !permuted_rows || !expanded_to_permuted)
    return MOE_ERROR_INVALID_VALUE;
  if (variant == MOE_ROUTING_AUTO) variant = moe::routing_plan(T, E, k, num_local);
  if (!moe::routing_variant_applies(variant, T, E, num_local)) return MOE_ERROR_UNSUPPORTED;
  const size_t need = moe::permute_workspace_bytes(T, E, num_local);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return MOE_ERROR_WORKSPACE;
  clear_stale_error();
  return launched(moe::launch_route_permute(variant, logits, T, E, k, first_expert, num_local,
                                            topk_ids, topk_weights, expert_counts, expert_offsets,
                                            permuted_rows, expanded_to_permuted, ws, moe::PlanOut{},
                                            as_stream(stream)));
}

moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t first_expert, int32_t num_local, int32_t* topk_ids,
                             float* topk_weights, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* permuted_rows, int32_t* expanded_to_permuted, void* ws,
                             size_t ws_bytes, void* stream) {
  return moe_route_permute_variant(logits, T, E, k, first_expert, num_local, topk_ids,
                                   topk_weights, expert_counts, expert_offsets, permuted_rows,
                                   expanded_to_permuted, ws, ws_bytes, MOE_ROUTING_AUTO, stream);
}

moe_status moe_grouped_ffn(const uint16_t* x, const int32_t* permuted_rows,
                           const int32_t* expert_offsets, int32_t num_local, int32_t T, int32_t k,
                           int32_t H, int32_t I, const uint16_t* w1, const uint16_t* w2,
                           float* expert_out, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || num_local < 0) return MOE_ERROR_INVALID_VALUE;
  if (k > kMaxTopK || num_local > kMaxExperts || (int64_t)T * k >= kMaxIndex)
    return MOE_ERROR_UNSUPPORTED;
  moe_status st = check_dims(T, k, H, I);
  if (st != MOE_SUCCESS) return st;
  if (T == 0 || num_local == 0) return MOE_SUCCESS;
  if (!x || !permuted_rows || !expert_offsets || !w1 || !w2 || !expert_out)
    return MOE_ERROR_INVALID_VALUE;
  const size_t need = moe::ffn_workspace_bytes(T, k, I, num_local);
  if (!ws || ws_bytes < need || !aligned256(ws)) return MOE_ERROR_WORKSPACE;
  clear_stale_error();
  return launched(moe::launch_grouped_ffn(x, permuted_rows, expert_offsets, num_local, T, k, H, I,
                                          w1, w2, expert_out, ws, false, as_stream(stream)));
}

moe_status moe_grouped_ffn_fp8(const uint16_t* x, const int32_t* permuted_rows,
                               const int32_t* expert_offsets, int32_t num_local, int32_t T,
                               int32_t k, int32_t H, int32_t I, const uint8_t* w1q,
                               const float* w1s, const uint8_t* w2q, const float* w2s,
                               float* expert_out, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || num_local < 0) return MOE_ERROR_INVALID_VALUE;
  if (k > kMaxTopK || num_local > kMaxExperts || (int64_t)T * k >= kMaxIndex)
    return MOE_ERROR_UNSUPPORTED;
  moe_status st = check_dims(T, k, H, I);
  if (st != MOE_SUCCESS) return st;
  if (T == 0 || num_local == 0) return MOE_SUCCESS;
  if (!x || !permuted_rows || !expert_offsets || !w1q || !w1s || !w2q || !w2s || !expert_out)
    return MOE_ERROR_INVALID_VALUE;
  const size_t need = moe::ffn_workspace_bytes(T, k, I, num_local);
  if (!ws || ws_bytes < need || !aligned256(ws)) return MOE_ERROR_WORKSPACE;
  clear_stale_error();
  return launched(moe::launch_grouped_ffn_fp8(x, permuted_rows, expert_offsets, num_local, T, k, H,
                                              I, w1q, w1s, w2q, w2s, expert_out, ws, false,
                                              as_stream(stream)));
}

moe_status moe_combine(const float* expert_out, const int32_t* expanded_to_permuted,
                       const float* topk_weights, int32_t T, int32_t k, int32_t H, uint16_t* y,
                       void* stream) {
  if (T < 0 || k < 1 || H < 1) return MOE_ERROR_INVALID_VALUE;
  if (k > kMaxTopK || (int64_t)T * k * H >= kMaxIndex) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!expert_out || !expanded_to_permuted || !topk_weights || !y) return MOE_ERROR_INVALID_VALUE;
  clear_stale_error();
  return launched(moe::launch_combine(expert_out, expanded_to_permuted, topk_weights, T, k, H, y,
                                      as_stream(stream)));
}

moe_status moe_forward(const uint16_t* x, const float* w_gate, const float* router_bias,
                       const uint16_t* w1, const uint16_t* w2, int32_t T, int32_t H, int32_t I,
                       int32_t E, int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                       float* logits_out, int32_t* topk_ids_out, float* topk_weights_out,
                       void* ws, size_t ws_bytes, void* stream) {
  return forward_layer(
      x, w_gate, router_bias, T, H, I, E, k, first_expert, num_local, y, logits_out,
      topk_ids_out, topk_weights_out, ws, ws_bytes, stream, w1 && w2, w1, w2, false,
      [&](const int32_t* perm, const int32_t* offsets, float* eo, void* fws, bool ready,
          hipStream_t s) {
        return moe::launch_grouped_ffn(x, perm, offsets, num_local, T, k, H, I, w1, w2, eo, fws,
                                       ready, s);
      });
}

moe_status moe_forward_fp8(const uint16_t* x, const float* w_gate, const float* router_bias,
                           const uint8_t* w1q, const float* w1s, const uint8_t* w2q,
                           const float* w2s, int32_t T, int32_t H, int32_t I, int32_t E,
                           int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                           float* logits_out, int32_t* topk_ids_out, float* topk_weights_out,
                           void* ws, size_t ws_bytes, void* stream) {
  return forward_layer(
      x, w_gate, router_bias, T, H, I, E, k, first_expert, num_local, y, logits_out,
      topk_ids_out, topk_weights_out, ws, ws_bytes, stream, w1q && w1s && w2q && w2s, w1q, w2q,
      true,
      [&](const int32_t* perm, const int32_t* offsets, float* eo, void* fws, bool ready,
          hipStream_t s) {
        return moe::launch_grouped_ffn_fp8(x, perm, offsets, num_local, T, k, H, I, w1q, w1s, w2q,
                                           w2s, eo, fws, ready, s);
      });
}

moe_status moe_forward_no_alloc(const uint16_t* x, const float* w_gate,
                                const float* router_bias, const uint16_t* w1,
                                const uint16_t* w2, int32_t T, int32_t H, int32_t I, int32_t E,
                                int32_t k, int32_t first_expert, int32_t num_local, uint16_t* y,
                                float* logits_out, int32_t* topk_ids_out,
                                float* topk_weights_out, void* stream) {
  moe_status st = check_common(T, E, k);
  if (st == MOE_SUCCESS) st = check_share(E, first_expert, num_local);
  if (st == MOE_SUCCESS) st = check_dims(T, k, H, I);
  if (st != MOE_SUCCESS) return st;
  if (T == 0) return MOE_SUCCESS;
  if (layout(T, H, I, E, k, num_local).total > MOE_NO_ALLOC_SCRATCH_BYTES)
    return MOE_ERROR_WORKSPACE;
  hipError_t err = hipSuccess;
  void* ws = scratch_address(&err);
  if (!ws) {
    t_last_launch_error = err;
    return MOE_ERROR_LAUNCH;
  }
  return moe_forward(x, w_gate, router_bias, w1, w2, T, H, I, E, k, first_expert, num_local, y,
                     logits_out, topk_ids_out, topk_weights_out, ws, MOE_NO_ALLOC_SCRATCH_BYTES,
                     stream);
}

}  // extern "C"
