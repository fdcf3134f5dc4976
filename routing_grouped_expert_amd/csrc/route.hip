// Routing: top-k of each token's fp32 logits, then the softmax renormalised
// over the k selected experts.
//
// Page "TRTLLM-Gen MoE routing optimisation in FlashInfer: relieving register
// pressure" (flashinfer PR #3751), section 1 "Dynamic thread block size":
// the launch shape follows the work (there, the block size follows the token
// count so registers do not spill). Here one wave64 owns one token; the
// kernel is instantiated per values-per-lane tier (E / 64 rounded up to a
// power of two) so a lane keeps its share of the logits in registers
// whatever E is, and the tier table plays the role of that page's section 2
// (valid expert-count / block-size combinations fixed at compile time).
//
// Selection: k rounds of a wave-wide maximum of the order-preserving 32-bit
// image of the logits; on equal logits the lower id wins; -0 is folded onto
// +0 first so the two compare equal. Weights: w_j = exp(l_j - l_0) /
// sum_i exp(l_i - l_0) over the k selected logits (the full-softmax
// normaliser cancels in the renormalisation).
#include "device.h"

namespace moe {

namespace {

// Order-preserving unsigned image of a logit (-0 folded onto +0): larger
// logit, larger value. Lanes past E hold 0, below every logit's image.
__device__ __forceinline__ uint32_t mono(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_mono(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// Selection: every lane keeps the two best of its entries not yet taken
// (h1 before h2 in the order: larger value first, then lower expert). A round
// takes the wave-wide maximum of the h1 values; when several lanes hold it,
// the lowest of their experts (a second reduction, skipped when one lane
// holds it). The winning lane moves h2 up, and when it wins a second time
// (its h2 already moved up) it rescans its entries after the one just taken.
// Lane j keeps the entry taken in round j. A lane's entries are visited in
// increasing expert order, so "greater than" keeps the lower expert on ties.
// VEC (E a multiple of 4, 16-byte aligned logits, VPL >= 4): a lane loads its
// values as groups of 4 consecutive experts, expert 4 (lane + 64 g) + c;
// otherwise entry i of a lane is expert lane + 64 i.
template <int VPL, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int* __restrict__ ids,
                                                   float* __restrict__ weights) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves leave: every selection round runs on a full wave
  const float* l = logits + (size_t)t * E;
  auto expert = [&](int i) -> uint32_t {
    return VEC ? 4 * (lane + kWave * (i / 4)) + (i % 4) : lane + kWave * i;
  };
  uint32_t val[VPL];
  if constexpr (VEC) {
    f32x4 v[VPL / 4];
#pragma unroll
    for (int g = 0; g < VPL / 4; ++g) {
      const int e = 4 * (lane + kWave * g);
      v[g] = e < E ? *reinterpret_cast<const f32x4*>(l + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) val[i] = (int)expert(i) < E ? mono(v[i / 4][i % 4]) : 0u;
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = expert(i);
      val[i] = e < E ? mono(l[e]) : 0u;
    }
  }
  uint32_t h1v = 0, h1e = 0, h2v = 0, h2e = 0;
  // the lane's best two entries after (bv, be) in the selection order
  auto top2 = [&](bool bounded, uint32_t bv, uint32_t be) {
    h1v = 0;
    h2v = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint32_t e = expert(i);
      uint32_t v = val[i];
      if (bounded) v = (v < bv || (v == bv && e > be)) ? v : 0u;
      const bool c1 = v > h1v, c2 = v > h2v;
      h2v = c1 ? h1v : (c2 ? v : h2v);
      h2e = c1 ? h1e : (c2 ? e : h2e);
      h1v = c1 ? v : h1v;
      h1e = c1 ? e : h1e;
    }
  };
  top2(false, 0u, 0u);
  bool h2_fresh = true;  // h2 is this lane's second best below h1
  uint32_t mine_v = 0, mine_e = 0, top_v = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_max_u32(h1v);
    const bool cand = h1v == m;
    const uint64_t cm = __builtin_amdgcn_ballot_w64(cand);
    uint32_t be;
    bool win;
    if (__builtin_popcountll(cm) == 1) {
      be = __builtin_amdgcn_readlane(static_cast<int>(h1e), __builtin_ctzll(cm));
      win = cand;
    } else {
      be = wave_min_u32(cand ? h1e : 0xFFFFFFFFu);
      win = cand && h1e == be;
    }
    if (j == 0) top_v = m;
    if (lane == j) {
      mine_v = m;
      mine_e = be;
    }
    const bool rescan = win && !h2_fresh;
    if (win) {
      h1v = h2v;
      h1e = h2e;
      h2_fresh = false;
    }
    if (__builtin_amdgcn_ballot_w64(rescan)) {
      if (rescan) {
        top2(true, m, be);
        h2_fresh = true;
      }
    }
  }
  const float topf = from_mono(top_v);
  const float ex = lane < k ? expf(from_mono(mine_v) - topf) : 0.0f;
  float s = 0.0f;  // sum in slot order
  for (int j = 0; j < k; ++j) s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = static_cast<int>(mine_e);
    weights[(size_t)t * k + lane] = ex / s;
  }
}

template <int VPL>
hipError_t launch_tier(const float* logits, int T, int E, int k, int* ids, float* w,
                       hipStream_t stream) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block);
  const bool vec = VPL >= 4 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
  if constexpr (VPL >= 4) {
    if (vec) {
      hipLaunchKernelGGL((route_kernel<VPL, true>), grid, dim3(waves_per_block * kWave), 0, stream,
                         logits, T, E, k, ids, w);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_kernel<VPL, false>), grid, dim3(waves_per_block * kWave), 0, stream,
                     logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t stream) {
  if (E <= 64) return launch_tier<1>(logits, T, E, k, ids, w, stream);
  if (E <= 128) return launch_tier<2>(logits, T, E, k, ids, w, stream);
  if (E <= 256) return launch_tier<4>(logits, T, E, k, ids, w, stream);
  if (E <= 512) return launch_tier<8>(logits, T, E, k, ids, w, stream);
  if (E <= 1024) return launch_tier<16>(logits, T, E, k, ids, w, stream);
  if (E <= 2048) return launch_tier<32>(logits, T, E, k, ids, w, stream);
  return launch_tier<64>(logits, T, E, k, ids, w, stream);
}

}  // namespace moe
