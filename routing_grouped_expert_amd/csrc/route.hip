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
// Selection: k rounds of a wave-wide maximum over 64-bit keys
//   key = (order-preserving bits of the logit) << 32 | (0xFFFFFFFF - id)
// so the larger logit wins and, on equal logits, the lower id; -0 is folded
// onto +0 first so the two compare equal. Weights: w_j = exp(l_j - l_0) /
// sum_i exp(l_i - l_0) over the k selected logits (the full-softmax
// normaliser cancels in the renormalisation).
#include "device.h"

namespace moe {

namespace {

__device__ __forceinline__ uint64_t make_key(float v, int id) {
  v = v + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(v);
  uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(mono) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(id));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t mono = static_cast<uint32_t>(key >> 32);
  uint32_t u = (mono & 0x80000000u) ? (mono & 0x7FFFFFFFu) : ~mono;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// Lane-local top two of the keys below `limit` (0 = none).
template <int VPL>
__device__ __forceinline__ void top2_below(const uint64_t (&key)[VPL], uint64_t limit, uint64_t& h1,
                                           uint64_t& h2) {
  h1 = 0;
  h2 = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint64_t k = key[i] < limit ? key[i] : 0ull;
    const bool c1 = k > h1, c2 = k > h2;
    h2 = c1 ? h1 : (c2 ? k : h2);
    h1 = c1 ? k : h1;
  }
}

// Selection: every lane keeps the two largest of its keys not yet taken
// (h1 > h2). A round takes the wave-wide maximum of the h1s; the lane that
// held it moves h2 up, and when it wins a second time (its h2 already moved
// up) it rescans its keys below the last one it gave. Lane j keeps the key
// taken in round j.
// VEC (E a multiple of 4, 16-byte aligned logits, VPL >= 4): a lane loads its
// values as groups of 4 consecutive experts, expert 4 (lane + 64 g) + c.
template <int VPL, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int* __restrict__ ids,
                                                   float* __restrict__ weights) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves leave: every selection round runs on a full wave
  const float* l = logits + (size_t)t * E;
  uint64_t key[VPL];
  if constexpr (VEC) {
    f32x4 v[VPL / 4];
#pragma unroll
    for (int g = 0; g < VPL / 4; ++g) {
      const int e = 4 * (lane + kWave * g);
      v[g] = e < E ? *reinterpret_cast<const f32x4*>(l + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int g = 0; g < VPL / 4; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * (lane + kWave * g) + c;
        key[4 * g + c] = e < E ? make_key(v[g][c], e) : 0ull;  // a valid key is never 0
      }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      key[i] = e < E ? make_key(l[e], e) : 0ull;  // a valid key is never 0
    }
  }
  uint64_t h1, h2;
  top2_below(key, ~0ull, h1, h2);
  bool h2_fresh = true;  // h2 is this lane's second largest key below h1
  uint64_t mine = 0, top = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(h1);
    if (j == 0) top = best;
    if (lane == j) mine = best;
    const bool win = h1 == best;  // keys are unique: one lane
    const bool rescan = win && !h2_fresh;
    if (win) {
      h1 = h2;
      h2_fresh = false;
    }
    if (__builtin_amdgcn_ballot_w64(rescan)) {
      if (rescan) {
        top2_below(key, best, h1, h2);
        h2_fresh = true;
      }
    }
  }
  const float topv = key_value(top);
  const float ex = lane < k ? expf(key_value(mine) - topv) : 0.0f;
  float s = 0.0f;  // sum in slot order
  for (int j = 0; j < k; ++j) s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = key_id(mine);
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
