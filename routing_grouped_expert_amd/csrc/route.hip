// Routing: top-k of each token's fp32 logits, then the softmax renormalised
// over the k selected experts (selection and weights: select.h).
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
// Two forms of the kernel:
//  - route_kernel<..., false>: 4 waves (tokens) per block; moe_route.
//  - route_kernel<..., true>: 16 waves per block, one 16-token slice of a
//    64-token tile; besides ids and weights it writes that slice of the
//    tile's 64-bit token masks per expert (masks[tile][e], 16 bits of it),
//    the input of the permutation's scan, so the layer needs no separate
//    mask kernel.
#include "select.h"

namespace moe {

namespace {

constexpr int kMaskWaves = 16;  // tokens per block of the masked form

template <int VPL, bool VEC, bool MASKS>
__global__ __launch_bounds__(MASKS ? kMaskWaves * kWave : 4 * kWave) void route_kernel(
    const float* __restrict__ logits, int T, int E, int k, int* __restrict__ ids,
    float* __restrict__ weights, uint16_t* __restrict__ masks16) {
  constexpr int NW = MASKS ? kMaskWaves : 4;
  constexpr bool THRESH = VPL >= 4;
  __shared__ unsigned long long cand[THRESH ? NW : 1][THRESH ? kWave : 1];
  extern __shared__ uint32_t msk[];  // MASKS: E token masks of this slice
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t = blockIdx.x * NW + wave;
  float v[VPL];
  if (t < T) sel::load_logits<VPL, VEC>(logits + (size_t)t * E, lane, E, v);
  if constexpr (MASKS) {  // (the logits are in flight meanwhile)
    for (int e = threadIdx.x; e < E; e += NW * kWave) msk[e] = 0u;
    __syncthreads();
  }
  if (t < T) {
    const uint32_t e =
        sel::route_token<VPL, VEC, THRESH>(v, lane, E, k, &cand[THRESH ? wave : 0][0], ids, weights,
                                           (size_t)t);
    if constexpr (MASKS) {
      if (lane < k) atomicOr(&msk[e], 1u << wave);
    }
  }
  if constexpr (MASKS) {
    __syncthreads();
    // slice s = blockIdx % 4 of tile blockIdx / 4: bits 16 s .. 16 s + 15 of
    // each 64-bit mask (little-endian: the s-th 16-bit half-word)
    const int tile = blockIdx.x / 4, s = blockIdx.x % 4;
    const bool last = blockIdx.x == (int)gridDim.x - 1;
    for (int e = threadIdx.x; e < E; e += NW * kWave) {
      uint16_t* w = masks16 + ((size_t)tile * E + e) * 4;
      w[s] = static_cast<uint16_t>(msk[e]);
      if (last)  // slices of the last tile past T: no tokens
        for (int q = s + 1; q < 4; ++q) w[q] = 0;
    }
  }
}

template <int VPL, bool MASKS>
hipError_t launch_tier(const float* logits, int T, int E, int k, int* ids, float* w,
                       uint16_t* masks16, hipStream_t stream) {
  constexpr int NW = MASKS ? kMaskWaves : 4;
  dim3 grid((T + NW - 1) / NW);
  const size_t lds = MASKS ? (size_t)E * 4 : 0;
  const bool vec = VPL >= 4 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
  if constexpr (VPL >= 4) {
    if (vec) {
      hipLaunchKernelGGL((route_kernel<VPL, true, MASKS>), grid, dim3(NW * kWave), lds, stream,
                         logits, T, E, k, ids, w, masks16);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_kernel<VPL, false, MASKS>), grid, dim3(NW * kWave), lds, stream,
                     logits, T, E, k, ids, w, masks16);
  return hipGetLastError();
}

template <bool MASKS>
hipError_t launch_any(const float* logits, int T, int E, int k, int* ids, float* w,
                      uint16_t* masks16, hipStream_t stream) {
  if (E <= 64) return launch_tier<1, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  if (E <= 128) return launch_tier<2, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  if (E <= 256) return launch_tier<4, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  if (E <= 512) return launch_tier<8, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  if (E <= 1024) return launch_tier<16, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  if (E <= 2048) return launch_tier<32, MASKS>(logits, T, E, k, ids, w, masks16, stream);
  return launch_tier<64, MASKS>(logits, T, E, k, ids, w, masks16, stream);
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t stream) {
  return launch_any<false>(logits, T, E, k, ids, w, nullptr, stream);
}

// Routing of T tokens that also writes the 64-token tile masks
// (masks [ceil(T / 64), E] u64).
hipError_t launch_route_masks(const float* logits, int T, int E, int k, int* ids, float* w,
                              unsigned long long* masks, hipStream_t stream) {
  return launch_any<true>(logits, T, E, k, ids, w, reinterpret_cast<uint16_t*>(masks), stream);
}

}  // namespace moe
