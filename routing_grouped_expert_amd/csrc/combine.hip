// Routing-weighted combine back to token order:
//   y[t, :] = bf16( sum_{j ascending} w[t, j] * expert_out[e2p[t*k + j], :] )
// skipping e2p = -1 (experts outside the share). The sum stays fp32 until the
// single round-to-nearest-even at the store (page "Attention optimisation for
// Hopper (SM90): FlashInfer 'Cake' backend", flashinfer PR #5586, section 3:
// partial results stay fp32 to the end).
// One block per token; 16-byte loads of expert rows, 8-byte bf16 stores.
#include "device.h"

namespace moe {

namespace {
constexpr int MAXK = 32;

template <bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ eo,
                                                      const int* __restrict__ e2p,
                                                      const float* __restrict__ w, int k, int H,
                                                      int nmax, uint16_t* __restrict__ y) {
  __shared__ int s_p[MAXK];
  __shared__ float s_w[MAXK];
  __shared__ int s_n;
  const int t = blockIdx.x;
  // The selections inside the share, compacted in ascending j (wave 0).
  if (threadIdx.x < kWave) {
    const int j = threadIdx.x;
    int p = -1;
    float wj = 0.f;
    if (j < k) {
      p = e2p[(size_t)t * k + j];
      wj = w[(size_t)t * k + j];
    }
    const bool on = j < k && p >= 0 && p < nmax;
    const uint64_t m = __ballot(on);
    if (on) {
      const int pos = __popcll(m & ((1ull << j) - 1));
      s_p[pos] = p;
      s_w[pos] = wj;
    }
    if (j == 0) s_n = __popcll(m);
  }
  __syncthreads();
  const int nv = s_n;
  uint16_t* yt = y + (size_t)t * H;
  if (VEC) {
    // Up to 8 column chunks of 1024 per round; for each selection the
    // chunks' loads are issued together, so a round waits for memory once per
    // selection inside the share.
    constexpr int CH = 8;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    for (int c0 = threadIdx.x * 4; c0 < H; c0 += CH * blockDim.x * 4) {
      f32x4 acc[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < nv; ++j) {
        const float wj = s_w[j];
        const float* row = eo + (size_t)s_p[j] * H;
        f32x4 v[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int c = c0 + i * blockDim.x * 4;
          v[i] = c < H ? *reinterpret_cast<const f32x4*>(row + c) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          acc[i][0] = fmaf(wj, v[i][0], acc[i][0]);
          acc[i][1] = fmaf(wj, v[i][1], acc[i][1]);
          acc[i][2] = fmaf(wj, v[i][2], acc[i][2]);
          acc[i][3] = fmaf(wj, v[i][3], acc[i][3]);
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = c0 + i * blockDim.x * 4;
        if (c < H)
          *reinterpret_cast<u16x4*>(yt + c) =
              u16x4{f32_to_bf16_bits(acc[i][0]), f32_to_bf16_bits(acc[i][1]),
                    f32_to_bf16_bits(acc[i][2]), f32_to_bf16_bits(acc[i][3])};
      }
    }
  } else {
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
      float acc = 0.f;
      for (int j = 0; j < nv; ++j) acc = fmaf(s_w[j], eo[(size_t)s_p[j] * H + c], acc);
      yt[c] = f32_to_bf16_bits(acc);
    }
  }
}
}  // namespace

hipError_t launch_combine(const float* eo, const int* e2p, const float* w, int T, int k, int H,
                          uint16_t* y, hipStream_t stream) {
  const bool vec = H % 4 == 0 && (reinterpret_cast<uintptr_t>(eo) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 7u) == 0;
  if (vec)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, stream, eo, e2p, w, k, H, T * k,
                       y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, stream, eo, e2p, w, k, H,
                       T * k, y);
  return hipGetLastError();
}

}  // namespace moe
