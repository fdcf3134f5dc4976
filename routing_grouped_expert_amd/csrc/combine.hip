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
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    int p = e2p[(size_t)t * k + threadIdx.x];
    s_p[threadIdx.x] = (p >= 0 && p < nmax) ? p : -1;
    s_w[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  uint16_t* yt = y + (size_t)t * H;
  if (VEC) {
    for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int p = s_p[j];
        if (p < 0) continue;
        const f32x4 v = *reinterpret_cast<const f32x4*>(eo + (size_t)p * H + c);
        const float wj = s_w[j];
        acc[0] = fmaf(wj, v[0], acc[0]);
        acc[1] = fmaf(wj, v[1], acc[1]);
        acc[2] = fmaf(wj, v[2], acc[2]);
        acc[3] = fmaf(wj, v[3], acc[3]);
      }
      typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
      *reinterpret_cast<u16x4*>(yt + c) =
          u16x4{f32_to_bf16_bits(acc[0]), f32_to_bf16_bits(acc[1]), f32_to_bf16_bits(acc[2]),
                f32_to_bf16_bits(acc[3])};
    }
  } else {
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) {
        const int p = s_p[j];
        if (p < 0) continue;
        acc = fmaf(s_w[j], eo[(size_t)p * H + c], acc);
      }
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
