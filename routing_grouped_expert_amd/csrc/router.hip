// Router logits: logits[t, e] = fp32( sum_h x[t, h] * w_gate[e, h] + bias[e] ).
//
// The pages leave the router unstated. The logit is defined as the fp32
// value of the exact affine map: x is bf16 and w_gate fp32, so each product
// is exact in fp64; the sum is carried in fp64 (any order agrees to ~1e-15
// relative) and rounded to fp32 once, after the bias. The top-k decision is
// then taken on these fp32 values.
//
// Two shapes of the same computation:
//  - few tokens (decode): one block per (token, 8 experts); the 256 threads
//    split H, each keeps 8 fp64 partial sums, and the block adds them up in a
//    fixed order (butterfly within a wave, then wave 0..3);
//  - many tokens: VALU fp64 GEMM tiled through LDS, 64 tokens x 64 experts
//    per 256-thread block, each thread a 4 x 4 register tile.
#include "device.h"

namespace moe {

namespace {
constexpr int RT = 64;  // tokens per block
constexpr int RE = 64;  // experts per block
constexpr int RK = 32;  // K chunk

template <bool HAS_BIAS>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            const float* __restrict__ bias, int T,
                                                            int H, int E,
                                                            float* __restrict__ logits) {
  __shared__ double xs[RK][RT + 2];
  __shared__ double ws[RK][RE + 2];
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * RE;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int h0 = 0; h0 < H; h0 += RK) {
    // Stage x[t0:t0+64, h0:h0+32] and w_gate[e0:e0+64, h0:h0+32] as fp64.
    for (int q = threadIdx.x; q < RT * RK; q += 256) {
      const int r = q / RK, c = q % RK;
      const int t = t0 + r, h = h0 + c;
      xs[c][r] = (t < T && h < H) ? (double)bf16_bits_to_f32(x[(size_t)t * H + h]) : 0.0;
      const int e = e0 + r;
      ws[c][r] = (e < E && h < H) ? (double)wg[(size_t)e * H + h] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < RK; ++c) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e >= E) continue;
      double v = acc[i][j];
      if (HAS_BIAS) v += (double)bias[e];
      logits[(size_t)t * E + e] = (float)v;
    }
  }
}
constexpr int SE = 8;  // experts per block in the few-token kernel

template <bool HAS_BIAS, bool VEC>
__global__ __launch_bounds__(256) void router_rows_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          const float* __restrict__ bias, int H,
                                                          int E, float* __restrict__ logits) {
  __shared__ double part[4][SE];
  const int t = blockIdx.x, e0 = blockIdx.y * SE;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int ne = min(SE, E - e0);
  const uint16_t* xr = x + (size_t)t * H;
  const float* wr = wg + (size_t)e0 * H;
  double acc[SE];
#pragma unroll
  for (int j = 0; j < SE; ++j) acc[j] = 0.0;
  if (VEC) {
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    for (int h = tid * 4; h < H; h += 256 * 4) {
      const u16x4 xv = *reinterpret_cast<const u16x4*>(xr + h);
      const double x0 = bf16_bits_to_f32(xv[0]), x1 = bf16_bits_to_f32(xv[1]);
      const double x2 = bf16_bits_to_f32(xv[2]), x3 = bf16_bits_to_f32(xv[3]);
#pragma unroll
      for (int j = 0; j < SE; ++j) {
        if (j < ne) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(wr + (size_t)j * H + h);
          acc[j] = fma(x0, (double)w[0], acc[j]);
          acc[j] = fma(x1, (double)w[1], acc[j]);
          acc[j] = fma(x2, (double)w[2], acc[j]);
          acc[j] = fma(x3, (double)w[3], acc[j]);
        }
      }
    }
  } else {
    for (int h = tid; h < H; h += 256) {
      const double xv = bf16_bits_to_f32(xr[h]);
#pragma unroll
      for (int j = 0; j < SE; ++j)
        if (j < ne) acc[j] = fma(xv, (double)wr[(size_t)j * H + h], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < SE; ++j) {
    double v = acc[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    if (lane == 0) part[wave][j] = v;
  }
  __syncthreads();
  if (tid < ne) {
    double v = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    if (HAS_BIAS) v += (double)bias[e0 + tid];
    logits[(size_t)t * E + e0 + tid] = (float)v;
  }
}

}  // namespace

// Up to this many tokens the few-token kernel runs.
constexpr int kRowsMaxTokens = 64;

hipError_t launch_router_logits(const uint16_t* x, const float* wg, const float* bias, int T, int H,
                                int E, float* logits, hipStream_t stream) {
  if (T <= kRowsMaxTokens) {
    const bool vec = H % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 7u) == 0 &&
                     (reinterpret_cast<uintptr_t>(wg) & 15u) == 0;
    dim3 g(T, (E + SE - 1) / SE);
    if (bias) {
      if (vec)
        hipLaunchKernelGGL((router_rows_kernel<true, true>), g, dim3(256), 0, stream, x, wg, bias,
                           H, E, logits);
      else
        hipLaunchKernelGGL((router_rows_kernel<true, false>), g, dim3(256), 0, stream, x, wg,
                           bias, H, E, logits);
    } else {
      if (vec)
        hipLaunchKernelGGL((router_rows_kernel<false, true>), g, dim3(256), 0, stream, x, wg,
                           bias, H, E, logits);
      else
        hipLaunchKernelGGL((router_rows_kernel<false, false>), g, dim3(256), 0, stream, x, wg,
                           bias, H, E, logits);
    }
    return hipGetLastError();
  }
  dim3 grid((T + RT - 1) / RT, (E + RE - 1) / RE);
  if (bias)
    hipLaunchKernelGGL(router_logits_kernel<true>, grid, dim3(256), 0, stream, x, wg, bias, T, H, E,
                       logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<false>, grid, dim3(256), 0, stream, x, wg, bias, T, H,
                       E, logits);
  return hipGetLastError();
}

}  // namespace moe
