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
//  - many tokens: fp64 MFMA GEMM, split over K into slices whose fp64 partial
//    sums a second kernel adds in slice order.
#include "device.h"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {
// ---- many tokens: fp64 MFMA (v_mfma_f64_16x16x4f64) ----------------------
// Any H and alignment (the full-chunk kernel below serves H a multiple of 32
// with 16-byte aligned rows): block tile 64 tokens x 64 experts, 4 waves of 32 x 32 (2 x 2 MFMA tiles),
// K staged through LDS in chunks of 32 as fp64 (k-major, so each 16-lane
// group of a fragment read is one contiguous 128-byte row). The K range is
// split over blockIdx.z; each slice writes fp64 partial sums, which a second
// kernel adds in slice order (then the bias) and rounds to fp32 once.
// fp64 MFMA layouts: A lane l = A[l % 16][l / 16], B lane l = B[l / 16][l % 16],
// D lane l, register r = D[l / 16 + 4 r][l % 16].
constexpr int MT = 64, MN = 64, MK = 32;
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <bool VEC>
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg, int T,
                                                          int H, int E, int kslice,
                                                          double* __restrict__ part) {
  __shared__ double xs[MK][MT];
  __shared__ double ws[MK][MN];
  const int t0 = blockIdx.x * MT, e0 = blockIdx.y * MN;
  const int kb0 = blockIdx.z * kslice, kb1 = min(H, kb0 + kslice);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  // staging: thread -> (row, 8 consecutive k)
  const int srow = tid >> 2, sk = (tid & 3) * 8;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = kb0; k0 < kb1; k0 += MK) {
    {
      const int t = t0 + srow, e = e0 + srow, kk = k0 + sk;
      double xv[8], wv[8];
      if (VEC && kk + 8 <= kb1) {
        u16x8 xr = {0, 0, 0, 0, 0, 0, 0, 0};
        f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
        if (t < T) xr = *reinterpret_cast<const u16x8*>(x + (size_t)t * H + kk);
        if (e < E) {
          w0 = *reinterpret_cast<const f32x4*>(wg + (size_t)e * H + kk);
          w1 = *reinterpret_cast<const f32x4*>(wg + (size_t)e * H + kk + 4);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = bf16_bits_to_f32(xr[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[j] = w0[j];
          wv[4 + j] = w1[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = kk + j < kb1;
          xv[j] = (ok && t < T) ? (double)bf16_bits_to_f32(x[(size_t)t * H + kk + j]) : 0.0;
          wv[j] = (ok && e < E) ? (double)wg[(size_t)e * H + kk + j] : 0.0;
        }
      }
      __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xs[sk + j][srow] = xv[j];
        ws[sk + j][srow] = wv[j];
      }
      __syncthreads();
    }
#pragma unroll
    for (int s4 = 0; s4 < MK / 4; ++s4) {
      const int kr = s4 * 4 + (lane >> 4);
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = xs[kr][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ws[kr][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  double* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * 32 + i * 16 + (lane >> 4) + 4 * r;
        if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
      }
    }
}

// The same GEMM for full chunks (H a multiple of 32, 16-byte aligned rows),
// on 128-token tiles (4 waves of 64 tokens x 32 experts: 4 x 2 MFMA tiles, so
// each fragment read from LDS feeds 2 or 4 MFMAs). x and w_gate are staged in
// LDS as they are (bf16 bits, fp32), row-major with one 16-byte store per
// piece, and widened to fp64 as the fragments are read. The rows are padded
// to 80 and 144 bytes (20 and 36 banks apart), so the 16 rows a fragment read
// touches at one K fall in different banks. Two LDS buffers, and the next
// chunk's global loads are issued before the current chunk's MFMAs, so one
// barrier per chunk and no wait on HBM inside it. Rows past T or E load the
// last valid row (their results are never stored), so every load is
// unconditional.
// Measured at share 0 (T4096 H7168 E384): 394-416 us, against 406-427 us
// with K-major tiles filled by 2- and 4-byte transposing stores, 414 us with
// 64 x 64 wave tiles (225 VGPRs, 2 blocks per CU), 414-427 us with 64-wide
// chunks (half the barriers; 170 VGPRs, 2 blocks per CU), and no change when
// the K slices were chosen to fill whole rounds of resident blocks.
constexpr int FT = 128;              // tokens per block tile
constexpr int XLD = MK + 8, WLD = MK + 4;  // LDS row lengths (elements)
// At most 168 registers (3 blocks per CU; the kernel takes 122, so 4 fit).
__global__ __launch_bounds__(256, 3) void router_mfma_full_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ wg,
                                                               int T, int H, int E, int kslice,
                                                               double* __restrict__ part) {
  constexpr int TI = FT / 32;  // MFMA token tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][FT][XLD];  // token-major
  __shared__ __attribute__((aligned(16))) float ws[2][MN][WLD];      // expert-major
  const int t0 = blockIdx.x * FT, e0 = blockIdx.y * MN;
  const int kb0 = blockIdx.z * kslice, kb1 = min(H, kb0 + kslice);
  const int nch = (kb1 - kb0) / MK;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  // staging: thread -> (row, 8 consecutive k); x rows srow and srow + 64
  const int srow = tid >> 2, sk = (tid & 3) * 8;
  const uint16_t* xrow0 = x + (size_t)min(t0 + srow, T - 1) * H + kb0 + sk;
  const uint16_t* xrow1 = x + (size_t)min(t0 + 64 + srow, T - 1) * H + kb0 + sk;
  const float* wrow = wg + (size_t)min(e0 + srow, E - 1) * H + kb0 + sk;
  u16x8 xr0, xr1;
  f32x4 w0, w1;
  auto load = [&](int c) {
    xr0 = *reinterpret_cast<const u16x8*>(xrow0 + c * MK);
    xr1 = *reinterpret_cast<const u16x8*>(xrow1 + c * MK);
    w0 = *reinterpret_cast<const f32x4*>(wrow + c * MK);
    w1 = *reinterpret_cast<const f32x4*>(wrow + c * MK + 4);
  };
  auto store = [&](int buf) {
    *reinterpret_cast<u16x8*>(&xs[buf][srow][sk]) = xr0;
    *reinterpret_cast<u16x8*>(&xs[buf][64 + srow][sk]) = xr1;
    *reinterpret_cast<f32x4*>(&ws[buf][srow][sk]) = w0;
    *reinterpret_cast<f32x4*>(&ws[buf][srow][sk + 4]) = w1;
  };
  f64x4 acc[TI][2];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    load(c + 1 < nch ? c + 1 : c);  // past the last chunk: reloaded, unused
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
#pragma unroll
    for (int s4 = 0; s4 < MK / 4; ++s4) {
      const int kr = s4 * 4 + (lane >> 4);
      double a[TI], b[2];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = bf16_bits_to_f32(xs[buf][wm * (FT / 2) + i * 16 + (lane & 15)][kr]);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ws[buf][wn * 32 + j * 16 + (lane & 15)][kr];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    store(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }
  double* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * (FT / 2) + i * 16 + (lane >> 4) + 4 * r;
        if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
      }
    }
}

// logits = fp32(sum over slices in order + bias)
template <bool HAS_BIAS>
__global__ __launch_bounds__(256) void router_reduce_kernel(const double* __restrict__ part,
                                                            const float* __restrict__ bias,
                                                            int T, int E, int nslices,
                                                            float* __restrict__ logits) {
  const size_t n = (size_t)T * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    double v = part[i];
    for (int z = 1; z < nslices; ++z) v += part[(size_t)z * n + i];
    if (HAS_BIAS) v += (double)bias[i % E];
    logits[i] = (float)v;
  }
}

constexpr int SE = 8;  // experts per block in the few-token kernel

// Sum over a full wave of fp64 values in a fixed order: rotations by 1, 2, 4,
// 8 within each row of 16 lanes (DPP), then the four row sums in row order.
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto rot = [](double x, auto ctrl) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    return __builtin_bit_cast(double, dpp_u64<decltype(ctrl)::value>(u));
  };
  v += rot(v, std::integral_constant<int, 0x121>{});
  v += rot(v, std::integral_constant<int, 0x122>{});
  v += rot(v, std::integral_constant<int, 0x124>{});
  v += rot(v, std::integral_constant<int, 0x128>{});
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  double r = __builtin_bit_cast(double, readlane_u64(u, 0));
  r += __builtin_bit_cast(double, readlane_u64(u, 16));
  r += __builtin_bit_cast(double, readlane_u64(u, 32));
  r += __builtin_bit_cast(double, readlane_u64(u, 48));
  return r;
}

// One block per (token, 8 experts): the 256 threads split H in 4-wide pieces,
// each keeps 8 fp64 partial sums; waves sum in a fixed order, then the block
// adds the four wave sums in wave order. All of a thread's loads are issued
// before its products (unrolled by 4 pieces), so a block waits for memory
// about once.
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
#pragma unroll 4
    for (int h = tid * 4; h < H; h += 256 * 4) {
      const u16x4 xv = *reinterpret_cast<const u16x4*>(xr + h);
      f32x4 w[SE];
#pragma unroll
      for (int j = 0; j < SE; ++j)
        w[j] = j < ne ? *reinterpret_cast<const f32x4*>(wr + (size_t)j * H + h)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double xc = bf16_bits_to_f32(xv[c]);
#pragma unroll
        for (int j = 0; j < SE; ++j) acc[j] = fma(xc, (double)w[j][c], acc[j]);
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
    const double v = wave_sum_f64(acc[j]);
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

namespace {
// K slices for the many-token kernels (block tiles of mt tokens): about 1024
// blocks, each slice at least 256 wide and a multiple of the 32-wide chunk.
int router_slices(int T, int H, int E, int mt, int* kslice) {
  const long tiles = (long)((T + mt - 1) / mt) * ((E + MN - 1) / MN);
  long want = (1024 + tiles - 1) / tiles;
  const long most = (H + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int ks = (int)((H + want - 1) / want);
  ks = (ks + MK - 1) / MK * MK;
  *kslice = ks;
  return (H + ks - 1) / ks;
}
}  // namespace

size_t router_workspace_bytes(int T, int H, int E) {
  if (T <= kRowsMaxTokens) return 0;
  int ks = 0;
  const int z = std::max(router_slices(T, H, E, MT, &ks), router_slices(T, H, E, FT, &ks));
  return (size_t)z * T * E * sizeof(double);
}

hipError_t launch_router_logits(const uint16_t* x, const float* wg, const float* bias, int T, int H,
                                int E, float* logits, void* ws, hipStream_t stream) {
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
  double* part = static_cast<double*>(ws);
  const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15u) == 0 &&
                       (reinterpret_cast<uintptr_t>(wg) & 15u) == 0;
  const bool full = aligned && H % MK == 0;
  int ks = 0;
  const int z = router_slices(T, H, E, full ? FT : MT, &ks);
  dim3 grid((T + (full ? FT : MT) - 1) / (full ? FT : MT), (E + MN - 1) / MN, z);
  if (full)
    hipLaunchKernelGGL(router_mfma_full_kernel, grid, dim3(256), 0, stream, x, wg, T, H, E, ks,
                       part);
  else if (aligned && H % 8 == 0)
    hipLaunchKernelGGL(router_mfma_kernel<true>, grid, dim3(256), 0, stream, x, wg, T, H, E, ks,
                       part);
  else
    hipLaunchKernelGGL(router_mfma_kernel<false>, grid, dim3(256), 0, stream, x, wg, T, H, E, ks,
                       part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t n = (size_t)T * E;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  if (bias)
    hipLaunchKernelGGL(router_reduce_kernel<true>, dim3(blocks), dim3(256), 0, stream, part, bias,
                       T, E, z, logits);
  else
    hipLaunchKernelGGL(router_reduce_kernel<false>, dim3(blocks), dim3(256), 0, stream, part, bias,
                       T, E, z, logits);
  return hipGetLastError();
}

}  // namespace moe
