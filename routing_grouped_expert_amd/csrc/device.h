// Device-side helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even on the fp32 bit pattern; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// DPP move within rows of 16 lanes (CTRL: a gfx9 dpp_ctrl code, e.g. 0x121 +
// n - 1 for row_ror:n); every lane of a full wave has a source.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Maximum over a full wave, wave-uniform: rotations by 1, 2, 4, 8 within each
// row of 16 lanes leave every lane with its row's maximum, then the four rows
// are combined from one lane each.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0x121>(v); v = o > v ? o : v;
  o = dpp_u64<0x122>(v); v = o > v ? o : v;
  o = dpp_u64<0x124>(v); v = o > v ? o : v;
  o = dpp_u64<0x128>(v); v = o > v ? o : v;
  uint64_t r = readlane_u64(v, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const uint64_t x = readlane_u64(v, 16 * row);
    r = x > r ? x : r;
  }
  return r;
}

// Workgroups are dispatched to the 8 XCDs round-robin (block b to XCD b % 8),
// and each XCD has its own L2. Renumber blocks so that consecutive work
// ranges -- the same experts, hence the same activation rows -- run on the
// same XCD: physical block b becomes (b % 8) * (NB / 8) + b / 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int b, int NB) {
  return NB % kXcds == 0 ? (b % kXcds) * (NB / kXcds) + b / kXcds : b;
}

// Eight FP8 E4M3 (OCP e4m3fn) weight codes, lo = codes 0..3 and hi = codes
// 4..7 in byte order, as eight bf16 values. Every E4M3 value is a bf16 value,
// so the conversion is exact; CDNA4's scaled decoder turns two codes into two
// bf16 in one instruction (scale 1: the plain value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  const u32x4_ r = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
  return __builtin_bit_cast(bf16x8, r);
#else
  (void)lo;
  (void)hi;
  return bf16x8{};
#endif
}

// Maximum / minimum of 32-bit unsigned values over a full wave, wave-uniform
// (row rotations as above; the compiler folds each move into the max / min).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x121>(v));
  v = max(v, dpp_u32<0x122>(v));
  v = max(v, dpp_u32<0x124>(v));
  v = max(v, dpp_u32<0x128>(v));
  const uint32_t a = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t b = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t c = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t d = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0x121>(v));
  v = min(v, dpp_u32<0x122>(v));
  v = min(v, dpp_u32<0x124>(v));
  v = min(v, dpp_u32<0x128>(v));
  const uint32_t a = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t b = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t c = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t d = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return min(min(a, b), min(c, d));
}

// Butterfly sum: every lane ends with the same value, summed in the same
// fixed order on every run.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes (lane i ends with the sum of lanes
// 0..i) by DPP: inside each row of 16 lanes, shifts by 1, 2, 4 and 8 (a lane
// with no source lane adds 0); then the last lane of row 0 is added to row 1
// and that of row 2 to row 3 (row broadcast of lane 15), and the last lane of
// row 1 (rows 0-1 in all) to rows 2 and 3 (row broadcast of lane 31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return v;
}

// Exclusive prefix sum over data[0, n) in shared memory by one block of nt
// threads (nt = blockDim.x, a multiple of 64, at most 1024; callers that know
// it at compile time pass it, which spares a load of the launch's block size);
// data[n] receives the total. `tmp` is shared scratch of at least nt / 64
// ints. Must be called by every thread of the block.
__device__ inline void block_exclusive_scan(int* data, int n, int* tmp, int nt) {
  const int tid = threadIdx.x;
  const int per = (n + nt - 1) / nt;
  const int b = tid * per, e = min(b + per, n);
  int local = 0;
  for (int i = b; i < e; ++i) local += data[i];
  // inclusive scan of `local` across the block
  const int lane = tid % kWave, wave = tid / kWave;
  const int v = wave_inclusive_sum(local);
  if (lane == kWave - 1) tmp[wave] = v;
  __syncthreads();
  if (wave == 0) {
    const int w = wave_inclusive_sum(lane < nt / kWave ? tmp[lane] : 0);
    if (lane < nt / kWave) tmp[lane] = w;
  }
  __syncthreads();
  int run = v - local + (wave > 0 ? tmp[wave - 1] : 0);
  const int total = tmp[nt / kWave - 1];
  __syncthreads();
  for (int i = b; i < e; ++i) {
    int c = data[i];
    data[i] = run;
    run += c;
  }
  if (tid == 0) data[n] = total;
  __syncthreads();
}

}  // namespace moe
