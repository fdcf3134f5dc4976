// Grouped expert FFN on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate):
// the entry points and the generic kernels. Shapes on the 16-byte fast path
// go to the persistent kernels of ffn_sk.hip (K-split for few entries per
// expert, staged for many); the generic kernels below take every other shape.
//
// Page "FlashInfer MoE optimisation: overlapping grouped activation staging
// on Ampere and Hopper" (flashinfer PR #7368):
//  - section 1 (Ampere): the routed activation rows of a group are gathered
//    with 128-bit copies into on-chip memory, a missing member loads as zeros,
//    and a scalar path covers unaligned inputs or other tile sizes. Here each
//    expert's rows x[permuted_rows[p] / k] are gathered with 16-byte loads into
//    an LDS tile; unused token slots are zero; a checked element-wise variant
//    runs when shapes or pointers miss the 16-byte / 128-element fast path.
//  - section 2 (Hopper): weights are the streamed operand and the gathered
//    activations are the small one; every writer's LDS stores are published
//    with a barrier before any wave reads them.
// The design for CDNA4: weight rows are the MFMA M dimension and stream
// straight from HBM into VGPRs in the A-operand layout (each weight byte is
// read once per pass over an expert's tokens); the expert's token rows are
// the N dimension, 16 per MFMA tile, staged in LDS per 128-wide K chunk.
//
// up kernel:   g = W1[e][0:I] x, u = W1[e][I:2I] x, a = silu(g) * u, written
//              as two bf16 arrays hi = bf16(a), lo = bf16(a - hi) whose sum
//              is a to about 2^-17 relative (a is never rounded to bf16 alone).
// down kernel: out = W2[e] (hi + lo) as two MFMAs into one fp32 accumulator.
#include "plan.h"

namespace moe {

namespace {
constexpr int KC = 128;  // K chunk staged in LDS
constexpr int PAD = 8;   // bf16 elements of padding per LDS row
constexpr int BLOCK_ROWS = 64;  // A rows per block: 4 waves x 16

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

__device__ __forceinline__ bf16x8 load8_checked(const uint16_t* row, int k0, int K, bool ok) {
  u16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (ok && k0 + j < K) ? row[k0 + j] : (uint16_t)0;
  return __builtin_bit_cast(bf16x8, v);
}

constexpr int STEPS = KC / 32;  // MFMA K-steps per chunk

// The A fragments of one K chunk for this lane: row `row`, columns
// k0 + 32 s + kq .. +8 for s < STEPS (the 16x16x32 A-operand layout). F8:
// the row holds FP8 E4M3 codes, 8 bytes per fragment, widened to bf16
// exactly (the row's scale is applied to the finished sums).
template <bool VEC, bool F8>
__device__ __forceinline__ void load_a(bf16x8 (&a)[STEPS], const void* row, int k0, int K,
                                       bool ok, int kq) {
  if constexpr (F8) {
    const uint8_t* r8 = static_cast<const uint8_t*>(row);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int c = k0 + s * 32 + kq;
      uint32_t lo = 0, hi = 0;
      if (VEC) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = *reinterpret_cast<const u32x2*>(r8 + c);
        lo = v[0];
        hi = v[1];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b = (ok && c + j < K) ? r8[c + j] : 0u;
          if (j < 4) lo |= b << (8 * j);
          else hi |= b << (8 * (j - 4));
        }
      }
      a[s] = e4m3x8_to_bf16(lo, hi);
    }
  } else {
    const uint16_t* r = static_cast<const uint16_t*>(row);
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
      a[s] = VEC ? load8(r + k0 + s * 32 + kq) : load8_checked(r, k0 + s * 32 + kq, K, ok);
  }
}

// Element `i` of a weight array of bf16 values (F8 false) or FP8 codes.
template <bool F8>
__device__ __forceinline__ const void* welem(const void* base, size_t i) {
  return F8 ? static_cast<const void*>(static_cast<const uint8_t*>(base) + i)
            : static_cast<const void*>(static_cast<const uint16_t*>(base) + i);
}

typedef uint16_t lds_row_t[KC + PAD];

// One K chunk of the up projection for NTILES 16-token tiles (a compile-time
// count, so accumulators and fragments stay in registers).
template <int NTILES>
__device__ __forceinline__ void up_chunk(const bf16x8 (&ag)[STEPS], const bf16x8 (&au)[STEPS],
                                         const lds_row_t* xs, int lane, int kq, f32x4* accg,
                                         f32x4* accu) {
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
#pragma unroll
    for (int nt = 0; nt < NTILES; ++nt) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&xs[nt * 16 + (lane & 15)][s * 32 + kq]);
      accg[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag[s], b, accg[nt], 0, 0, 0);
      accu[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au[s], b, accu[nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One K chunk of the down projection: W2 rows times (hi + lo) of the tiles.
template <int NTILES>
__device__ __forceinline__ void down_chunk(const bf16x8 (&a)[STEPS], const lds_row_t* xh,
                                           const lds_row_t* xl, int lane, int kq, f32x4* acc) {
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
#pragma unroll
    for (int nt = 0; nt < NTILES; ++nt) {
      const int n = nt * 16 + (lane & 15);
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&xh[n][s * 32 + kq]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&xl[n][s * 32 + kq]);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bh, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bl, acc[nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ void clamp_range(const int* offsets, int e, int nmax, int& beg,
                                            int& end) {
  beg = offsets[e];
  end = offsets[e + 1];
  beg = max(0, min(beg, nmax));
  end = max(beg, min(end, nmax));
}

template <int NT, bool VEC, bool F8>
__global__ __launch_bounds__(256) void ffn_up_kernel(const uint16_t* __restrict__ x,
                                                     const int* __restrict__ perm,
                                                     const int* __restrict__ offsets, int k, int H,
                                                     int I, int nmax,
                                                     const void* __restrict__ w1,
                                                     const float* __restrict__ s1,
                                                     uint16_t* __restrict__ h_hi,
                                                     uint16_t* __restrict__ h_lo) {
  constexpr int NR = NT * 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[NR][KC + PAD];
  __shared__ int s_tok[NR];
  const int e = blockIdx.y;
  int beg, end;
  clamp_range(offsets, e, nmax, beg, end);
  if (end <= beg) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int i0 = blockIdx.x * BLOCK_ROWS + wave * 16;
  const int arow = i0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  const bool arow_ok = arow < I;
  const void* wg = welem<F8>(w1, ((size_t)e * 2 * I + (arow_ok ? arow : 0)) * H);
  const void* wu = welem<F8>(wg, (size_t)I * H);

  for (int pb = beg; pb < end; pb += NR) {
    const int pc = min(NR, end - pb);
    const int ntiles = (pc + 15) / 16;
    __syncthreads();
    for (int n = threadIdx.x; n < NR; n += blockDim.x) {
      int tok = -1;
      if (n < pc) {
        const int r = perm[pb + n];
        if (r >= 0 && r < nmax) tok = r / k;
      }
      s_tok[n] = tok;
    }
    f32x4 accg[NT], accu[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      accg[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Weight fragments of one K chunk; the next chunk's are loaded while the
    // current one is multiplied, so HBM reads stay in flight across barriers.
    bf16x8 ag[STEPS], au[STEPS], ng[STEPS], nu[STEPS];
    load_a<VEC, F8>(ag, wg, 0, H, arow_ok, kq);
    load_a<VEC, F8>(au, wu, 0, H, arow_ok, kq);
    for (int k0 = 0; k0 < H; k0 += KC) {
      __syncthreads();
      if (VEC) {
        for (int q = threadIdx.x; q < ntiles * 16 * (KC / 8); q += blockDim.x) {
          const int n = q / (KC / 8), c = (q % (KC / 8)) * 8;
          const int tok = s_tok[n];
          u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
          if (tok >= 0) v = *reinterpret_cast<const u16x8*>(x + (size_t)tok * H + k0 + c);
          *reinterpret_cast<u16x8*>(&xs[n][c]) = v;
        }
      } else {
        for (int q = threadIdx.x; q < ntiles * 16 * KC; q += blockDim.x) {
          const int n = q / KC, c = q % KC;
          const int tok = s_tok[n];
          xs[n][c] = (tok >= 0 && k0 + c < H) ? x[(size_t)tok * H + k0 + c] : (uint16_t)0;
        }
      }
      __syncthreads();
      if (k0 + KC < H) {
        load_a<VEC, F8>(ng, wg, k0 + KC, H, arow_ok, kq);
        load_a<VEC, F8>(nu, wu, k0 + KC, H, arow_ok, kq);
      }
      switch (ntiles) {
#define MOE_UP_CASE(n) \
  case n:              \
    if (n <= NT) up_chunk<n>(ag, au, xs, lane, kq, accg, accu); \
    break;
        MOE_UP_CASE(1) MOE_UP_CASE(2) MOE_UP_CASE(3) MOE_UP_CASE(4)
        MOE_UP_CASE(5) MOE_UP_CASE(6) MOE_UP_CASE(7) MOE_UP_CASE(8)
#undef MOE_UP_CASE
      }
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        ag[s] = ng[s];
        au[s] = nu[s];
      }
    }
    // Lane l holds rows i0 + 4*(l/16) + j (j < 4) of token slot l % 16.
    const int ir = i0 + (lane >> 4) * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + (lane & 15);
      if (nt >= ntiles || n >= pc) continue;
      const size_t p = (size_t)(pb + n);
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float g = accg[nt][j], u = accu[nt][j];
        if (F8) {
          const int row = ir + j < I ? ir + j : 0;
          g *= s1[(size_t)e * 2 * I + row];
          u *= s1[(size_t)e * 2 * I + I + row];
        }
        const float a = g / (1.0f + expf(-g)) * u;
        hi[j] = f32_to_bf16_bits(a);
        lo[j] = f32_to_bf16_bits(a - bf16_bits_to_f32(hi[j]));
      }
      if (VEC) {
        typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<u16x4*>(h_hi + p * I + ir) = u16x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u16x4*>(h_lo + p * I + ir) = u16x4{lo[0], lo[1], lo[2], lo[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ir + j < I) {
            h_hi[p * I + ir + j] = hi[j];
            h_lo[p * I + ir + j] = lo[j];
          }
        }
      }
    }
  }
}

template <int NT, bool VEC, bool F8>
__global__ __launch_bounds__(256) void ffn_down_kernel(const uint16_t* __restrict__ h_hi,
                                                       const uint16_t* __restrict__ h_lo,
                                                       const int* __restrict__ offsets, int H,
                                                       int I, int nmax,
                                                       const void* __restrict__ w2,
                                                       const float* __restrict__ s2,
                                                       float* __restrict__ out) {
  constexpr int NR = NT * 16;
  __shared__ __attribute__((aligned(16))) uint16_t xh[NR][KC + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t xl[NR][KC + PAD];
  const int e = blockIdx.y;
  int beg, end;
  clamp_range(offsets, e, nmax, beg, end);
  if (end <= beg) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c0 = blockIdx.x * BLOCK_ROWS + wave * 16;
  const int arow = c0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  const bool arow_ok = arow < H;
  const void* w = welem<F8>(w2, ((size_t)e * H + (arow_ok ? arow : 0)) * I);

  for (int pb = beg; pb < end; pb += NR) {
    const int pc = min(NR, end - pb);
    const int ntiles = (pc + 15) / 16;
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a[STEPS], na[STEPS];
    load_a<VEC, F8>(a, w, 0, I, arow_ok, kq);
    for (int k0 = 0; k0 < I; k0 += KC) {
      __syncthreads();
      if (VEC) {
        for (int q = threadIdx.x; q < ntiles * 16 * (KC / 8); q += blockDim.x) {
          const int n = q / (KC / 8), c = (q % (KC / 8)) * 8;
          u16x8 vh = {0, 0, 0, 0, 0, 0, 0, 0}, vl = vh;
          if (n < pc) {
            const size_t off = (size_t)(pb + n) * I + k0 + c;
            vh = *reinterpret_cast<const u16x8*>(h_hi + off);
            vl = *reinterpret_cast<const u16x8*>(h_lo + off);
          }
          *reinterpret_cast<u16x8*>(&xh[n][c]) = vh;
          *reinterpret_cast<u16x8*>(&xl[n][c]) = vl;
        }
      } else {
        for (int q = threadIdx.x; q < ntiles * 16 * KC; q += blockDim.x) {
          const int n = q / KC, c = q % KC;
          const bool ok = n < pc && k0 + c < I;
          const size_t off = (size_t)(pb + n) * I + k0 + c;
          xh[n][c] = ok ? h_hi[off] : (uint16_t)0;
          xl[n][c] = ok ? h_lo[off] : (uint16_t)0;
        }
      }
      __syncthreads();
      if (k0 + KC < I) load_a<VEC, F8>(na, w, k0 + KC, I, arow_ok, kq);
      switch (ntiles) {
#define MOE_DOWN_CASE(n) \
  case n:                \
    if (n <= NT) down_chunk<n>(a, xh, xl, lane, kq, acc); \
    break;
        MOE_DOWN_CASE(1) MOE_DOWN_CASE(2) MOE_DOWN_CASE(3) MOE_DOWN_CASE(4)
        MOE_DOWN_CASE(5) MOE_DOWN_CASE(6) MOE_DOWN_CASE(7) MOE_DOWN_CASE(8)
#undef MOE_DOWN_CASE
      }
#pragma unroll
      for (int s = 0; s < STEPS; ++s) a[s] = na[s];
    }
    const int cr = c0 + (lane >> 4) * 4;
    if (F8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = s2[(size_t)e * H + (cr + j < H ? cr + j : 0)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][j] *= sc;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + (lane & 15);
      if (nt >= ntiles || n >= pc) continue;
      float* o = out + (size_t)(pb + n) * H + cr;
      if (VEC) {
        *reinterpret_cast<f32x4*>(o) = acc[nt];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (cr + j < H) o[j] = acc[nt][j];
      }
    }
  }
}

template <int NT, bool F8>
hipError_t launch_nt(const uint16_t* x, const int* perm, const int* offsets, int L, int k, int H,
                     int I, int nmax, const void* w1, const float* s1, const void* w2,
                     const float* s2, uint16_t* h_hi, uint16_t* h_lo, float* out, bool vec,
                     hipStream_t stream) {
  dim3 g1((I + BLOCK_ROWS - 1) / BLOCK_ROWS, L), g2((H + BLOCK_ROWS - 1) / BLOCK_ROWS, L);
  if (vec) {
    hipLaunchKernelGGL((ffn_up_kernel<NT, true, F8>), g1, dim3(256), 0, stream, x, perm, offsets,
                       k, H, I, nmax, w1, s1, h_hi, h_lo);
  } else {
    hipLaunchKernelGGL((ffn_up_kernel<NT, false, F8>), g1, dim3(256), 0, stream, x, perm, offsets,
                       k, H, I, nmax, w1, s1, h_hi, h_lo);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (vec) {
    hipLaunchKernelGGL((ffn_down_kernel<NT, true, F8>), g2, dim3(256), 0, stream, h_hi, h_lo,
                       offsets, H, I, nmax, w2, s2, out);
  } else {
    hipLaunchKernelGGL((ffn_down_kernel<NT, false, F8>), g2, dim3(256), 0, stream, h_hi, h_lo,
                       offsets, H, I, nmax, w2, s2, out);
  }
  return hipGetLastError();
}

template <bool F8>
hipError_t launch_generic(const uint16_t* x, const int* perm, const int* offsets, int L, int T,
                          int k, int H, int I, const void* w1, const float* s1, const void* w2,
                          const float* s2, uint16_t* h_hi, uint16_t* h_lo, float* out, bool vec,
                          hipStream_t stream) {
  const int nmax = T * k;
  // A token picks an expert at most once, so an expert has at most T entries.
  const int bound = T < nmax ? T : nmax;
  if (bound <= 16)
    return launch_nt<1, F8>(x, perm, offsets, L, k, H, I, nmax, w1, s1, w2, s2, h_hi, h_lo, out, vec, stream);
  if (bound <= 32)
    return launch_nt<2, F8>(x, perm, offsets, L, k, H, I, nmax, w1, s1, w2, s2, h_hi, h_lo, out, vec, stream);
  if (bound <= 64)
    return launch_nt<4, F8>(x, perm, offsets, L, k, H, I, nmax, w1, s1, w2, s2, h_hi, h_lo, out, vec, stream);
  return launch_nt<8, F8>(x, perm, offsets, L, k, H, I, nmax, w1, s1, w2, s2, h_hi, h_lo, out, vec, stream);
}
}  // namespace

bool ffn_sk_applies(const void* x, const void* w1, const void* w2, const void* out, int T, int k,
                    int L, int H, int I);
size_t ffn_sk_workspace_bytes(int T, int k, int L);
bool ffn_sk_fp8_applies(const void* x, const void* w1q, const void* w2q, const void* out, int T,
                        int k, int L, int H, int I);
hipError_t launch_grouped_ffn_sk_fp8(const uint16_t* x, const int* perm, const int* offsets,
                                     int L, int T, int k, int H, int I, const uint8_t* w1q,
                                     const float* w1s, const uint8_t* w2q, const float* w2s,
                                     uint16_t* h_hi, uint16_t* h_lo, float* out, void* ws,
                                     bool plan_ready, hipStream_t stream);
hipError_t launch_grouped_ffn_sk(const uint16_t* x, const int* perm, const int* offsets, int L,
                                 int T, int k, int H, int I, const uint16_t* w1,
                                 const uint16_t* w2, uint16_t* h_hi, uint16_t* h_lo, float* out,
                                 void* ws, bool plan_ready, hipStream_t stream);
PlanOut ffn_sk_plan_out(int T, int k, int L, int H, int I, bool f8, void* ws);

namespace {
size_t h_array_bytes(int T, int k, int I) {
  const size_t n = (size_t)T * k * I * 2;  // one bf16 array
  return (n + 255) & ~(size_t)255;
}
}  // namespace

// Workspace: h_hi, h_lo ([T*k, I] bf16 each), then the stream-K plan / slots.
size_t ffn_workspace_bytes(int T, int k, int I, int L) {
  return 2 * h_array_bytes(T, k, I) + ffn_sk_workspace_bytes(T, k, L);
}

bool ffn_vector_path(const void* x, const void* w1, const void* w2, const void* ws,
                     const void* out, int H, int I) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return al(x) && al(w1) && al(w2) && al(ws) && al(out) && H % KC == 0 && I % KC == 0 &&
         H % BLOCK_ROWS == 0 && I % BLOCK_ROWS == 0;
}

// Whether the persistent kernels run for these arguments and, if so, where
// their pass plan goes (*po) in the FFN workspace ws: a caller that computes
// the expert offsets can write the plan itself and pass plan_ready.
bool ffn_plan_target(const void* x, const void* w1, const void* w2, const void* out, int T, int k,
                     int L, int H, int I, bool f8, void* ws, PlanOut* po) {
  const bool sk = f8 ? ffn_sk_fp8_applies(x, w1, w2, out, T, k, L, H, I)
                     : ffn_sk_applies(x, w1, w2, out, T, k, L, H, I);
  if (!sk || L < 1) return false;
  *po = ffn_sk_plan_out(T, k, L, H, I, f8, static_cast<char*>(ws) + 2 * h_array_bytes(T, k, I));
  return true;
}

hipError_t launch_grouped_ffn(const uint16_t* x, const int* perm, const int* offsets, int L, int T,
                              int k, int H, int I, const uint16_t* w1, const uint16_t* w2,
                              float* out, void* ws, bool plan_ready, hipStream_t stream) {
  const size_t half = h_array_bytes(T, k, I);
  uint16_t* h_hi = static_cast<uint16_t*>(ws);
  uint16_t* h_lo = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + half);
  if (ffn_sk_applies(x, w1, w2, out, T, k, L, H, I))
    return launch_grouped_ffn_sk(x, perm, offsets, L, T, k, H, I, w1, w2, h_hi, h_lo, out,
                                 static_cast<char*>(ws) + 2 * half, plan_ready, stream);
  return launch_generic<false>(x, perm, offsets, L, T, k, H, I, w1, nullptr, w2, nullptr, h_hi,
                               h_lo, out, ffn_vector_path(x, w1, w2, ws, out, H, I), stream);
}

// FP8 E4M3 weights with per-row fp32 scales (w1s [L, 2I], w2s [L, H]).
hipError_t launch_grouped_ffn_fp8(const uint16_t* x, const int* perm, const int* offsets, int L,
                                  int T, int k, int H, int I, const uint8_t* w1q,
                                  const float* w1s, const uint8_t* w2q, const float* w2s,
                                  float* out, void* ws, bool plan_ready, hipStream_t stream) {
  const size_t half = h_array_bytes(T, k, I);
  uint16_t* h_hi = static_cast<uint16_t*>(ws);
  uint16_t* h_lo = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + half);
  if (ffn_sk_fp8_applies(x, w1q, w2q, out, T, k, L, H, I))
    return launch_grouped_ffn_sk_fp8(x, perm, offsets, L, T, k, H, I, w1q, w1s, w2q, w2s, h_hi,
                                     h_lo, out, static_cast<char*>(ws) + 2 * half, plan_ready,
                                     stream);
  return launch_generic<true>(x, perm, offsets, L, T, k, H, I, w1q, w1s, w2q, w2s, h_hi, h_lo,
                              out, ffn_vector_path(x, w1q, w2q, ws, out, H, I), stream);
}

}  // namespace moe
