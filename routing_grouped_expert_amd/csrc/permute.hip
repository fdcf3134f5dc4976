// Per-expert histogram, prefix scan and stable permutation of the expanded
// indices r = t * k + j, all integer work, no atomics on positions.
//
// Tokens are taken in tiles of 64. For every (tile, expert) a 64-bit mask
// records which tokens of the tile chose the expert (each token chooses an
// expert at most once). Then
//   count(e)       = sum over tiles of popcount(mask)
//   position(t, e) = offsets[e] + (entries of e in earlier tiles)
//                               + popcount(mask & bits below t)
// which is exactly the stable counting sort by expert: within an expert the
// entries keep ascending t, hence ascending r. Masks are built with LDS
// atomic OR (order-free, so the result is deterministic).
//
// While every tile's masks fit in LDS one block does all of it. Otherwise
// three kernels through the workspace: tile masks; a scan over the tiles of
// each expert (a thread per expert) giving the counts and each tile's base;
// scatter, whose blocks each scan the local experts' counts into offsets.
//
// Routing and permutation together (launch_route_permute: the layer's path)
// come in three variants; a cost model fitted to measurements picks one
// (routing_plan):
//   ONE_BLOCK   (T <= 64) one block selects every token's experts
//               (select.h) and permutes them in LDS: one launch;
//   TWO_KERNELS the routing kernel (a wave per token), then the single-block
//               permutation above: two launches;
//   TILED       the routing kernel also writes the tile masks (route.hip),
//               then the scan and the scatter: three launches, any T.
#include "plan.h"
#include "select.h"

namespace moe {

// Routing variants (the values of moe_routing_variant in moe.h).
constexpr int kRoutingOneBlock = 1, kRoutingTwoKernels = 2, kRoutingTiled = 3;

namespace {
constexpr int TILE = 64;

// One block of 1024 threads for all nb = ceil(T / 64) tiles, when the masks
// and each tile's base per expert fit in LDS (block_permute_fits): masks in
// LDS, then a thread per expert walks its tiles in order for the count and the
// bases, and the block scans the local counts into offsets (then, given a
// PlanOut, writes the grouped FFN's pass plan). Dynamic LDS: nb E uint64
// masks, nb E ints of bases, 2 ((L + 1) + 16) ints.
constexpr size_t kBlockLds = 65536;
bool block_permute_fits(int T, int E, int L) {
  const size_t nb = (T + TILE - 1) / TILE;
  return nb * E * 12 + 2 * (size_t)(L + 1 + 16) * 4 <= kBlockLds;
}

// Share `part` of `parts` of zeroing the FFN fixup counters (given a plan),
// by a block of nt threads.
__device__ inline void zero_plan_counters(const PlanOut& po, int part, int parts, int nt) {
  if (!po.plan) return;
  for (int i = part * nt + threadIdx.x; i < po.ncounters; i += parts * nt) po.counters[i] = 0;
}

// After the block's offsets scan: zero this block's share of the FFN fixup
// counters and (block 0) write the FFN pass plan. s_pass: L + 1 + 16 ints.
__device__ inline void maybe_write_plan(const int* off, int L, const PlanOut& po, int* s_pass,
                                        int nt) {
  zero_plan_counters(po, blockIdx.x, gridDim.x, nt);
  if (po.plan && blockIdx.x == 0) write_ffn_plan(off, L, po, s_pass, nt);
}

// The first kPermRegs entries of each thread are loaded into registers before
// the masks are cleared (their latency overlaps the clearing) and kept for the
// placement; entries beyond that (more than 1024 kPermRegs) are read again.
constexpr int kPermRegs = 4;
__global__ __launch_bounds__(1024) void permute_block_kernel(const int* __restrict__ ids, int T,
                                                             int k, int E, int first, int L,
                                                             int* __restrict__ counts,
                                                             int* __restrict__ offsets,
                                                             int* __restrict__ perm,
                                                             int* __restrict__ e2p, PlanOut po) {
  constexpr int nt = 1024;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nb = (T + TILE - 1) / TILE;
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);  // [nb][E]
  int* base = reinterpret_cast<int*>(mask + (size_t)nb * E);              // [nb][E]
  int* off = base + (size_t)nb * E;
  int* tmp = off + (L + 1);
  int* s_pass = tmp + 16;
  const int tid = threadIdx.x;
  const int n = T * k;
  int ex[kPermRegs];
#pragma unroll
  for (int j = 0; j < kPermRegs; ++j) {
    const int r = tid + j * nt;
    ex[j] = r < n ? ids[r] : -1;
  }
  for (int i = tid; i < nb * E; i += nt) mask[i] = 0ull;
  __syncthreads();
  auto mark = [&](int r, int e) {
    const int t = r / k;
    if (e >= 0 && e < E) atomicOr(&mask[(t / TILE) * E + e], 1ull << (t % TILE));
  };
#pragma unroll
  for (int j = 0; j < kPermRegs; ++j) mark(tid + j * nt, ex[j]);
  for (int r = tid + kPermRegs * nt; r < n; r += nt) mark(r, ids[r]);
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      base[b * E + e] = run;
      run += __popcll(mask[b * E + e]);
    }
    counts[e] = run;
    if (e >= first && e < first + L) off[e - first] = run;
  }
  __syncthreads();
  block_exclusive_scan(off, L, tmp, nt);
  for (int i = tid; i <= L; i += nt) offsets[i] = off[i];
  maybe_write_plan(off, L, po, s_pass, nt);
  auto place = [&](int r, int e) {
    int p = -1;
    if (e >= first && e < first + L) {
      const int t = r / k, b = t / TILE, tl = t % TILE;
      p = off[e - first] + base[b * E + e] + __popcll(mask[b * E + e] & ((1ull << tl) - 1ull));
      perm[p] = r;
    }
    e2p[r] = p;
  };
#pragma unroll
  for (int j = 0; j < kPermRegs; ++j)
    if (tid + j * nt < n) place(tid + j * nt, ex[j]);
  for (int r = tid + kPermRegs * nt; r < n; r += nt) place(r, ids[r]);
}

// Grid: one block per 64-token tile. masks[tile * E + e].
__global__ __launch_bounds__(256) void tile_masks_kernel(const int* __restrict__ ids, int T, int k,
                                                         int E,
                                                         unsigned long long* __restrict__ masks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int t0 = b * TILE;
  const int n = min(TILE, T - t0) * k;
  const int* tid_ids = ids + (size_t)t0 * k;
  for (int q = tid; q < n; q += 256) {
    const int e = tid_ids[q];
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (q / k));
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) masks[(size_t)b * E + e] = mask[e];
}

// Grid: ceil(E / 64) blocks of SW waves; lane j of every wave owns expert
// 64 * block + j and wave w the w-th of SW equal parts of the tiles:
// counts[e], and base[tile * L + i] = entries of local expert i in earlier
// tiles. A wave keeps the popcounts of up to SCAN_REG of its tiles in
// registers between the two passes (more tiles: their masks are read again).
constexpr int SW = 16;
constexpr int SCAN_REG = 8;
__global__ __launch_bounds__(SW * 64) void expert_scan_kernel(const unsigned long long* __restrict__ masks,
                                                              int nb, int E, int first, int L,
                                                              int* __restrict__ counts,
                                                              int* __restrict__ base) {
  __shared__ int part[SW][kWave];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int e = blockIdx.x * kWave + lane;
  const int per = (nb + SW - 1) / SW;
  const int b0 = min(nb, wave * per), b1 = min(nb, b0 + per);
  const bool inreg = per <= SCAN_REG;
  int pc[SCAN_REG];
  int c = 0;
  if (e < E) {
    if (inreg) {
#pragma unroll
      for (int j = 0; j < SCAN_REG; ++j) {
        pc[j] = b0 + j < b1 ? __popcll(masks[(size_t)(b0 + j) * E + e]) : 0;
        c += pc[j];
      }
    } else {
#pragma unroll 4
      for (int b = b0; b < b1; ++b) c += __popcll(masks[(size_t)b * E + e]);
    }
  }
  part[wave][lane] = c;
  __syncthreads();
  int run = 0;  // entries of expert e in tiles before b0 (independent reads)
#pragma unroll
  for (int w = 0; w < SW; ++w) {
    const int x = part[w][lane];
    run += w < wave ? x : 0;
  }
  const int i = e - first;
  if (e < E && i >= 0 && i < L) {
    if (inreg) {
#pragma unroll
      for (int j = 0; j < SCAN_REG; ++j) {
        if (b0 + j < b1) base[(size_t)(b0 + j) * L + i] = run;
        run += pc[j];
      }
    } else {
#pragma unroll 4
      for (int b = b0; b < b1; ++b) {
        base[(size_t)b * L + i] = run;
        run += __popcll(masks[(size_t)b * E + e]);
      }
    }
  }
  if (wave == 0 && e < E) {
    int tot = 0;
    for (int w = 0; w < SW; ++w) tot += part[w][lane];
    counts[e] = tot;
  }
}

// Grid: one block per 64-token tile, kScatterThreads threads. Every block
// scans the local experts' counts into offsets in LDS (block 0 also writes
// them out, and the FFN pass plan given a PlanOut), then places its tile's
// entries. The entries, their masks and their bases do not depend on the
// offsets, so they are loaded first and arrive while the block scans (the
// counts, which the scan needs first, are loaded before them). Dynamic LDS:
// 2 ((L + 1) + 16) ints.
constexpr int kScatterThreads = 256;
constexpr int kScatterRegs = TILE * 32 / kScatterThreads;      // entries per thread at k = 32
constexpr int kScatterCounts = 4096 / kScatterThreads;         // counts per thread at L = 4096
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(
    const int* __restrict__ ids, int T, int k, int E, int first, int L,
    const unsigned long long* __restrict__ masks, const int* __restrict__ counts,
    int* __restrict__ offsets, const int* __restrict__ base, int* __restrict__ perm,
    int* __restrict__ e2p, PlanOut po) {
  extern __shared__ int off[];
  const int b = blockIdx.x;
  const int t0 = b * TILE;
  const int n = min(TILE, T - t0) * k;
  const int r0 = t0 * k;
  int cnt[kScatterCounts], ex[kScatterRegs], bs[kScatterRegs];
  unsigned long long m[kScatterRegs];
#pragma unroll
  for (int j = 0; j < kScatterCounts; ++j) {
    const int i = threadIdx.x + j * kScatterThreads;
    cnt[j] = i < L ? counts[first + i] : 0;
  }
#pragma unroll
  for (int j = 0; j < kScatterRegs; ++j) {
    const int q = threadIdx.x + j * kScatterThreads;
    ex[j] = q < n ? ids[r0 + q] : -1;
  }
#pragma unroll
  for (int j = 0; j < kScatterRegs; ++j) {
    const bool local = ex[j] >= first && ex[j] < first + L;
    m[j] = local ? masks[(size_t)b * E + ex[j]] : 0ull;
    bs[j] = local ? base[(size_t)b * L + (ex[j] - first)] : 0;
  }
#pragma unroll
  for (int j = 0; j < kScatterCounts; ++j) {
    const int i = threadIdx.x + j * kScatterThreads;
    if (i < L) off[i] = cnt[j];
  }
  __syncthreads();
  block_exclusive_scan(off, L, off + L + 1, kScatterThreads);
  if (blockIdx.x == 0)
    for (int j = threadIdx.x; j <= L; j += kScatterThreads) offsets[j] = off[j];
  maybe_write_plan(off, L, po, off + L + 1 + 16, kScatterThreads);
#pragma unroll
  for (int j = 0; j < kScatterRegs; ++j) {
    const int q = threadIdx.x + j * kScatterThreads;
    if (q < n) {
      const int r = r0 + q, e = ex[j];
      int p = -1;
      if (e >= first && e < first + L) {
        const int tl = q / k;
        p = off[e - first] + bs[j] + __popcll(m[j] & ((1ull << tl) - 1ull));
        perm[p] = r;
      }
      e2p[r] = p;
    }
  }
}
}  // namespace

// Routing and permutation of T <= 64 tokens in one block of NW waves: wave w
// routes tokens w, w + NW, .. (each token's logits are loaded before the
// previous token is selected), records its selections in the LDS masks and
// the LDS copy of the ids, then the block counts, scans and scatters as
// permute_block_kernel does for one tile. Dynamic LDS: E uint64 masks,
// (L + 1) + 16 ints, T k ints of ids, (L + 1) + 16 ints of plan scratch.
template <int VPL, bool VEC, int NW>
__global__ __launch_bounds__(NW * kWave) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int first, int L,
    int* __restrict__ ids, float* __restrict__ weights, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ perm, int* __restrict__ e2p, PlanOut po) {
  constexpr bool THRESH = VPL >= 4;
  constexpr bool AHEAD = VPL <= 16;  // registers for the next token's logits
  __shared__ unsigned long long cand[THRESH ? NW : 1][THRESH ? kWave : 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  int* off = reinterpret_cast<int*>(mask + E);
  int* tmp = off + (L + 1);
  int* ids_s = tmp + 16;
  int* s_pass = ids_s + T * k;
  constexpr int nt = NW * kWave;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = T * k;
  for (int e = tid; e < E; e += nt) mask[e] = 0ull;
  __syncthreads();
  float v[VPL], vn[AHEAD ? VPL : 1];
  if (wave < T) sel::load_logits<VPL, VEC>(logits + (size_t)wave * E, lane, E, v);
  for (int t = wave; t < T; t += NW) {
    if constexpr (AHEAD) {
      if (t + NW < T) sel::load_logits<VPL, VEC>(logits + (size_t)(t + NW) * E, lane, E, vn);
    } else if (t != wave) {
      sel::load_logits<VPL, VEC>(logits + (size_t)t * E, lane, E, v);
    }
    const uint32_t e = sel::route_token<VPL, VEC, THRESH>(v, lane, E, k, &cand[THRESH ? wave : 0][0],
                                                         ids, weights, (size_t)t);
    if (lane < k) {
      ids_s[t * k + lane] = static_cast<int>(e);
      atomicOr(&mask[e], 1ull << t);
    }
    if constexpr (AHEAD) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) v[i] = vn[i];
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) counts[e] = __popcll(mask[e]);
  for (int i = tid; i < L; i += nt) off[i] = __popcll(mask[first + i]);
  __syncthreads();
  block_exclusive_scan(off, L, tmp, nt);
  for (int i = tid; i <= L; i += nt) offsets[i] = off[i];
  maybe_write_plan(off, L, po, s_pass, nt);
  for (int r = tid; r < n; r += nt) {
    const int e = ids_s[r];
    int p = -1;
    if (e >= first && e < first + L) {
      const int t = r / k;
      p = off[e - first] + __popcll(mask[e] & ((1ull << t) - 1ull));
      perm[p] = r;
    }
    e2p[r] = p;
  }
}

// Workspace of the tiled variant (every T, so that any variant can run in
// the same workspace): tile masks [nb, E] u64 and bases [nb, L] int.
size_t permute_workspace_bytes(int T, int E, int L) {
  if (T <= 0) return 0;
  const size_t nb = (T + TILE - 1) / TILE;
  size_t masks = nb * (size_t)E * 8;
  masks = (masks + 255) & ~(size_t)255;
  size_t base = nb * (size_t)(L > 0 ? L : 1) * 4;
  return masks + ((base + 255) & ~(size_t)255);
}

namespace {
struct PermWs {
  unsigned long long* masks;
  int* base;
};
PermWs perm_ws(void* ws, int T, int E) {
  const int nb = (T + TILE - 1) / TILE;
  const size_t mbytes = ((size_t)nb * E * 8 + 255) & ~(size_t)255;
  char* w = static_cast<char*>(ws);
  return PermWs{reinterpret_cast<unsigned long long*>(w), reinterpret_cast<int*>(w + mbytes)};
}

hipError_t launch_scan_scatter(const int* ids, int T, int k, int E, int first, int L, int* counts,
                               int* offsets, int* perm, int* e2p, const PermWs& w,
                               const PlanOut& po, hipStream_t stream) {
  const int nb = (T + TILE - 1) / TILE;
  if (L > kScatterThreads * kScatterCounts) return hipErrorInvalidValue;  // (E <= 4096)
  hipLaunchKernelGGL(expert_scan_kernel, dim3((E + kWave - 1) / kWave), dim3(SW * kWave), 0,
                     stream, w.masks, nb, E, first, L, counts, w.base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nb), dim3(kScatterThreads), 2 * (size_t)(L + 1 + 16) * 4, stream,
                     ids, T, k, E, first, L, w.masks, counts, offsets, w.base, perm, e2p, po);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_small_tier(const float* logits, int T, int E, int k, int first, int L, int* ids,
                             float* w, int* counts, int* offsets, int* perm, int* e2p,
                             const PlanOut& po, hipStream_t stream) {
  constexpr int NW = VPL <= 16 ? 16 : 8;  // 128 VGPRs at 16 waves, 256 at 8
  const size_t lds = (size_t)E * 8 + 2 * (size_t)(L + 1 + 16) * 4 + (size_t)T * k * 4;
  const bool vec = VPL >= 4 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
  if constexpr (VPL >= 4) {
    if (vec) {
      hipLaunchKernelGGL((route_permute_small_kernel<VPL, true, NW>), dim3(1), dim3(NW * kWave),
                         lds, stream, logits, T, E, k, first, L, ids, w, counts, offsets, perm,
                         e2p, po);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_permute_small_kernel<VPL, false, NW>), dim3(1), dim3(NW * kWave), lds,
                     stream, logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* w,
                        hipStream_t stream);
hipError_t launch_route_masks(const float* logits, int T, int E, int k, int* ids, float* w,
                              unsigned long long* masks, hipStream_t stream);

namespace {
hipError_t launch_permute_block(const int* ids, int T, int k, int E, int first, int L, int* counts,
                                int* offsets, int* perm, int* e2p, const PlanOut& po,
                                hipStream_t stream) {
  const size_t nb = (T + TILE - 1) / TILE;
  const size_t lds = nb * E * 12 + 2 * (size_t)(L + 1 + 16) * 4;
  hipLaunchKernelGGL(permute_block_kernel, dim3(1), dim3(1024), lds, stream, ids, T, k, E, first,
                     L, counts, offsets, perm, e2p, po);
  return hipGetLastError();
}
}  // namespace

// Measured cost of the routing variants (microseconds per call of
// selection + permutation, back-to-back calls replayed from a captured
// graph on MI355X; N(0, 1) logits, all experts local), by values-per-lane
// tier (E = 64, 128, .., 4096), token count (1, 4, 16, .., 4096) and variant
// (ONE_BLOCK, TWO_KERNELS, TILED); 0 where the variant does not apply to that
// cell. Two tables: k = 8 and k = 2 selections per token (below 4 values per
// lane the selection takes k rounds, so the one-block variant, which selects
// every token on one CU, costs much less at small k).
constexpr int kCostTiers = 7, kCostPoints = 7;
constexpr float kCost8[kCostTiers][kCostPoints][3] = {
    {{3.83f, 5.28f, 8.08f}, {3.95f, 5.35f, 8.13f}, {4.69f, 5.76f, 8.96f}, {11.89f, 5.96f, 9.75f}, {0.f, 7.15f, 10.17f}, {0.f, 12.61f, 10.68f}, {0.f, 35.09f, 12.04f}},  // VPL 1 (E = 64)
    {{3.95f, 5.36f, 8.55f}, {4.21f, 5.70f, 9.36f}, {5.20f, 6.10f, 10.16f}, {12.59f, 6.30f, 10.20f}, {0.f, 7.44f, 10.24f}, {0.f, 13.59f, 11.36f}, {0.f, 0.f, 12.49f}},  // VPL 2 (E = 128)
    {{3.90f, 5.13f, 8.23f}, {3.92f, 5.11f, 8.38f}, {4.51f, 5.77f, 9.08f}, {10.15f, 5.91f, 9.30f}, {0.f, 7.11f, 9.88f}, {0.f, 13.43f, 10.36f}, {0.f, 0.f, 11.82f}},  // VPL 4 (E = 256)
    {{3.92f, 5.27f, 8.65f}, {4.24f, 5.60f, 8.94f}, {5.23f, 6.08f, 10.23f}, {11.75f, 6.24f, 9.93f}, {0.f, 7.46f, 10.44f}, {0.f, 0.f, 11.45f}, {0.f, 0.f, 12.39f}},  // VPL 8 (E = 512)
    {{4.61f, 5.62f, 9.38f}, {5.29f, 6.25f, 10.12f}, {6.12f, 6.55f, 11.17f}, {14.30f, 7.00f, 11.11f}, {0.f, 8.39f, 11.89f}, {0.f, 0.f, 12.10f}, {0.f, 0.f, 13.58f}},  // VPL 16 (E = 1024)
    {{6.13f, 6.45f, 11.14f}, {6.57f, 6.88f, 11.95f}, {9.75f, 7.72f, 13.29f}, {26.32f, 7.96f, 13.13f}, {0.f, 0.f, 13.54f}, {0.f, 0.f, 13.83f}, {0.f, 0.f, 18.07f}},  // VPL 32 (E = 2048)
    {{10.54f, 0.f, 15.60f}, {13.48f, 0.f, 15.80f}, {24.27f, 0.f, 18.26f}, {56.28f, 0.f, 18.14f}, {0.f, 0.f, 17.97f}, {0.f, 0.f, 18.39f}, {0.f, 0.f, 28.93f}},  // VPL 64 (E = 4096)
};
constexpr float kCost2[kCostTiers][kCostPoints][3] = {
    {{2.76f, 4.12f, 6.66f}, {2.98f, 4.30f, 7.51f}, {3.18f, 4.60f, 7.48f}, {5.96f, 4.75f, 8.00f}, {0.f, 5.04f, 8.35f}, {0.f, 6.21f, 8.47f}, {0.f, 12.85f, 9.92f}},  // VPL 1 (E = 64)
    {{2.89f, 4.28f, 7.63f}, {3.11f, 4.47f, 7.41f}, {3.42f, 4.78f, 7.87f}, {6.35f, 4.74f, 7.88f}, {0.f, 5.16f, 8.29f}, {0.f, 6.48f, 8.64f}, {0.f, 0.f, 10.08f}},  // VPL 2 (E = 128)
    {{3.45f, 4.61f, 7.98f}, {3.66f, 4.79f, 8.01f}, {3.97f, 5.34f, 8.72f}, {8.32f, 5.23f, 9.01f}, {0.f, 5.67f, 9.39f}, {0.f, 7.12f, 9.58f}, {0.f, 0.f, 11.15f}},  // VPL 4 (E = 256)
    {{3.71f, 4.92f, 8.41f}, {3.90f, 5.05f, 8.66f}, {4.68f, 5.68f, 9.19f}, {9.65f, 5.91f, 9.03f}, {0.f, 6.11f, 9.85f}, {0.f, 0.f, 10.31f}, {0.f, 0.f, 11.60f}},  // VPL 8 (E = 512)
    {{4.51f, 5.41f, 9.15f}, {4.89f, 6.02f, 9.65f}, {5.36f, 6.18f, 10.33f}, {11.80f, 6.45f, 10.10f}, {0.f, 6.79f, 10.27f}, {0.f, 0.f, 10.84f}, {0.f, 0.f, 13.15f}},  // VPL 16 (E = 1024)
    {{5.92f, 6.18f, 10.77f}, {5.95f, 6.21f, 11.35f}, {8.63f, 7.01f, 12.51f}, {22.13f, 6.95f, 12.23f}, {0.f, 0.f, 12.16f}, {0.f, 0.f, 12.62f}, {0.f, 0.f, 16.45f}},  // VPL 32 (E = 2048)
    {{9.29f, 0.f, 14.85f}, {12.19f, 0.f, 15.18f}, {21.33f, 0.f, 17.11f}, {46.86f, 0.f, 16.75f}, {0.f, 0.f, 16.40f}, {0.f, 0.f, 17.09f}, {0.f, 0.f, 27.36f}},  // VPL 64 (E = 4096)
};

// Predicted microseconds of a variant from one table for T tokens and E
// experts: the measured costs of E's tier, linear in log2 T between the
// measured token counts; past the last measured point of the variant (it
// stops applying there, or T > 4096) the last segment's slope continues.
double routing_cost_table(const float (&cost)[kCostTiers][kCostPoints][3], int variant, int T,
                          int E) {
  int tier = 0;
  for (int vpl = 1; vpl * 64 < E && tier < kCostTiers - 1; vpl *= 2) ++tier;
  const int v = variant - kRoutingOneBlock;
  double lt = 0.0;
  for (int t = 1; t < T; t *= 2) lt += 1.0;  // ceil(log2 T)
  const double x = lt / 2.0;                 // the measured points are 2 doublings apart
  int last = -1;
  for (int p = 0; p < kCostPoints; ++p)
    if (cost[tier][p][v] > 0.f) last = p;
  if (last < 0) return 1e9;
  int lo = x >= last ? last - 1 : (int)x;
  if (lo < 0) return cost[tier][0][v];
  const double c0 = cost[tier][lo][v], c1 = cost[tier][lo + 1][v];
  return c0 + (c1 - c0) * (x - lo);
}

// Predicted microseconds for k selections per token: the k = 2 and k = 8
// tables, linear in log2 k between them (clamped outside).
double routing_cost(int variant, int T, int E, int k) {
  const double c2 = routing_cost_table(kCost2, variant, T, E);
  const double c8 = routing_cost_table(kCost8, variant, T, E);
  double lk = 0.0;
  for (int j = 1; j < k; j *= 2) lk += 1.0;  // ceil(log2 k)
  const double w = lk <= 1.0 ? 0.0 : lk >= 3.0 ? 1.0 : (lk - 1.0) / 2.0;
  return c2 + (c8 - c2) * w;
}

bool routing_variant_applies(int variant, int T, int E, int L) {
  switch (variant) {
    case kRoutingOneBlock: return T <= TILE;
    case kRoutingTwoKernels: return block_permute_fits(T, E, L);
    case kRoutingTiled: return true;
  }
  return false;
}

// Routing (selection, weights) followed by the permutation, for moe_forward
// and moe_route_permute, in the given variant (routing_variant_applies must
// hold). ws: permute_workspace_bytes(T, E, L). po.plan non-NULL: the
// permutation kernel also writes the grouped FFN's pass plan (moe_forward).
hipError_t launch_route_permute(int variant, const float* logits, int T, int E, int k, int first,
                                int L, int* ids, float* w, int* counts, int* offsets, int* perm,
                                int* e2p, void* ws, const PlanOut& po, hipStream_t stream) {
  if (variant == kRoutingOneBlock) {
    if (E <= 64) return launch_small_tier<1>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    if (E <= 128) return launch_small_tier<2>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    if (E <= 256) return launch_small_tier<4>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    if (E <= 512) return launch_small_tier<8>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    if (E <= 1024) return launch_small_tier<16>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    if (E <= 2048) return launch_small_tier<32>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
    return launch_small_tier<64>(logits, T, E, k, first, L, ids, w, counts, offsets, perm, e2p, po, stream);
  }
  if (variant == kRoutingTwoKernels) {
    hipError_t err = launch_route(logits, T, E, k, ids, w, stream);
    if (err != hipSuccess) return err;
    return launch_permute_block(ids, T, k, E, first, L, counts, offsets, perm, e2p, po, stream);
  }
  const PermWs pw = perm_ws(ws, T, E);
  hipError_t err = launch_route_masks(logits, T, E, k, ids, w, pw.masks, stream);
  if (err != hipSuccess) return err;
  return launch_scan_scatter(ids, T, k, E, first, L, counts, offsets, perm, e2p, pw, po, stream);
}

// The variant moe_route_permute runs: the one with the smallest predicted
// time among those that apply (routing_cost).
int routing_plan(int T, int E, int k, int L) {
  int best = kRoutingTiled;
  double best_us = routing_cost(kRoutingTiled, T, E, k);
  for (int v : {kRoutingOneBlock, kRoutingTwoKernels}) {
    if (!routing_variant_applies(v, T, E, L)) continue;
    const double us = routing_cost(v, T, E, k);
    if (us < best_us) {
      best_us = us;
      best = v;
    }
  }
  return best;
}

hipError_t launch_permute(const int* ids, int T, int k, int E, int first, int L, int* counts,
                          int* offsets, int* perm, int* e2p, void* ws, hipStream_t stream) {
  const PlanOut none{};
  if (block_permute_fits(T, E, L))
    return launch_permute_block(ids, T, k, E, first, L, counts, offsets, perm, e2p, none, stream);
  const int nb = (T + TILE - 1) / TILE;
  const PermWs pw = perm_ws(ws, T, E);
  hipLaunchKernelGGL(tile_masks_kernel, dim3(nb), dim3(256), (size_t)E * 8, stream, ids, T, k, E,
                     pw.masks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_scan_scatter(ids, T, k, E, first, L, counts, offsets, perm, e2p, pw, none, stream);
}

}  // namespace moe
