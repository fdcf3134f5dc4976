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
// T <= 64: one block does all of it in LDS. Larger T: three kernels through
// the workspace: tile masks; a scan over the tiles of each expert (a thread per
// expert), whose last block to finish scans the local experts' counts into
// offsets; scatter.
#include "device.h"

namespace moe {

namespace {
constexpr int TILE = 64;

// One block of up to 1024 threads, T <= 64.
// Dynamic LDS: E uint64 masks + (L + 1) ints + 16 ints of scan scratch.
__global__ __launch_bounds__(1024) void permute_small_kernel(const int* __restrict__ ids, int T,
                                                             int k, int E, int first, int L,
                                                             int* __restrict__ counts,
                                                             int* __restrict__ offsets,
                                                             int* __restrict__ perm,
                                                             int* __restrict__ e2p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  int* off = reinterpret_cast<int*>(mask + E);
  int* tmp = off + (L + 1);
  const int tid = threadIdx.x, nt = blockDim.x;
  const int n = T * k;
  for (int e = tid; e < E; e += nt) mask[e] = 0ull;
  __syncthreads();
  for (int r = tid; r < n; r += nt) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (r / k));
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) counts[e] = __popcll(mask[e]);
  for (int i = tid; i < L; i += nt) off[i] = __popcll(mask[first + i]);
  __syncthreads();
  block_exclusive_scan(off, L, tmp);
  for (int i = tid; i <= L; i += nt) offsets[i] = off[i];
  for (int r = tid; r < n; r += nt) {
    const int e = ids[r];
    int p = -1;
    if (e >= first && e < first + L) {
      const int t = r / k;
      p = off[e - first] + __popcll(mask[e] & ((1ull << t) - 1ull));
      perm[p] = r;
    }
    e2p[r] = p;
  }
}

// Grid: one block per 64-token tile. masks[tile * E + e].
__global__ __launch_bounds__(256) void tile_masks_kernel(const int* __restrict__ ids, int T, int k,
                                                         int E,
                                                         unsigned long long* __restrict__ masks,
                                                         int* __restrict__ done) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0 && tid == 0) *done = 0;  // the scan kernel's arrival counter
  for (int e = tid; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  const int t0 = b * TILE;
  const int n = min(TILE, T - t0) * k;
  const int* tid_ids = ids + (size_t)t0 * k;
  for (int q = tid; q < n; q += blockDim.x) {
    const int e = tid_ids[q];
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (q / k));
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) masks[(size_t)b * E + e] = mask[e];
}

// Grid: ceil(E / 64) blocks of SW waves; lane j of every wave owns expert
// 64 * block + j and wave w the w-th of SW equal parts of the tiles:
// counts[e], and base[tile * L + i] = entries of local expert i in earlier
// tiles. The last block to finish writes offsets, the exclusive scan of the
// local experts' counts. Dynamic LDS: (L + 1) + 16 ints.
constexpr int SW = 16;
__global__ __launch_bounds__(SW * 64) void expert_scan_kernel(const unsigned long long* __restrict__ masks,
                                                              int nb, int E, int first, int L,
                                                              int* counts, int* __restrict__ offsets,
                                                              int* __restrict__ base, int* done) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int part[SW][kWave];
  __shared__ int is_last;
  int* off = reinterpret_cast<int*>(smem);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int e = blockIdx.x * kWave + lane;
  const int per = (nb + SW - 1) / SW;
  const int b0 = min(nb, wave * per), b1 = min(nb, b0 + per);
  int c = 0;
  if (e < E) {
#pragma unroll 4
    for (int b = b0; b < b1; ++b) c += __popcll(masks[(size_t)b * E + e]);
  }
  part[wave][lane] = c;
  __syncthreads();
  int run = 0;  // entries of expert e in tiles before b0
  for (int w = 0; w < wave; ++w) run += part[w][lane];
  const int i = e - first;
  if (e < E && i >= 0 && i < L) {
#pragma unroll 4
    for (int b = b0; b < b1; ++b) {
      base[(size_t)b * L + i] = run;
      run += __popcll(masks[(size_t)b * E + e]);
    }
  }
  if (wave == 0 && e < E) {
    int tot = 0;
    for (int w = 0; w < SW; ++w) tot += part[w][lane];
    counts[e] = tot;
  }
  // Counts are published (release, once per block) before the block is
  // counted; only the last block acquires. Each device-scope fence writes
  // back or invalidates the XCD's L2, so the other blocks skip the acquire.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // this wave's stores have reached L2
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int last = atomicAdd(done, 1) == (int)gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  for (int j = tid; j < L; j += blockDim.x)
    off[j] = __hip_atomic_load(&counts[first + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  block_exclusive_scan(off, L, off + L + 1);
  for (int j = tid; j <= L; j += blockDim.x) offsets[j] = off[j];
}

__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ ids, int T, int k,
                                                      int E, int first, int L,
                                                      const unsigned long long* __restrict__ masks,
                                                      const int* __restrict__ offsets,
                                                      const int* __restrict__ base,
                                                      int* __restrict__ perm,
                                                      int* __restrict__ e2p) {
  const int b = blockIdx.x;
  const int t0 = b * TILE;
  const int n = min(TILE, T - t0) * k;
  const int r0 = t0 * k;
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    const int r = r0 + q;
    const int e = ids[r];
    int p = -1;
    if (e >= first && e < first + L) {
      const int tl = q / k;
      const unsigned long long m = masks[(size_t)b * E + e];
      p = offsets[e - first] + base[(size_t)b * L + (e - first)] +
          __popcll(m & ((1ull << tl) - 1ull));
      perm[p] = r;
    }
    e2p[r] = p;
  }
}
}  // namespace

// Workspace for T > 64: tile masks [nb, E] u64, bases [nb, L] int, and the
// scan kernel's arrival counter.
size_t permute_workspace_bytes(int T, int E, int L) {
  if (T <= TILE) return 0;
  const size_t nb = (T + TILE - 1) / TILE;
  size_t masks = nb * (size_t)E * 8;
  masks = (masks + 255) & ~(size_t)255;
  size_t base = nb * (size_t)(L > 0 ? L : 1) * 4;
  return masks + ((base + 255) & ~(size_t)255) + 256;
}

hipError_t launch_permute(const int* ids, int T, int k, int E, int first, int L, int* counts,
                          int* offsets, int* perm, int* e2p, void* ws, hipStream_t stream) {
  if (T <= TILE) {
    const int n = T * k;
    int threads = n < 1024 ? ((n + 63) / 64) * 64 : 1024;
    threads = threads < 256 ? 256 : threads;
    const size_t lds = (size_t)E * 8 + (size_t)(L + 1) * 4 + 16 * 4;
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(threads), lds, stream, ids, T, k, E,
                       first, L, counts, offsets, perm, e2p);
    return hipGetLastError();
  }
  const int nb = (T + TILE - 1) / TILE;
  unsigned long long* masks = static_cast<unsigned long long*>(ws);
  const size_t mbytes = ((size_t)nb * E * 8 + 255) & ~(size_t)255;
  const size_t bbytes = ((size_t)nb * (L > 0 ? L : 1) * 4 + 255) & ~(size_t)255;
  int* base = reinterpret_cast<int*>(static_cast<char*>(ws) + mbytes);
  int* done = reinterpret_cast<int*>(static_cast<char*>(ws) + mbytes + bbytes);
  hipLaunchKernelGGL(tile_masks_kernel, dim3(nb), dim3(256), (size_t)E * 8, stream, ids, T, k, E,
                     masks, done);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(expert_scan_kernel, dim3((E + kWave - 1) / kWave), dim3(SW * kWave),
                     (size_t)(L + 1 + 16) * 4, stream, masks, nb, E, first, L, counts, offsets,
                     base, done);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nb), dim3(256), 0, stream, ids, T, k, E, first, L, masks,
                     offsets, base, perm, e2p);
  return hipGetLastError();
}

}  // namespace moe
