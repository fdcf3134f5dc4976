// HBM read probe (measurement only, not part of the MoE path): streams a
// device buffer once with 16-byte loads, every wave reading 8 consecutive
// 1 KB pieces per round, so the achievable read bandwidth of the part can be
// reported beside the 8 TB/s peak. Built as its own library, libhbmprobe.so.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t wave = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const size_t nwaves = (size_t)gridDim.x * blockDim.x / 64;
  const int lane = threadIdx.x % 64;
  uint32_t acc = 0;
  // round r of a wave covers pieces [(r * nwaves + wave) * 8, +8) of 64 vectors
  for (size_t base = wave * kUnroll * 64; base < n16; base += nwaves * kUnroll * 64) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * 64 + lane;
      v[u] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never taken
}
}  // namespace

// Reads bytes (a multiple of 16) from the 16-byte aligned device buffer buf
// on stream; sink is a device word the kernel may write. Returns a hipError_t.
extern "C" int hbm_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
  if (!buf || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return hipErrorInvalidValue;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  hipLaunchKernelGGL(read_probe_kernel, dim3(cus * 4), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}
