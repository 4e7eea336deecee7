// A plain streaming read, for the measured read rate that the kernels' bandwidth figures
// are compared with (beside the spec peak).  Not a step of the decode path.
#include "hk_internal.h"

namespace hk {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;              // 16-byte loads in flight per thread
constexpr int64_t kProbeChunk = (int64_t)kProbeThreads * kProbeUnroll;   // vectors per workgroup

// One pass: workgroup b reads the 32 KB of vectors [b*kProbeChunk, (b+1)*kProbeChunk),
// every load issued before any is used (the access pattern of the Hamming scan), and
// writes the XOR of what it read to sink[b] so the loads are kept.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src,
                                                                   int64_t n,
                                                                   uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kProbeChunk + threadIdx.x;
  u32x4 v[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kProbeThreads;
    v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int64_t read_probe_blocks(size_t bytes) {
  const int64_t n = (int64_t)(bytes / 16);
  return (n + kProbeChunk - 1) / kProbeChunk;
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t st) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)read_probe_blocks(bytes)),
                     dim3(kProbeThreads), 0, st, static_cast<const u32x4 *>(src), n, sink);
  return hipGetLastError();
}

}  // namespace hk
