// A plain streaming read and a plain random-row gather, for the measured rates that the
// kernels' bandwidth figures are compared with (beside the spec peak).  Not steps of the
// decode path: this translation unit is the library libhk_probe.so of its own, with the C
// entry points of hk_probe.h.
#include "hk_internal.h"
#include "hk_probe.h"

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

// Random-row gather in the access pattern of the attention core: workgroup b takes rows
// [b*rpb, (b+1)*rpb) of the index list, stages their token indices in LDS with one
// coalesced read, and each wavefront then requests two 16-row tiles at a time, the
// 256-byte K row and V row of every token (16 lanes of 16-byte loads per row).  Tokens
// outside [0, table_rows) read row 0.  sink[b] = XOR of every word read.
constexpr int kGatherMaxRows = 4096;         // rows per workgroup (LDS index slice)
constexpr int kGatherTiles = 2;              // 16-row tiles in flight per wavefront

__global__ __launch_bounds__(kProbeThreads) void gather_probe_kernel(
    const u32x4 *__restrict__ kt, const u32x4 *__restrict__ vt, int64_t table_rows,
    const int32_t *__restrict__ idx, int64_t n, int rpb, uint32_t *__restrict__ sink) {
  __shared__ int32_t s_idx[kGatherMaxRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * rpb;
  const int len = (int)(n - r0 < rpb ? n - r0 : rpb);
  for (int r = threadIdx.x; r < len; r += kProbeThreads) {
    const int32_t tok = idx[r0 + r];
    s_idx[r] = (tok >= 0 && tok < table_rows) ? tok : 0;
  }
  __syncthreads();
  uint32_t acc = 0;
  for (int t0 = wave * 16 * kGatherTiles; t0 < len; t0 += 4 * 16 * kGatherTiles) {
    u32x4 kx[kGatherTiles][4], vx[kGatherTiles][4];
#pragma unroll
    for (int u = 0; u < kGatherTiles; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = t0 + 16 * u + 4 * grp + j;
        if (r < len) {
          const int64_t e = (int64_t)s_idx[r] * 16 + col;
          kx[u][j] = kt[e];
          vx[u][j] = vt[e];
        } else {
          kx[u][j] = u32x4{0u, 0u, 0u, 0u};
          vx[u][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
    for (int u = 0; u < kGatherTiles; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc ^= kx[u][j].x ^ kx[u][j].y ^ kx[u][j].z ^ kx[u][j].w ^ vx[u][j].x ^ vx[u][j].y ^
               vx[u][j].z ^ vx[u][j].w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int64_t gather_probe_blocks(int64_t n_idx, int rows_per_block) {
  return rows_per_block > 0 ? (n_idx + rows_per_block - 1) / rows_per_block : 0;
}

bool gather_probe_rows_ok(int rows_per_block) {
  return rows_per_block >= 16 && rows_per_block <= kGatherMaxRows && rows_per_block % 16 == 0;
}

hipError_t launch_gather_probe(const void *k, const void *v, int64_t table_rows,
                               const int32_t *idx, int64_t n_idx, int rows_per_block,
                               uint32_t *sink, hipStream_t st) {
  if (n_idx == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_probe_kernel, dim3((unsigned)gather_probe_blocks(n_idx, rows_per_block)),
                     dim3(kProbeThreads), 0, st, static_cast<const u32x4 *>(k),
                     static_cast<const u32x4 *>(v), table_rows, idx, n_idx, rows_per_block, sink);
  return hipGetLastError();
}

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

}  // namespace
}  // namespace hk

using namespace hk;

namespace {
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline hk_status from_hip(hipError_t e) { return e == hipSuccess ? HK_OK : HK_ERR_HIP; }
inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }
}  // namespace

extern "C" {

size_t hk_read_probe_sink_words(size_t bytes) { return (size_t)read_probe_blocks(bytes); }

hk_status hk_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (bytes % 16 != 0) return HK_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return HK_OK;
  if (!src || !sink) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned16(src)) return HK_ERR_UNSUPPORTED;
  if (read_probe_blocks(bytes) > 0x7FFFFFFF) return HK_ERR_UNSUPPORTED;
  return from_hip(launch_read_probe(src, bytes, sink, as_stream(stream)));
}

size_t hk_gather_probe_sink_words(int64_t n_idx, int rows_per_block) {
  if (n_idx <= 0 || !gather_probe_rows_ok(rows_per_block)) return 0;
  return (size_t)gather_probe_blocks(n_idx, rows_per_block);
}

hk_status hk_gather_probe(const void *k, const void *v, int64_t table_rows, const int32_t *idx,
                          int64_t n_idx, int rows_per_block, uint32_t *sink, void *stream) {
  if (n_idx < 0 || !gather_probe_rows_ok(rows_per_block)) return HK_ERR_INVALID_ARGUMENT;
  if (n_idx == 0) return HK_OK;
  if (!k || !v || !idx || !sink || table_rows < 1) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v)) return HK_ERR_UNSUPPORTED;
  if (gather_probe_blocks(n_idx, rows_per_block) > 0x7FFFFFFF) return HK_ERR_UNSUPPORTED;
  return from_hip(launch_gather_probe(k, v, table_rows, idx, n_idx, rows_per_block, sink,
                                      as_stream(stream)));
}

}  // extern "C"
