// HashEvict's eviction step (HashEvict: Abstract): at every decode step the cached token
// least similar to the current query -- the largest Hamming distance between its key
// code and the query code -- is the victim, and the current token's key, value and key
// code take its slot.
//
//   evict_scan     grid (S, B*Hkv): one workgroup per chunk of 2048 candidates reads
//                  each code once (the same coalesced 16- or 8-byte loads as the
//                  retrieval scan), and writes the chunk's best candidate as one 64-bit
//                  key (distance << 32 | ~token): the largest key is the largest
//                  distance, and among equal distances the lowest token.  Bound by HBM
//                  bandwidth.
//   evict_reduce   one workgroup per head: the largest key of the head's chunks, i.e.
//                  its victim (or -1 when the head has no candidate).
//   evict_replace  one workgroup per head: copies the new key and value rows and the new
//                  key code into the victim's slot.
// Deterministic: no atomics.
#include "hk_internal.h"

namespace hk {
namespace {

constexpr int kEvictThreads = 256;
constexpr int kEvictLpt = 8;
constexpr int kEvictChunk = kEvictThreads * kEvictLpt;

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v) {
  __shared__ uint64_t part[kEvictThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = umax64(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t m = 0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kEvictThreads / 64; ++w) m = umax64(m, part[w]);
  }
  return m;
}

template <int W>
__global__ __launch_bounds__(kEvictThreads) void evict_scan_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes, int64_t cap,
    int64_t lo, int64_t C, int S, uint64_t *__restrict__ part) {
  using CV = CodeVec<W>;
  using V = typename CV::T;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  uint32_t q[W];
#pragma unroll
  for (int w = 0; w < W; ++w) q[w] = qcodes[(int64_t)bh * W + w];
  const int64_t p0 = (int64_t)c * kEvictChunk + t;          // item i: p0 + 256*i
  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  V v[kEvictLpt];
#pragma unroll
  for (int i = 0; i < kEvictLpt; ++i) {
    const int64_t p = p0 + (int64_t)kEvictThreads * i;
    v[i] = p < C ? __builtin_nontemporal_load(base + p) : CV::zero();
  }
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < kEvictLpt; ++i) {
    const int64_t p = p0 + (int64_t)kEvictThreads * i;
    if (p < C) {
      const uint32_t tok = (uint32_t)(lo + p);
      best = umax64(best, ((uint64_t)CV::dist(v[i], q) << 32) | (uint64_t)(0xFFFFFFFFu - tok));
    }
  }
  best = block_max_u64(best);
  if (t == 0) part[(int64_t)bh * S + c] = best;
}

__global__ __launch_bounds__(kEvictThreads) void evict_reduce_kernel(
    const uint64_t *__restrict__ part, int S, int32_t *__restrict__ victim) {
  const int bh = blockIdx.x;
  uint64_t best = 0;
  for (int c = threadIdx.x; c < S; c += kEvictThreads) best = umax64(best, part[(int64_t)bh * S + c]);
  best = block_max_u64(best);
  if (threadIdx.x == 0) victim[bh] = best ? (int32_t)(0xFFFFFFFFu - (uint32_t)best) : -1;
}

// One workgroup of 64 threads per head; `row16` 16-byte pieces per K or V row.
__global__ __launch_bounds__(64) void evict_replace_kernel(
    const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
    const uint32_t *__restrict__ code_new, int row16, int W, int64_t cap,
    const int32_t *__restrict__ victim, uint4 *__restrict__ kc, uint4 *__restrict__ vc,
    uint32_t *__restrict__ codes) {
  const int bh = blockIdx.x;
  const int32_t j = victim[bh];
  if (j < 0 || j >= cap) return;
  const size_t slot = (size_t)bh * (size_t)cap + (size_t)j;
  for (int e = threadIdx.x; e < row16; e += 64) {
    kc[slot * row16 + e] = k_new[(size_t)bh * row16 + e];
    vc[slot * row16 + e] = v_new[(size_t)bh * row16 + e];
  }
  if (threadIdx.x < W) codes[slot * W + threadIdx.x] = code_new[(size_t)bh * W + threadIdx.x];
}

}  // namespace

EvictPlan plan_evict(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local) {
  EvictPlan p;
  p.W = bits / 32;
  p.BH = B * Hkv;
  p.lo = n_sink;
  const int64_t hi = n_ctx - n_local;
  p.C = hi > p.lo ? hi - p.lo : 0;
  p.S = (int)((p.C + kEvictChunk - 1) / kEvictChunk);
  p.total = align_up((size_t)p.BH * (size_t)(p.S > 0 ? p.S : 1) * sizeof(uint64_t), 256);
  return p;
}

hipError_t launch_evict_select(const EvictPlan &p, const uint32_t *codes, const uint32_t *qcodes,
                               int64_t cap, int32_t *victim, void *ws, hipStream_t st) {
  uint64_t *part = static_cast<uint64_t *>(ws);
  if (p.S > 0) {
    if (p.W == 4)
      hipLaunchKernelGGL(evict_scan_kernel<4>, dim3(p.S, p.BH), dim3(kEvictThreads), 0, st, codes,
                         qcodes, cap, p.lo, p.C, p.S, part);
    else
      hipLaunchKernelGGL(evict_scan_kernel<2>, dim3(p.S, p.BH), dim3(kEvictThreads), 0, st, codes,
                         qcodes, cap, p.lo, p.C, p.S, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(evict_reduce_kernel, dim3(p.BH), dim3(kEvictThreads), 0, st, part, p.S,
                     victim);
  return hipGetLastError();
}

hipError_t launch_evict_replace(const void *k_new, const void *v_new, const uint32_t *code_new,
                                int elem_bytes, int W, int BH, int64_t cap, const int32_t *victim,
                                void *kc, void *vc, uint32_t *codes, hipStream_t st) {
  const int row16 = kHeadDim * elem_bytes / 16;
  hipLaunchKernelGGL(evict_replace_kernel, dim3(BH), dim3(64), 0, st,
                     static_cast<const uint4 *>(k_new), static_cast<const uint4 *>(v_new),
                     code_new, row16, W, cap, victim, static_cast<uint4 *>(kc),
                     static_cast<uint4 *>(vc), codes);
  return hipGetLastError();
}

}  // namespace hk
