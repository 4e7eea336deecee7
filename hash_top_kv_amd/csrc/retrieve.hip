// Per-head top-k retrieval by Hamming distance between packed sign-bit codes.
//
// The query code of a (batch, KV head) is compared with every cached key code of that
// head (HashEvict: Abstract; Spotlight Attention: Key results, "bitwise hashing
// retrieval"), and the k nearest candidates are kept with ties broken by token index.
//
// Three kernels, all of them deterministic (no result depends on the order of atomics):
//   hamming_scan   reads each candidate code once with 16-byte (or 8-byte) loads,
//                  XOR + popcount against the query code, stores the distance as one
//                  byte, and builds the chunk's distance histogram in LDS (one private
//                  histogram per wavefront).  The chunk's cumulative histogram goes to
//                  the workspace.  This kernel is bound by HBM bandwidth.
//   topk_threshold one workgroup per head: sums the chunk histograms, finds the
//                  threshold T = min{t : #(D <= t) >= k_eff} and the tie quota
//                  k_eff - #(D < T), and an exclusive prefix over chunks of the counts
//                  below and at T.  No sort is needed: the histogram select replaces it.
//   topk_emit      re-reads the one-byte distances of a chunk and writes the selected
//                  tokens (all with D < T, and the first `quota` with D == T in index
//                  order) at their final positions, so the output is ascending.
#include "select_core.h"

namespace hk {
namespace {

constexpr int kSelThreads = 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int W> struct CodeVec;
template <> struct CodeVec<4> {
  using T = u32x4;
  __device__ static T zero() { return T{0u, 0u, 0u, 0u}; }
  __device__ static uint32_t dist(const T &v, const uint32_t *q) {
    return __builtin_popcount(v.x ^ q[0]) + __builtin_popcount(v.y ^ q[1]) +
           __builtin_popcount(v.z ^ q[2]) + __builtin_popcount(v.w ^ q[3]);
  }
};
template <> struct CodeVec<2> {
  using T = u32x2;
  __device__ static T zero() { return T{0u, 0u}; }
  __device__ static uint32_t dist(const T &v, const uint32_t *q) {
    return __builtin_popcount(v.x ^ q[0]) + __builtin_popcount(v.y ^ q[1]);
  }
};

// grid (S, BH); chunk c of head bh covers candidate offsets [c*CH, (c+1)*CH).
template <int W, int LPT>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes, int64_t cap,
    int64_t lo, int64_t C, int S, uint32_t *__restrict__ stash, uint32_t *__restrict__ cum) {
  constexpr int NB = 32 * W + 1;
  constexpr int NBP = (NB + 3) & ~3;
  constexpr int CH = kScanThreads * LPT;
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ uint32_t hist[kScanThreads / 64][NBP];

  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;

  const int64_t p0 = (int64_t)c * CH;
  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  // Stream the chunk's codes first (non-temporal: they are read exactly once).
  V v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int64_t p = p0 + i * kScanThreads + t;
    v[i] = (p < C) ? __builtin_nontemporal_load(base + p) : CV::zero();
  }
  for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0])[i] = 0u;
  uint32_t q[W];
#pragma unroll
  for (int w = 0; w < W; ++w) q[w] = qcodes[(int64_t)bh * W + w];
  __syncthreads();

  uint32_t *st = stash + ((int64_t)bh * S + c) * stash_words_per_chunk<LPT>();
#pragma unroll
  for (int i4 = 0; i4 < LPT / 4; ++i4) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * i4 + j;
      const int64_t p = p0 + i * kScanThreads + t;
      uint32_t d = 0xFFu;                      // past the last candidate: never selected
      if (p < C) {
        d = CV::dist(v[i], q);
        atomicAdd(&hist[wave][d], 1u);
      }
      packed |= d << (8 * j);
    }
    st[i4 * kScanThreads + t] = packed;
  }
  __syncthreads();
  // Inclusive cumulative histogram by one wavefront: lane l owns bins 2l, 2l+1 (and the
  // last lane also bin NB-1 when NB is odd).
  if (wave == 0) {
    auto bin = [&](int b) -> uint32_t {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w) s += hist[w][b];
      return s;
    };
    constexpr int PAIRS = (NB - 1) / 2;                // 64 or 32
    uint32_t a = 0, b = 0;
    if (lane < PAIRS) {
      a = bin(2 * lane);
      b = bin(2 * lane + 1);
    }
    const uint32_t inc = wave_incl_scan_u32(a + b);
    uint32_t *out = cum + ((int64_t)bh * S + c) * NB;
    if (lane < PAIRS) {
      out[2 * lane] = inc - b;
      out[2 * lane + 1] = inc;
    }
    if (lane == PAIRS - 1) out[NB - 1] = inc + bin(NB - 1);
  }
}

// grid (BH); one workgroup per head.  Every load phase keeps all its loads in flight.
template <int NB>
__global__ __launch_bounds__(kSelThreads) void topk_threshold_kernel(
    const uint32_t *__restrict__ cum, int S, int keff, int4 *__restrict__ meta,
    int2 *__restrict__ params, int32_t *__restrict__ count) {
  constexpr int BINS = NB - 1;                 // 128 or 64 (the last bin is extra)
  constexpr int NGR = kSelThreads / BINS;      // 8 or 16 groups of chunks
  constexpr int UNR = 8;
  __shared__ uint32_t part[NGR][NB];
  __shared__ uint32_t gcum[NB];
  __shared__ uint32_t scan_lds[2][kSelThreads / 64];
  __shared__ int sT, sQ;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t *cb = cum + (int64_t)bh * S * NB;

  if (tid == 0) {
    sT = -1;
    sQ = 0;
  }
  if (keff > 0) {
    const int tb = tid % BINS, g = tid / BINS;
    uint32_t s = 0, s_last = 0;
    for (int c0 = g; c0 < S; c0 += NGR * UNR) {
      uint32_t vals[UNR], lastv[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * NGR;
        vals[u] = c < S ? cb[(int64_t)c * NB + tb] : 0u;
        lastv[u] = (c < S && tb == 0) ? cb[(int64_t)c * NB + BINS] : 0u;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        s += vals[u];
        s_last += lastv[u];
      }
    }
    part[g][tb] = s;
    if (tb == 0) part[g][BINS] = s_last;
    __syncthreads();
    if (tid < NB) {
      uint32_t a = 0;
#pragma unroll
      for (int gg = 0; gg < NGR; ++gg) a += part[gg][tid];
      gcum[tid] = a;
    }
    __syncthreads();
    if (tid < NB) {
      const uint32_t below = tid ? gcum[tid - 1] : 0u;
      if (gcum[tid] >= (uint32_t)keff && below < (uint32_t)keff) {
        sT = tid;
        sQ = keff - (int)below;
      }
    }
  }
  __syncthreads();
  const int T = sT;
  const int quota = sQ;
  uint32_t carry_lt = 0, carry_eq = 0;
  for (int base = 0; base < S; base += kSelThreads) {
    const int c = base + tid;
    uint32_t lt = 0, eq = 0;
    if (c < S && T >= 0) {
      const uint32_t a = T > 0 ? cb[(int64_t)c * NB + T - 1] : 0u;
      const uint32_t b = cb[(int64_t)c * NB + T];
      lt = a;
      eq = b - a;
    }
    uint32_t tl, te;
    const uint32_t lt_ex = block_excl_scan_u32<kSelThreads>(lt, scan_lds[0], tl);
    const uint32_t eq_ex = block_excl_scan_u32<kSelThreads>(eq, scan_lds[1], te);
    if (c < S)
      meta[(int64_t)bh * S + c] =
          make_int4((int)(carry_lt + lt_ex), (int)(carry_eq + eq_ex), (int)lt, (int)eq);
    carry_lt += tl;
    carry_eq += te;
  }
  if (tid == 0) {
    params[bh] = make_int2(T, quota);
    count[bh] = keff;
  }
}

// grid (S, BH).  Same thread <-> token mapping as the scan.
template <int LPT>
__global__ __launch_bounds__(kScanThreads) void topk_emit_kernel(
    const uint32_t *__restrict__ stash, const int4 *__restrict__ meta,
    const int2 *__restrict__ params, int S, int64_t lo, int k, int32_t *__restrict__ idx) {
  constexpr int CH = kScanThreads * LPT;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  // Issue every load of the block before branching on any of them.
  const int2 pr = params[bh];
  const int4 mt = meta[(int64_t)bh * S + c];
  const uint32_t *sp = stash + ((int64_t)bh * S + c) * stash_words_per_chunk<LPT>();
  uint32_t w[LPT / 4];
#pragma unroll
  for (int i4 = 0; i4 < LPT / 4; ++i4) w[i4] = sp[i4 * kScanThreads + t];
  const int T = pr.x;
  const int quota = pr.y;
  if (T < 0 || chunk_selected(mt, quota) == 0) return;
  int32_t *out = idx + (int64_t)bh * k;
  emit_chunk<LPT>(w, T, quota, mt.x, mt.y, lo + (int64_t)c * CH,
                  [&](int pos, int, int32_t tok) { out[pos] = tok; });
}

__global__ void window_indices_kernel(int32_t n_sinks, int64_t local0, int32_t n,
                                      int32_t *__restrict__ idx) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) idx[i] = (i < n_sinks) ? i : (int32_t)(local0 + (i - n_sinks));
}

template <int W, int LPT>
void scan_launch(const RetrievePlan &p, const uint32_t *codes, const uint32_t *qcodes,
                 int64_t cap, uint32_t *stash, uint32_t *cum, hipStream_t st) {
  hipLaunchKernelGGL((hamming_scan_kernel<W, LPT>), dim3(p.S, p.BH), dim3(kScanThreads), 0,
                     st, codes, qcodes, cap, p.lo, p.C, p.S, stash, cum);
}

}  // namespace

RetrievePlan plan_retrieve(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                           int k) {
  RetrievePlan p;
  p.W = bits / 32;
  p.NB = bits + 1;
  p.BH = B * Hkv;
  p.lo = n_sink;
  const int64_t hi = n_ctx - n_local;
  p.C = hi > p.lo ? hi - p.lo : 0;
  p.keff = (int)(k < p.C ? k : p.C);
  if (p.keff < 0) p.keff = 0;
  // Chunk size: the largest of 16/8/4 codes per thread that still gives >= 1024
  // workgroups, so that 256 CUs each see several.
  const int64_t tok = (int64_t)p.BH * p.C;
  p.lpt = 16;
  if ((tok + 4095) / 4096 < 1024) p.lpt = 8;
  if (p.lpt == 8 && (tok + 2047) / 2048 < 1024) p.lpt = 4;
  p.ch = kScanThreads * p.lpt;
  p.S = (int)((p.C + p.ch - 1) / p.ch);
  size_t off = 0;
  p.off_stash = off;
  off = align_up(off + (size_t)p.BH * p.S * p.ch, 256);
  p.off_cum = off;
  off = align_up(off + (size_t)p.BH * p.S * p.NB * sizeof(uint32_t), 256);
  p.off_meta = off;
  off = align_up(off + (size_t)p.BH * p.S * sizeof(int4), 256);
  p.off_params = off;
  off = align_up(off + (size_t)p.BH * sizeof(int2), 256);
  p.total = off;
  return p;
}

hipError_t launch_hamming_scan(const RetrievePlan &p, const uint32_t *codes,
                               const uint32_t *qcodes, int64_t cap, void *ws,
                               hipStream_t st) {
  if (p.BH == 0 || p.S == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint32_t *stash = reinterpret_cast<uint32_t *>(w8 + p.off_stash);
  uint32_t *cum = reinterpret_cast<uint32_t *>(w8 + p.off_cum);
  if (p.W == 4) {
    if (p.lpt == 16) scan_launch<4, 16>(p, codes, qcodes, cap, stash, cum, st);
    else if (p.lpt == 8) scan_launch<4, 8>(p, codes, qcodes, cap, stash, cum, st);
    else scan_launch<4, 4>(p, codes, qcodes, cap, stash, cum, st);
  } else {
    if (p.lpt == 16) scan_launch<2, 16>(p, codes, qcodes, cap, stash, cum, st);
    else if (p.lpt == 8) scan_launch<2, 8>(p, codes, qcodes, cap, stash, cum, st);
    else scan_launch<2, 4>(p, codes, qcodes, cap, stash, cum, st);
  }
  return hipGetLastError();
}

hipError_t launch_topk_threshold(const RetrievePlan &p, int32_t *count, void *ws,
                                 hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  const uint32_t *cum = reinterpret_cast<const uint32_t *>(w8 + p.off_cum);
  int4 *meta = reinterpret_cast<int4 *>(w8 + p.off_meta);
  int2 *params = reinterpret_cast<int2 *>(w8 + p.off_params);
  if (p.NB == 129)
    hipLaunchKernelGGL((topk_threshold_kernel<129>), dim3(p.BH), dim3(kSelThreads), 0, st,
                       cum, p.S, p.keff, meta, params, count);
  else
    hipLaunchKernelGGL((topk_threshold_kernel<65>), dim3(p.BH), dim3(kSelThreads), 0, st,
                       cum, p.S, p.keff, meta, params, count);
  return hipGetLastError();
}

hipError_t launch_topk_select(const RetrievePlan &p, int k, int32_t *idx, int32_t *count,
                              void *ws, hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  hipError_t e = launch_topk_threshold(p, count, ws, st);
  if (e != hipSuccess || p.S == 0 || p.keff == 0) return e;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  const uint32_t *stash = reinterpret_cast<const uint32_t *>(w8 + p.off_stash);
  const int4 *meta = reinterpret_cast<const int4 *>(w8 + p.off_meta);
  const int2 *params = reinterpret_cast<const int2 *>(w8 + p.off_params);
  if (p.lpt == 16)
    hipLaunchKernelGGL((topk_emit_kernel<16>), dim3(p.S, p.BH), dim3(kScanThreads), 0, st,
                       stash, meta, params, p.S, p.lo, k, idx);
  else if (p.lpt == 8)
    hipLaunchKernelGGL((topk_emit_kernel<8>), dim3(p.S, p.BH), dim3(kScanThreads), 0, st,
                       stash, meta, params, p.S, p.lo, k, idx);
  else
    hipLaunchKernelGGL((topk_emit_kernel<4>), dim3(p.S, p.BH), dim3(kScanThreads), 0, st,
                       stash, meta, params, p.S, p.lo, k, idx);
  return hipGetLastError();
}

hipError_t launch_window_indices(int64_t n_ctx, int n_sink, int n_local, int32_t *idx,
                                 hipStream_t st) {
  const int64_t sinks = n_sink < n_ctx ? n_sink : n_ctx;
  const int64_t local0 = (n_ctx - n_local) > n_sink ? (n_ctx - n_local) : n_sink;
  const int64_t n = sinks + (n_ctx > local0 ? n_ctx - local0 : 0);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(window_indices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     st, (int32_t)sinks, local0, (int32_t)n, idx);
  return hipGetLastError();
}

}  // namespace hk
