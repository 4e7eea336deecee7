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
//                  histogram per wavefront), written out per chunk.  This kernel is
//                  bound by HBM bandwidth.
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

// grid (S, BH); chunk c of head bh covers candidate offsets [c*CH, (c+1)*CH).  The
// histogram of the chunk goes to hist[bh][c]: bins 0 .. 32W-1, then 4W "superbins", each
// the count of 8 consecutive distances (the count at distance 32W follows from the
// chunk size).
template <int W, int LPT>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes, int64_t cap,
    int64_t lo, int64_t C, int S, uint32_t *__restrict__ stash, uint32_t *__restrict__ hist_out) {
  constexpr int BINS = 32 * W;
  constexpr int NBP = BINS + 4;
  constexpr int CH = kScanThreads * LPT;
  static_assert(BINS + BINS / 8 <= kScanThreads, "one thread per histogram entry");
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ uint32_t hist[kScanThreads / 64][NBP];

  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6;

  // The histograms are cleared and the query code read before the codes are requested:
  // a barrier after the code loads would make every thread wait for all of them, while
  // here each token is processed as soon as its own load has landed.
  for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0])[i] = 0u;
  uint32_t q[W];
#pragma unroll
  for (int w = 0; w < W; ++w) q[w] = qcodes[(int64_t)bh * W + w];
  __syncthreads();

  const int64_t p0 = (int64_t)c * CH;
  const int64_t pw = p0 + (int64_t)wave * (64 * LPT) + (t & 63);   // item i: pw + 64*i
  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  // Non-temporal loads: the codes are read exactly once.  Whole chunks load without
  // predication; only the last chunk of a head can be partial.
  V v[LPT];
  if (p0 + CH <= C) {
    const V *bp = base + pw;
#pragma unroll
    for (int i = 0; i < LPT; ++i) v[i] = __builtin_nontemporal_load(bp + 64 * i);
  } else {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int64_t p = pw + 64 * i;
      v[i] = (p < C) ? __builtin_nontemporal_load(base + p) : CV::zero();
    }
  }

  uint32_t *st = stash + ((int64_t)bh * S + c) * stash_words_per_chunk<LPT>();
#pragma unroll
  for (int i4 = 0; i4 < LPT / 4; ++i4) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * i4 + j;
      const int64_t p = pw + 64 * i;
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
  constexpr int NSB = BINS / 8;
  uint32_t *out = hist_out + ((int64_t)bh * S + c) * (BINS + NSB);
  if (t < BINS) {
    uint32_t sum = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) sum += hist[w][t];
    out[t] = sum;
  } else if (t < BINS + NSB) {
    const int b0 = 8 * (t - BINS);
    uint32_t sum = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += hist[w][b0 + e];
    out[t] = sum;
  }
}

// grid (BH); one workgroup per head, one thread per chunk (tiles of kThrThreads chunks).
// A two-level radix select over the chunk histograms:
//   1. superbin totals over all chunks -> the superbin holding T (or T = BINS when the
//      histogrammed distances hold fewer than k_eff candidates);
//   2. that superbin's 8 bins, totalled over the chunks -> T and the tie quota;
//   3. per chunk, #(D < T) (its superbins below T's plus its bins of T's superbin below
//      T) and #(D == T), then an exclusive prefix of both over chunks into meta.
// For up to kThrThreads chunks per head every value is read once and kept in registers.
constexpr int kThrThreads = 256;

template <int K>
__device__ __forceinline__ void load_u32x(const uint32_t *p, uint32_t (&x)[K]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

// Sum of K values over the workgroup: per-wavefront transposed sums, then LDS.
// Returns the total of value i in thread i < K (others: undefined).  red holds
// kThrThreads / 64 * 16 entries.
template <int K>
__device__ __forceinline__ uint32_t block_sum_k(uint32_t (&x)[K], uint32_t *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t r = wave_transpose_sum<K>(x);
  if (lane < K) red[wave * 16 + bitrev_k<K>(lane)] = r;
  __syncthreads();
  uint32_t t = 0;
  if ((int)threadIdx.x < K) {
#pragma unroll
    for (int w = 0; w < kThrThreads / 64; ++w) t += red[w * 16 + threadIdx.x];
  }
  __syncthreads();
  return t;
}

template <int BINS>
__global__ __launch_bounds__(kThrThreads) void topk_threshold_kernel(
    const uint32_t *__restrict__ hist, int S, int64_t C, int CH, int keff,
    int4 *__restrict__ meta, int2 *__restrict__ params, int32_t *__restrict__ count) {
  constexpr int NSB = BINS / 8;                // 16 or 8 superbins
  constexpr int ROW = BINS + NSB;
  constexpr int NT = kThrThreads;
  __shared__ uint32_t red[NT / 64 * 16];
  __shared__ uint32_t tot[16];
  __shared__ uint32_t scan_lds[2][NT / 64];
  __shared__ int sh[4];                        // T, quota, superbin of T, count below it
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t *hb = hist + (int64_t)bh * S * ROW;
  auto row = [&](int c) { return hb + (int64_t)(c < S ? c : S - 1) * ROW; };

  uint32_t sb0[NSB], bb0[8];                   // the first tile's values, kept
  if (keff > 0) {
    // 1. superbin totals
    uint32_t acc[NSB];
#pragma unroll
    for (int i = 0; i < NSB; ++i) acc[i] = 0u;
    for (int c0 = 0; c0 < S; c0 += NT) {
      uint32_t x[NSB];
      load_u32x<NSB>(row(c0 + tid) + BINS, x);
      const bool ok = c0 + tid < S;
#pragma unroll
      for (int i = 0; i < NSB; ++i) {
        x[i] = ok ? x[i] : 0u;
        acc[i] += x[i];
        if (c0 == 0) sb0[i] = x[i];
      }
    }
    const uint32_t st = block_sum_k<NSB>(acc, red);
    if (tid < NSB) tot[tid] = st;
    __syncthreads();
    if (tid == 0) {
      uint32_t below = 0;
      int s = 0;
      while (s < NSB && below + tot[s] < (uint32_t)keff) below += tot[s++];
      sh[2] = s;                               // NSB: T = BINS
      sh[3] = (int)below;
    }
    __syncthreads();
    const int Ts = sh[2];
    if (Ts < NSB) {
      // 2. the 8 bins of superbin Ts
      uint32_t bacc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bacc[i] = 0u;
      for (int c0 = 0; c0 < S; c0 += NT) {
        uint32_t x[8];
        load_u32x<8>(row(c0 + tid) + 8 * Ts, x);
        const bool ok = c0 + tid < S;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[i] = ok ? x[i] : 0u;
          bacc[i] += x[i];
          if (c0 == 0) bb0[i] = x[i];
        }
      }
      const uint32_t bt = block_sum_k<8>(bacc, red);
      if (tid < 8) tot[tid] = bt;
      __syncthreads();
      if (tid == 0) {
        uint32_t below = (uint32_t)sh[3];
        int b = 0;
        while (below + tot[b] < (uint32_t)keff) below += tot[b++];   // stops at b < 8
        sh[0] = 8 * Ts + b;
        sh[1] = keff - (int)below;
      }
    } else if (tid == 0) {
      sh[0] = BINS;
      sh[1] = keff - sh[3];
    }
  } else if (tid == 0) {
    sh[0] = -1;
    sh[1] = 0;
  }
  __syncthreads();
  const int T = sh[0];
  const int quota = sh[1];
  // 3. per-chunk counts and their prefix over chunks
  uint32_t carry_lt = 0, carry_eq = 0;
  for (int c0 = 0; c0 < S && T >= 0; c0 += NT) {
    const int c = c0 + tid;
    const int Ts = T >> 3;
    uint32_t sbv[NSB], bbv[8];
    if (c0 == 0) {
#pragma unroll
      for (int i = 0; i < NSB; ++i) sbv[i] = sb0[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) bbv[i] = bb0[i];
    } else {
      load_u32x<NSB>(row(c) + BINS, sbv);
      if (T < BINS) load_u32x<8>(row(c) + 8 * Ts, bbv);
    }
    uint32_t lt = 0, eq = 0;
    if (c < S) {
#pragma unroll
      for (int i = 0; i < NSB; ++i) lt += (i < Ts) ? sbv[i] : 0u;
      if (T < BINS) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lt += (8 * Ts + i < T) ? bbv[i] : 0u;
          eq += (8 * Ts + i == T) ? bbv[i] : 0u;
        }
      } else {                                 // distance BINS is not in the histogram
        const int64_t n = C - (int64_t)c * CH;
        eq = (uint32_t)(n < CH ? n : CH) - lt;
      }
    }
    uint32_t tl, te;
    const uint32_t lt_ex = block_excl_scan_u32<NT>(lt, scan_lds[0], tl);
    const uint32_t eq_ex = block_excl_scan_u32<NT>(eq, scan_lds[1], te);
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
  emit_chunks<LPT, 1>([&](int, int kk) { return w[kk]; }, [&](int) { return mt; }, 1, T, quota,
                      lo + (int64_t)c * CH, [&](int pos, int32_t tok) { out[pos] = tok; });
}

__global__ void window_indices_kernel(int32_t n_sinks, int64_t local0, int32_t n,
                                      int32_t *__restrict__ idx) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) idx[i] = (i < n_sinks) ? i : (int32_t)(local0 + (i - n_sinks));
}

// grid (S, B*Hkv): as hamming_scan_kernel, for the G query codes of one KV head at once
// (per-query-head selection): each code is read once and compared with every query code
// of the group; query head g of the group gets its own distance stash and histograms,
// laid out as if it were a head of its own (head index bh*G + g).
template <int W, int LPT, int G>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_group_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes, int64_t cap,
    int64_t lo, int64_t C, int S, uint32_t *__restrict__ stash, uint32_t *__restrict__ hist_out) {
  constexpr int BINS = 32 * W;
  constexpr int NBP = BINS + 4;
  constexpr int CH = kScanThreads * LPT;
  constexpr int NSB = BINS / 8;
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ uint32_t hist[G][kScanThreads / 64][NBP];

  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  for (int i = t; i < G * (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0][0])[i] = 0u;
  uint32_t q[G][W];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int w = 0; w < W; ++w) q[g][w] = qcodes[((int64_t)bh * G + g) * W + w];
  __syncthreads();

  const int64_t p0 = (int64_t)c * CH;
  const int64_t pw = p0 + (int64_t)wave * (64 * LPT) + (t & 63);
  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  V v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int64_t p = pw + 64 * i;
    v[i] = (p < C) ? __builtin_nontemporal_load(base + p) : CV::zero();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t *st = stash + (((int64_t)bh * G + g) * S + c) * stash_words_per_chunk<LPT>();
#pragma unroll
    for (int i4 = 0; i4 < LPT / 4; ++i4) {
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * i4 + j;
        const int64_t p = pw + 64 * i;
        uint32_t d = 0xFFu;
        if (p < C) {
          d = CV::dist(v[i], q[g]);
          atomicAdd(&hist[g][wave][d], 1u);
        }
        packed |= d << (8 * j);
      }
      st[i4 * kScanThreads + t] = packed;
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t *out = hist_out + (((int64_t)bh * G + g) * S + c) * (BINS + NSB);
    if (t < BINS) {
      uint32_t sum = 0;
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w) sum += hist[g][w][t];
      out[t] = sum;
    } else if (t < BINS + NSB) {
      const int b0 = 8 * (t - BINS);
      uint32_t sum = 0;
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += hist[g][w][b0 + e];
      out[t] = sum;
    }
  }
}

template <int W, int LPT>
void scan_group_launch(const RetrievePlan &p, int G, const uint32_t *codes,
                       const uint32_t *qcodes, int64_t cap, uint32_t *stash, uint32_t *hist,
                       hipStream_t st) {
  const dim3 grid(p.S, p.BH / G), blk(kScanThreads);
#define HK_GS(GG)                                                                            \
  case GG:                                                                                   \
    hipLaunchKernelGGL((hamming_scan_group_kernel<W, LPT, GG>), grid, blk, 0, st, codes,     \
                       qcodes, cap, p.lo, p.C, p.S, stash, hist);                            \
    break;
  switch (G) { HK_GS(2) HK_GS(3) HK_GS(4) HK_GS(5) HK_GS(6) HK_GS(7) HK_GS(8) default: break; }
#undef HK_GS
}

template <int W, int LPT>
void scan_launch(const RetrievePlan &p, const uint32_t *codes, const uint32_t *qcodes,
                 int64_t cap, uint32_t *stash, uint32_t *hist, hipStream_t st) {
  hipLaunchKernelGGL((hamming_scan_kernel<W, LPT>), dim3(p.S, p.BH), dim3(kScanThreads), 0,
                     st, codes, qcodes, cap, p.lo, p.C, p.S, stash, hist);
}

}  // namespace

RetrievePlan plan_retrieve(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                           int k) {
  RetrievePlan p;
  p.W = bits / 32;
  p.BINS = bits;
  p.BH = B * Hkv;
  p.lo = n_sink;
  const int64_t hi = n_ctx - n_local;
  p.C = hi > p.lo ? hi - p.lo : 0;
  p.keff = (int)(k < p.C ? k : p.C);
  if (p.keff < 0) p.keff = 0;
  // Chunk size: 2048 codes (8 per thread) when that still gives >= 1024 workgroups, so
  // that 256 CUs each see several, else 1024.  Larger chunks lengthen each workgroup's
  // tail (the histogram and distance stores follow its last load) and measured slower.
  const int64_t tok = (int64_t)p.BH * p.C;
  p.lpt = (tok + 2047) / 2048 >= 1024 ? 8 : 4;
  p.ch = kScanThreads * p.lpt;
  p.S = (int)((p.C + p.ch - 1) / p.ch);
  size_t off = 0;
  p.off_stash = off;
  off = align_up(off + (size_t)p.BH * p.S * p.ch, 256);
  p.off_hist = off;
  off = align_up(off + (size_t)p.BH * p.S * (p.BINS + p.BINS / 8) * sizeof(uint32_t), 256);
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
  uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + p.off_hist);
  if (p.W == 4) {
    if (p.lpt == 8) scan_launch<4, 8>(p, codes, qcodes, cap, stash, hist, st);
    else scan_launch<4, 4>(p, codes, qcodes, cap, stash, hist, st);
  } else {
    if (p.lpt == 8) scan_launch<2, 8>(p, codes, qcodes, cap, stash, hist, st);
    else scan_launch<2, 4>(p, codes, qcodes, cap, stash, hist, st);
  }
  return hipGetLastError();
}

hipError_t launch_hamming_scan_qheads(const RetrievePlan &p, int G, const uint32_t *codes,
                                      const uint32_t *qcodes, int64_t cap, void *ws,
                                      hipStream_t st) {
  if (G == 1) return launch_hamming_scan(p, codes, qcodes, cap, ws, st);
  if (p.BH == 0 || p.S == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint32_t *stash = reinterpret_cast<uint32_t *>(w8 + p.off_stash);
  uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + p.off_hist);
  if (p.W == 4) {
    if (p.lpt == 8) scan_group_launch<4, 8>(p, G, codes, qcodes, cap, stash, hist, st);
    else scan_group_launch<4, 4>(p, G, codes, qcodes, cap, stash, hist, st);
  } else {
    if (p.lpt == 8) scan_group_launch<2, 8>(p, G, codes, qcodes, cap, stash, hist, st);
    else scan_group_launch<2, 4>(p, G, codes, qcodes, cap, stash, hist, st);
  }
  return hipGetLastError();
}

hipError_t launch_topk_threshold(const RetrievePlan &p, int32_t *count, void *ws,
                                 hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  const uint32_t *hist = reinterpret_cast<const uint32_t *>(w8 + p.off_hist);
  int4 *meta = reinterpret_cast<int4 *>(w8 + p.off_meta);
  int2 *params = reinterpret_cast<int2 *>(w8 + p.off_params);
  if (p.BINS == 128)
    hipLaunchKernelGGL((topk_threshold_kernel<128>), dim3(p.BH), dim3(kThrThreads), 0, st,
                       hist, p.S, p.C, p.ch, p.keff, meta, params, count);
  else
    hipLaunchKernelGGL((topk_threshold_kernel<64>), dim3(p.BH), dim3(kThrThreads), 0, st,
                       hist, p.S, p.C, p.ch, p.keff, meta, params, count);
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
  if (p.lpt == 8)
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
