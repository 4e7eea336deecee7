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
//   topk_emit      re-reads the one-byte distances of a group of chunks and writes the selected
//                  tokens (all with D < T, and the first `quota` with D == T in index
//                  order) at their final positions, so the output is ascending.
#include "encode_core.h"
#include "select_core.h"

namespace hk {
namespace {

// grid (S, BH); chunk c of head bh covers candidate offsets [c*CH, (c+1)*CH).  The
// histogram of the chunk goes to hist[bh][c]: bins 0 .. 32W-1, then 4W "superbins", each
// the count of 8 consecutive distances (the count at distance 32W follows from the
// chunk size).
// ctx_len (device, [B]; NULL = every sequence has the full context) gives each sequence
// its own context length n_b <= max_ctx: head bh (of sequence bh / Hkv) then has
// C_b = max(0, n_b - n_local - lo) candidates, and workgroups past its last chunk end
// at once (the threshold reads only the head's own chunks).
// NT_STASH: the distance bytes are stored non-temporally.  Measured: with 16.7 MB of
// distance bytes (16 x 8 heads x 131072 tokens) the scan takes 47.5 us against 49.2 with
// ordinary stores, with 4.2 MB (8 x 524288) 13.0 against 12.4 -- so the launch picks
// non-temporal stores when the distance bytes exceed a quarter of the 32 MB of L2.
constexpr int64_t kStashNtBytes = 8 << 20;
// The parameters that the first memory requests need come first: the first 16 dwords of
// the arguments are preloaded into SGPRs, so the code loads issue without waiting for a
// scalar load of the arguments.
// grid (Sx, BH) with Sx <= S: workgroup x scans chunks x, x + Sx, x + 2 Sx, ... of its
// head, requesting the next chunk's codes as soon as the current one's distances are
// computed (the registers are free then), so that they are in flight while it writes
// out the current histogram; two LDS histograms alternate.  The launch gives every
// workgroup one chunk (Sx = S): four chunks per workgroup, one round of 2048 workgroups
// on 16 x 8 heads of 131072 tokens, measured 51.9 us against 47.1 with a workgroup per
// chunk, while this form of the kernel at one chunk per workgroup measured 1.5-1.7%
// faster than the earlier straight-line one (8 heads x 524288 128-bit codes: 12.12
// against 12.32 us; 16 x 8 heads of 131072: 46.9 against 47.1), with the same loads in
// the same order.
template <int W, int LPT, bool NT_STASH>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes,
    const int32_t *__restrict__ ctx_len, int64_t cap, int64_t lo, int64_t C,
    uint8_t *__restrict__ stash, int S, uint32_t *__restrict__ hist_out, int Hkv,
    int64_t n_local, int64_t max_ctx) {
  constexpr int BINS = 32 * W;
  constexpr int NBP = BINS + 4;
  constexpr int CH = kScanThreads * LPT;
  constexpr int NSB = BINS / 8;
  static_assert(BINS + BINS / 8 <= kScanThreads, "one thread per histogram entry");
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ uint32_t hist[2][kScanThreads / 64][NBP];

  int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  if (ctx_len) {
    C = head_candidates(ctx_len, bh / Hkv, max_ctx, lo, n_local);
    if ((int64_t)c * CH >= C) return;
  }

  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  // Non-temporal loads: the codes are read exactly once.  Whole chunks load without
  // predication; only the last chunk of a head can be partial.
  auto request = [&](int cc, V (&v)[LPT]) {
    const int64_t p0 = (int64_t)cc * CH;
    const int64_t pw = p0 + (int64_t)wave * (64 * LPT) + (t & 63);   // item i: pw + 64*i
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
  };
  V v[LPT];
  request(c, v);

  // The histograms are cleared and the query code read while the codes are in flight
  // (the barrier waits for the LDS stores, not for the loads), and each token is then
  // processed as soon as its own load has landed.
  for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0][0])[i] = 0u;
  uint32_t q[W];
#pragma unroll
  for (int w = 0; w < W; ++w) q[w] = qcodes[(int64_t)bh * W + w];
  __syncthreads();

  for (int buf = 0;; buf ^= 1) {
    // Distance bytes in token order: item i of the wavefront is one 64-byte store.
    const int64_t pw = (int64_t)c * CH + (int64_t)wave * (64 * LPT) + (t & 63);
    uint8_t *st = stash + (int64_t)bh * S * CH + pw;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int64_t p = pw + 64 * i;
      uint32_t d = 0xFFu;                      // past the last candidate: never selected
      if (p < C) {
        d = CV::dist(v[i], q);
        atomicAdd(&hist[buf][wave][d], 1u);
      }
      if constexpr (NT_STASH)
        __builtin_nontemporal_store((uint8_t)d, st + 64 * i);
      else
        st[64 * i] = (uint8_t)d;
    }
    const int cn = c + (int)gridDim.x;
    const bool more = cn < S && (int64_t)cn * CH < C;                  // uniform
    if (more) request(cn, v);
    __syncthreads();
    uint32_t *out = hist_out + ((int64_t)bh * S + c) * (BINS + NSB);
    if (t < BINS) {
      uint32_t sum = 0;
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w) sum += hist[buf][w][t];
      out[t] = sum;
    } else if (t < BINS + NSB) {
      const int b0 = 8 * (t - BINS);
      uint32_t sum = 0;
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += hist[buf][w][b0 + e];
      out[t] = sum;
    }
    if (!more) break;
    for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads)
      (&hist[buf ^ 1][0][0])[i] = 0u;
    __syncthreads();
    c = cn;
  }
}

// As hamming_scan_kernel (ordinary distance stores, every sequence at full length), with
// the query hash computed by each workgroup from the query rows itself (enc::
// wg_query_code), which removes the query encoder's kernel and its dependent round
// trip from a latency-bound step; chunk 0 of every head writes the code it used to
// qcodes.  The code loads are issued first and land while the code is computed.
template <int W, int LPT, bool BF16, int KIND>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_query_kernel(
    const uint32_t *__restrict__ codes, int64_t cap, int64_t lo, int64_t C,
    uint8_t *__restrict__ stash, int S, uint32_t *__restrict__ hist_out, enc::HashPtrs hp,
    const void *__restrict__ q, int Hq, int Hkv, uint32_t *__restrict__ qcodes) {
  constexpr int BINS = 32 * W;
  constexpr int NBP = BINS + 4;
  constexpr int CH = kScanThreads * LPT;
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ uint32_t hist[kScanThreads / 64][NBP];
  __shared__ float xs[kHeadDim];
  __shared__ float hid[kHidden];
  __shared__ uint32_t qw[W];

  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int64_t p0 = (int64_t)c * CH;
  const int64_t pw = p0 + (int64_t)wave * (64 * LPT) + (t & 63);
  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  V v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int64_t p = pw + 64 * i;
    v[i] = (p < C) ? __builtin_nontemporal_load(base + p) : CV::zero();
  }
  for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0])[i] = 0u;
  const int64_t b = bh / Hkv;
  enc::wg_query_code<BF16, KIND, 32 * W>(hp, q, b, (int)(bh - b * Hkv), Hq, Hkv, xs, hid, qw);
  uint32_t qq[W];
#pragma unroll
  for (int w = 0; w < W; ++w) qq[w] = qw[w];
  if (c == 0 && t < W) qcodes[(int64_t)bh * W + t] = qw[t];

  uint8_t *st = stash + (int64_t)bh * S * CH + pw;
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int64_t p = pw + 64 * i;
    uint32_t d = 0xFFu;
    if (p < C) {
      d = CV::dist(v[i], qq);
      atomicAdd(&hist[wave][d], 1u);
    }
    st[64 * i] = (uint8_t)d;
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

// grid (BH); one workgroup per head: head_threshold, with meta, params and count
// written to the workspace.
template <int BINS>
__global__ __launch_bounds__(kThrThreads) void topk_threshold_kernel(
    const uint32_t *__restrict__ hist, int S, int64_t C, int CH, int keff,
    int4 *__restrict__ meta, int2 *__restrict__ params, int32_t *__restrict__ count) {
  const int bh = blockIdx.x;
  int T, quota;
  head_threshold<BINS>(hist + (int64_t)bh * S * (BINS + BINS / 8), S, C, CH, keff, T, quota,
                       [&](int c, const int4 &m) { meta[(int64_t)bh * S + c] = m; });
  if (threadIdx.x == 0) {
    params[bh] = make_int2(T, quota);
    count[bh] = keff;
  }
}

// grid (ceil(S / CPE), BH): group g of head bh covers chunks [g*CPE, min(S, (g+1)*CPE)),
// one run of the head's distance bytes; thread t takes its tokens [t*TPT, (t+1)*TPT) with
// TPT = CPE*LPT.  The group's counts below / at T before it are its first chunk's meta,
// and its own counts follow from its last chunk's.
template <int LPT, int CPE>
__global__ __launch_bounds__(kScanThreads) void topk_emit_kernel(
    const uint8_t *__restrict__ stash, const int4 *__restrict__ meta,
    const int2 *__restrict__ params, int S, int64_t lo, int k, int32_t *__restrict__ idx) {
  constexpr int CH = kScanThreads * LPT;
  constexpr int TPT = CPE * LPT;
  __shared__ uint32_t lds[kScanThreads / 64];
  const int c0 = blockIdx.x * CPE;
  const int c1 = min(S, c0 + CPE);
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  // Issue every load of the block before branching on any of them.
  const int2 pr = params[bh];
  const int4 mf = meta[(int64_t)bh * S + c0];
  const int4 ml = meta[(int64_t)bh * S + c1 - 1];
  uint32_t w[TPT / 4];
  load_run<TPT>(stash + ((int64_t)bh * S + c0) * CH, (int64_t)t * TPT,
                (int64_t)t * TPT < (int64_t)(c1 - c0) * CH, w);
  const int T = pr.x;
  const int quota = pr.y;
  const int lt = ml.x + ml.z - mf.x;           // the group's tokens below T
  const int eq = ml.y + ml.w - mf.y;           // and at T
  const int ties = quota - mf.y;
  if (T < 0 || lt + (ties <= 0 ? 0 : (ties < eq ? ties : eq)) == 0) return;
  RunSelect<TPT> rs;
  rs.build(w, T, quota, mf.x, mf.y, lds);
  int32_t *out = idx + (int64_t)bh * k + rs.first;
  const int32_t tok0 = (int32_t)(lo + (int64_t)c0 * CH) + TPT * t;
  rs.emit(0, rs.total, [&](int pos, int off) { out[pos] = tok0 + off; });
}

// Chunks per emit workgroup: the fewest (a power of two, at most 8) with which the grid
// fits in one round of resident workgroups (8 per CU).  One chunk per workgroup leaves
// the emit a chain of short rounds on many chunks (16384 chunks of the 112 query heads of
// 4 sequences x 262144 tokens: seven rounds), each paying a load round trip and a scan.
constexpr int64_t kEmitResident = 2048;
template <int LPT>
void emit_launch(const RetrievePlan &p, const uint8_t *stash, const int4 *meta,
                 const int2 *params, int k, int32_t *idx, hipStream_t st) {
  int cpe = 1;
  while (cpe < 8 && (int64_t)((p.S + cpe - 1) / cpe) * p.BH > kEmitResident) cpe *= 2;
  const dim3 grid((unsigned)((p.S + cpe - 1) / cpe), (unsigned)p.BH), blk(kScanThreads);
#define HK_EMIT(CC)                                                                          \
  case CC:                                                                                   \
    hipLaunchKernelGGL((topk_emit_kernel<LPT, CC>), grid, blk, 0, st, stash, meta, params,  \
                       p.S, p.lo, k, idx);                                                   \
    break;
  switch (cpe) { HK_EMIT(1) HK_EMIT(2) HK_EMIT(4) HK_EMIT(8) default: break; }
#undef HK_EMIT
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
template <int W, int LPT, int G, bool NT_STASH>
__global__ __launch_bounds__(kScanThreads) void hamming_scan_group_kernel(
    const uint32_t *__restrict__ codes, const uint32_t *__restrict__ qcodes, int64_t cap,
    int64_t lo, int64_t C, int S, uint8_t *__restrict__ stash, uint32_t *__restrict__ hist_out) {
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
    uint8_t *st = stash + ((int64_t)bh * G + g) * S * CH + pw;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int64_t p = pw + 64 * i;
      uint32_t d = 0xFFu;
      if (p < C) {
        d = CV::dist(v[i], q[g]);
        atomicAdd(&hist[g][wave][d], 1u);
      }
      if constexpr (NT_STASH)
        __builtin_nontemporal_store((uint8_t)d, st + 64 * i);
      else
        st[64 * i] = (uint8_t)d;
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
                       const uint32_t *qcodes, int64_t cap, uint8_t *stash, uint32_t *hist,
                       hipStream_t st) {
  const dim3 grid(p.S, p.BH / G), blk(kScanThreads);
  // p.BH counts query heads here: the distance bytes of all of them
  const bool nt = (int64_t)p.BH * p.S * p.ch > kStashNtBytes;
#define HK_GS(GG)                                                                            \
  case GG:                                                                                   \
    if (nt)                                                                                  \
      hipLaunchKernelGGL((hamming_scan_group_kernel<W, LPT, GG, true>), grid, blk, 0, st,    \
                         codes, qcodes, cap, p.lo, p.C, p.S, stash, hist);                   \
    else                                                                                     \
      hipLaunchKernelGGL((hamming_scan_group_kernel<W, LPT, GG, false>), grid, blk, 0, st,   \
                         codes, qcodes, cap, p.lo, p.C, p.S, stash, hist);                   \
    break;
  switch (G) { HK_GS(2) HK_GS(3) HK_GS(4) HK_GS(5) HK_GS(6) HK_GS(7) HK_GS(8) default: break; }
#undef HK_GS
}

template <int W, int LPT>
void scan_launch(const RetrievePlan &p, const uint32_t *codes, const uint32_t *qcodes,
                 int64_t cap, uint8_t *stash, uint32_t *hist, const int32_t *ctx_len, int Hkv,
                 int64_t n_local, int64_t max_ctx, hipStream_t st) {
  const dim3 grid((unsigned)p.S, (unsigned)p.BH);              // one chunk per workgroup
  if ((int64_t)p.BH * p.S * p.ch > kStashNtBytes)
    hipLaunchKernelGGL((hamming_scan_kernel<W, LPT, true>), grid, dim3(kScanThreads),
                       0, st, codes, qcodes, ctx_len, cap, p.lo, p.C, stash, p.S, hist, Hkv,
                       n_local, max_ctx);
  else
    hipLaunchKernelGGL((hamming_scan_kernel<W, LPT, false>), grid, dim3(kScanThreads),
                       0, st, codes, qcodes, ctx_len, cap, p.lo, p.C, stash, p.S, hist, Hkv,
                       n_local, max_ctx);
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
                               hipStream_t st, const int32_t *ctx_len, int Hkv,
                               int64_t n_local, int64_t max_ctx) {
  if (p.BH == 0 || p.S == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint8_t *stash = w8 + p.off_stash;
  uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + p.off_hist);
#define HK_SCAN(WW, LL) \
  scan_launch<WW, LL>(p, codes, qcodes, cap, stash, hist, ctx_len, Hkv, n_local, max_ctx, st)
  if (p.W == 4) {
    if (p.lpt == 8) HK_SCAN(4, 8);
    else HK_SCAN(4, 4);
  } else {
    if (p.lpt == 8) HK_SCAN(2, 8);
    else HK_SCAN(2, 4);
  }
#undef HK_SCAN
  return hipGetLastError();
}

bool scan_hashes_query(const RetrievePlan &p, const hk_hash &h) {
  if (p.BH == 0 || p.S == 0) return false;
  // Sign codes need no weights: every scan workgroup only averages its group's query
  // rows, which costs less than the query encoder's kernel and its boundary (4 x 262144
  // tokens, 4 KV heads: 35.1 against 38.4 us per step).
  if (h.kind == HK_HASH_SIGN) return true;
  // Every scan workgroup reads the hash's weight rows (128 KB for a bf16 MLP, 16 KB for
  // bf16 LSH-64): worth a kernel boundary only while the workgroups are few (on the same
  // workload LSH-64 in 2048 workgroups took 35.8 against 33.4 us per step).
  return (int64_t)p.BH * p.S * p.ch <= kStashNtBytes && (int64_t)p.BH * p.S <= kScanQueryMaxBlocks;
}

hipError_t launch_hamming_scan_query(const RetrievePlan &p, const hk_hash &h, const void *q,
                                     int Hq, int Hkv, const uint32_t *codes, int64_t cap,
                                     uint32_t *qcodes, void *ws, hipStream_t st) {
  if (p.BH == 0 || p.S == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint8_t *stash = w8 + p.off_stash;
  uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + p.off_hist);
  const enc::HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const dim3 grid(p.S, p.BH), blk(kScanThreads);
#define HK_SQ(WW, LL, BF, KK)                                                                 \
  hipLaunchKernelGGL((hamming_scan_query_kernel<WW, LL, BF, KK>), grid, blk, 0, st, codes, cap, \
                     p.lo, p.C, stash, p.S, hist, hp, q, Hq, Hkv, qcodes)
#define HK_SQ_K(WW, LL, BF)                                                                   \
  if (h.kind == HK_HASH_MLP) HK_SQ(WW, LL, BF, enc::kMlp);                                    \
  else if (h.kind == HK_HASH_LSH) HK_SQ(WW, LL, BF, enc::kLsh);                               \
  else if (WW == 4) HK_SQ(4, LL, BF, enc::kSign);
#define HK_SQ_B(WW, LL)                                                                       \
  if (h.dtype == HK_BF16) { HK_SQ_K(WW, LL, true) } else { HK_SQ_K(WW, LL, false) }
  if (p.W == 4) {
    if (p.lpt == 8) { HK_SQ_B(4, 8) } else { HK_SQ_B(4, 4) }
  } else {
    if (p.lpt == 8) { HK_SQ_B(2, 8) } else { HK_SQ_B(2, 4) }
  }
#undef HK_SQ_B
#undef HK_SQ_K
#undef HK_SQ
  return hipGetLastError();
}

hipError_t launch_hamming_scan_qheads(const RetrievePlan &p, int G, const uint32_t *codes,
                                      const uint32_t *qcodes, int64_t cap, void *ws,
                                      hipStream_t st) {
  if (G == 1) return launch_hamming_scan(p, codes, qcodes, cap, ws, st);
  if (p.BH == 0 || p.S == 0) return hipSuccess;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint8_t *stash = w8 + p.off_stash;
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
  const uint8_t *stash = w8 + p.off_stash;
  const int4 *meta = reinterpret_cast<const int4 *>(w8 + p.off_meta);
  const int2 *params = reinterpret_cast<const int2 *>(w8 + p.off_params);
  if (p.lpt == 8)
    emit_launch<8>(p, stash, meta, params, k, idx, st);
  else
    emit_launch<4>(p, stash, meta, params, k, idx, st);
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
