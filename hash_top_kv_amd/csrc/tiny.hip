// The whole decode step of a small head in one workgroup: query hash, Hamming scan,
// top-k selection, attention over the selection and the window.
//
// For a head of at most kTinyC candidates with one query head per KV head (G = 1), the
// parallel path's three kernels (scan, select+attend, merge) and their dependent round
// trips cost more than the work itself.  One workgroup per (b, KV head) then does all of
// it:
//   1. requests its head's codes (token p = 256 i + t, so the loads coalesce);
//   2. computes the query code (enc::wg_query_code, the fp32 query encoder's arithmetic)
//      while the codes are in flight, and writes it to qcodes;
//   3. stores each candidate's distance in LDS (token order) and counts it in a
//      per-wavefront LDS histogram;
//   4. derives T = min{t : #(D <= t) >= k_eff} and the tie quota from the histogram by one
//      block scan (HashEvict: Abstract; Spotlight Attention: Key results);
//   5. selects with RunSelect over each thread's run of consecutive tokens, writing the
//      ascending index list to idx and to an LDS list;
//   6. attends in one online softmax over the sink + local window (RetrievalAttention:
//      the static tokens kept beside the retrieved ones; their rows are known at once, so
//      the attention starts with them while the codes load) and then over the selection,
//      storing the final o and lse (no partials, no merge).
// The selection is the same set as hk_retrieve_topk's for the same code; attention over
// the union in one pass equals the log-sum-exp merge of the two partial attentions up to
// rounding (RetrievalAttention, atlas summary: Approach).
#include "attend_core.h"
#include "encode_core.h"
#include "select_core.h"

namespace hk {
namespace {

constexpr int kTinyTpt = kTinyC / kScanThreads;       // tokens per thread
static_assert(kTinyTpt == 16, "RunSelect runs of 16 tokens");

template <int W, bool BF16, int KIND>
__global__ __launch_bounds__(kScanThreads) void tiny_step_kernel(
    const uint32_t *__restrict__ codes, const void *__restrict__ q, int64_t cap, int64_t lo,
    int64_t C, int keff, int k, enc::HashPtrs hp, int Hq, int Hkv, const void *__restrict__ kc,
    const void *__restrict__ vc, float scale_log2, int win_sinks, int64_t win_local0, int n_win,
    uint32_t *__restrict__ qcodes, int32_t *__restrict__ idx, int32_t *__restrict__ count,
    float *__restrict__ o, float *__restrict__ lse) {
  constexpr int BINS = 32 * W;
  constexpr int NBP = BINS + 4;
  constexpr int NI = kTinyTpt;                         // loads per thread
  using CV = CodeVec<W>;
  using V = typename CV::T;
  __shared__ __attribute__((aligned(16))) uint8_t dist[kTinyC];
  __shared__ uint32_t hist[kScanThreads / 64][NBP];
  __shared__ int32_t sel[kTinyList];                   // the selected tokens
  __shared__ float xs[kHeadDim];
  __shared__ float hid[kHidden];
  __shared__ uint32_t qw[W];
  __shared__ uint32_t scan_lds[kScanThreads / 64];
  __shared__ uint32_t ex_lds[BINS];
  __shared__ int first_lds[kScanThreads / 64];

  const int bh = blockIdx.x;
  const int64_t b = bh / Hkv;
  const int hg = (int)(bh - b * Hkv);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;

  const V *base = reinterpret_cast<const V *>(codes + ((int64_t)bh * cap + lo) * W);
  V v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t p = (int64_t)kScanThreads * i + t;
    v[i] = p < C ? base[p] : CV::zero();
  }
  for (int i = t; i < (kScanThreads / 64) * NBP; i += kScanThreads) (&hist[0][0])[i] = 0u;
  // The window's rows are known before the scan: the attention starts with them, so their
  // gather overlaps the code loads and the query hash.
  typename AttentionCore<BF16, 1>::type ga;
  const int64_t row0 = b * Hq + hg;                    // G = 1: query head = KV head
  const size_t head_row0 = (size_t)bh * (size_t)cap;
  ga.init(q, row0, scale_log2);
  ga.run_block(kc, vc, head_row0, n_win, [&](int r) {
    return r < win_sinks ? r : (int32_t)(win_local0 + (r - win_sinks));
  });
  enc::wg_query_code<BF16, KIND, BINS>(hp, q, b, hg, Hq, Hkv, xs, hid, qw);
  uint32_t qq[W];
#pragma unroll
  for (int w = 0; w < W; ++w) qq[w] = qw[w];
  if (t < W) qcodes[(int64_t)bh * W + t] = qw[t];

#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = kScanThreads * i + t;
    uint32_t d = 0xFFu;                                // past the last candidate
    if (p < C) {
      d = CV::dist(v[i], qq);
      atomicAdd(&hist[wave][d], 1u);
    }
    dist[p] = (uint8_t)d;
  }
  __syncthreads();

  // Threshold and tie quota from the bin totals: one block scan.
  int T = -1, quota = 0;
  if (keff > 0) {                                      // uniform
    uint32_t cnt = 0;
    if (t < BINS) {
#pragma unroll
      for (int w = 0; w < kScanThreads / 64; ++w) cnt += hist[w][t];
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan_dpp(cnt, scan_lds, tot);
    const bool hit = t < BINS && ex + cnt >= (uint32_t)keff;
    if (t < BINS) ex_lds[t] = ex;
    const uint64_t m = __ballot(hit);
    if (lane == 0) first_lds[wave] = m ? 64 * wave + (int)__builtin_ctzll(m) : BINS;
    __syncthreads();
    int first = BINS;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) first = min(first, first_lds[w]);
    // T = BINS when the histogrammed distances hold fewer than k_eff candidates (the
    // rest are at distance BINS, which the bins do not count)
    T = first;
    quota = keff - (int)(first < BINS ? ex_lds[first] : tot);
  }

  if (T >= 0) {
    uint32_t w[kTinyTpt / 4];
    const uint4 r = reinterpret_cast<const uint4 *>(dist)[t];
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
    RunSelect<kTinyTpt> rs;
    rs.build(w, T, quota, 0, 0, scan_lds);
    const int32_t tok0 = (int32_t)lo + kTinyTpt * t;
    int32_t *out = idx + (int64_t)bh * k;
    rs.emit(0, rs.total, [&](int pos, int off) {
      sel[pos] = tok0 + off;
      out[pos] = tok0 + off;
    });
  }
  if (t == 0) count[bh] = keff;
  __syncthreads();
  ga.run_block(kc, vc, head_row0, keff > 0 ? keff : 0, [&](int rr) { return sel[rr]; });
  ga.combine_store(o + row0 * kHeadDim, lse + row0);
}

}  // namespace

bool tiny_step_fits(int B, int Hq, int Hkv, int64_t C, int keff, int n_win) {
  return Hkv > 0 && Hq == Hkv && C <= kTinyC && (int64_t)keff + n_win <= kTinyList &&
         (int64_t)B * Hkv <= kTinyMaxHeads;
}

hipError_t launch_tiny_step(const hk_hash &h, const RetrievePlan &p, const void *q,
                            const uint32_t *codes, const void *kc, const void *vc, int B,
                            int Hq, int Hkv, int64_t cap, int k, float scale, int win_sinks,
                            int64_t win_local0, int n_win, uint32_t *qcodes, int32_t *idx,
                            int32_t *count, float *o, float *lse, hipStream_t st) {
  const int rows = B * Hkv;
  if (rows == 0) return hipSuccess;
  const enc::HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const float sl2 = scale * kLog2e;
  const bool bf = h.dtype == HK_BF16;
#define HK_TINY(WW, BF, KK)                                                                   \
  hipLaunchKernelGGL((tiny_step_kernel<WW, BF, KK>), dim3(rows), dim3(kScanThreads), 0, st,   \
                     codes, q, cap, p.lo, p.C, p.keff, k, hp, Hq, Hkv, kc, vc, sl2, win_sinks, \
                     win_local0, n_win, qcodes, idx, count, o, lse)
#define HK_TINY_K(WW, BF)                                                                     \
  if (h.kind == HK_HASH_MLP) HK_TINY(WW, BF, enc::kMlp);                                      \
  else if (h.kind == HK_HASH_LSH) HK_TINY(WW, BF, enc::kLsh);                                 \
  else HK_TINY(4, BF, enc::kSign);
  if (h.bits == 128) {
    if (bf) { HK_TINY_K(4, true) } else { HK_TINY_K(4, false) }
  } else {
    if (bf) { HK_TINY_K(2, true) } else { HK_TINY_K(2, false) }
  }
#undef HK_TINY_K
#undef HK_TINY
  return hipGetLastError();
}

}  // namespace hk
