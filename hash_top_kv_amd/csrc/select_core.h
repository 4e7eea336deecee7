// Device core of the top-k selection shared by the emit kernel and the fused
// retrieve-and-attend kernel.
#pragma once

#include "hk_internal.h"

namespace hk {

constexpr int kScanThreads = 256;

// Token p of a chunk is handled by thread p % 256 as its item p / 256, so every load
// instruction of a wavefront reads one contiguous run of codes.  A thread's distances
// are stored four to a 32-bit word: word (i/4)*256 + t of the chunk holds items
// i..i+3 of thread t (one dword store per four tokens, coalesced).
template <int LPT>
__device__ __forceinline__ int64_t stash_words_per_chunk() { return (int64_t)LPT / 4 * kScanThreads; }

// Number of tokens a chunk contributes to the selection: all of its tokens below the
// threshold and the ties that fall inside the quota.
__device__ __forceinline__ int chunk_selected(const int4 &mt, int quota) {
  const int ties = quota - mt.y;
  return mt.z + (ties <= 0 ? 0 : (ties < mt.w ? ties : mt.w));
}

// Compacts the selected tokens of one chunk in token order (item-major, then thread)
// with wavefront ballots: the rank of token (i, t) among the chunk's selected tokens is
// the count over items i' < i, plus earlier wavefronts of item i, plus earlier lanes of
// its own wavefront.  For each selected token, sink(position in the head's list,
// position in the chunk's list, token) is called.  `w` holds the thread's stash words;
// T >= 0.  Called by all threads of the workgroup.
template <int LPT, class Sink>
__device__ __forceinline__ void emit_chunk(const uint32_t *w, int T, int quota, int lt_before,
                                           int eq_before, int64_t tok0, Sink sink) {
  constexpr int NW = kScanThreads / 64;
  __shared__ uint32_t cnt[2][LPT * NW];     // per (item, wave): #below T, #at T
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const uint64_t below_me = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int d = (w[i >> 2] >> (8 * (i & 3))) & 0xFF;
    const uint64_t blt = __ballot(d < T), beq = __ballot(d == T);
    if (lane == 0) {
      cnt[0][i * NW + wave] = (uint32_t)__popcll(blt);
      cnt[1][i * NW + wave] = (uint32_t)__popcll(beq);
    }
  }
  __syncthreads();
  // Exclusive scan of the (item, wave) counts, LPT*NW <= 64 entries, by wavefront 0.
  if (wave == 0) {
    const bool in = lane < LPT * NW;
    const uint32_t a = in ? cnt[0][lane] : 0u, b = in ? cnt[1][lane] : 0u;
    const uint32_t ia = wave_incl_scan_u32(a), ib = wave_incl_scan_u32(b);
    if (in) {
      cnt[0][lane] = ia - a;
      cnt[1][lane] = ib - b;
    }
  }
  __syncthreads();
  const int first = lt_before + (eq_before < quota ? eq_before : quota);
  // The ballots are taken again rather than kept from the counting pass: 2*LPT wave masks
  // held across the barriers would cost as many scalar or vector register pairs.
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int d = (w[i >> 2] >> (8 * (i & 3))) & 0xFF;
    const uint64_t blt = __ballot(d < T), beq = __ballot(d == T);
    if (d > T) continue;
    const int lt_rank = lt_before + (int)cnt[0][i * NW + wave] + __popcll(blt & below_me);
    const int eq_rank = eq_before + (int)cnt[1][i * NW + wave] + __popcll(beq & below_me);
    const int32_t tok = (int32_t)(tok0 + i * kScanThreads + t);
    int pos = -1;
    if (d < T) pos = lt_rank + min(eq_rank, quota);
    else if (eq_rank < quota) pos = lt_rank + eq_rank;
    if (pos >= 0) sink(pos, pos - first, tok);
  }
}

}  // namespace hk
