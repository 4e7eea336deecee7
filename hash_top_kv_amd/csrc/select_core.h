// Device core of the top-k selection shared by the emit kernel and the fused
// retrieve-and-attend kernel.
#pragma once

#include "hk_internal.h"

namespace hk {

constexpr int kScanThreads = 256;

// Token order within a chunk: wavefront w owns tokens [w*64*LPT, (w+1)*64*LPT), and its
// item i covers tokens w*64*LPT + 64*i + lane, so every load instruction of a wavefront
// reads 64 consecutive codes.  A thread's distances are stored four to a 32-bit word:
// word (i/4)*256 + t of the chunk holds items i..i+3 of thread t (one coalesced dword
// store per four tokens).
template <int LPT>
__device__ __forceinline__ int64_t stash_words_per_chunk() { return (int64_t)LPT / 4 * kScanThreads; }

// Number of tokens a chunk contributes to the selection: all of its tokens below the
// threshold and the ties that fall inside the quota.
__device__ __forceinline__ int chunk_selected(const int4 &mt, int quota) {
  const int ties = quota - mt.y;
  return mt.z + (ties <= 0 ? 0 : (ties < mt.w ? ties : mt.w));
}

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Writes the selected tokens of nch consecutive chunks (nch uniform, at most MAXC):
// word(i, k) is this thread's k-th stash word of chunk i, meta(i) the chunk's counts below
// / at T before it and its own, and chunk i starts at token tok0 + i*CH.  sink(position
// in the head's list, token) is called for every selected token.  Called by all threads
// of the workgroup.
//
// The tie quota splits at most one chunk of a head.  Every other chunk takes exactly its
// tokens with D < T (the quota is used up before it) or with D <= T (its ties all fit),
// so one ballot per item decides, and a token's position is the chunk's first position
// plus the selected count in earlier wavefronts of the chunk (one exchange through LDS),
// in the wavefront's earlier items (a running count) and in lower lanes (mbcnt).  The
// chunk holding the quota boundary ranks ties and non-ties separately.
template <int LPT, int MAXC, class Word, class Meta, class Sink>
__device__ __forceinline__ void emit_chunks(Word word, Meta meta, int nch, int T, int quota,
                                            int64_t tok0, Sink sink) {
  constexpr int NW = kScanThreads / 64;
  constexpr int CH = kScanThreads * LPT;
  __shared__ uint32_t wcnt[2][MAXC][NW];      // per (chunk, wavefront) counts
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  // mode of a chunk: 0 = D < T, 1 = D <= T, 2 = split by the quota
  auto mode_of = [&](const int4 &mt) {
    return mt.y >= quota ? 0 : (mt.y + mt.w <= quota ? 1 : 2);
  };
#pragma unroll 1
  for (int i = 0; i < nch; ++i) {
    const int mode = mode_of(meta(i));
    uint32_t wv[LPT / 4];
#pragma unroll
    for (int k = 0; k < LPT / 4; ++k) wv[k] = word(i, k);
    uint32_t n0 = 0, n1 = 0;
    if (mode < 2) {
      const int lim = T + mode;               // selected: D < lim
#pragma unroll
      for (int j = 0; j < LPT; ++j)
        n0 += (uint32_t)__popcll(__ballot((int)((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu) < lim));
    } else {
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int d = (int)((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu);
        n0 += (uint32_t)__popcll(__ballot(d < T));
        n1 += (uint32_t)__popcll(__ballot(d == T));
      }
    }
    if (lane == 0) {
      wcnt[0][i][wave] = n0;
      wcnt[1][i][wave] = n1;
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < nch; ++i) {
    const int4 mt = meta(i);
    const int mode = mode_of(mt);
    uint32_t wv[LPT / 4];
#pragma unroll
    for (int k = 0; k < LPT / 4; ++k) wv[k] = word(i, k);
    const int64_t tw = tok0 + (int64_t)i * CH + (int64_t)wave * (64 * LPT) + lane;
    if (mode < 2) {
      const int lim = T + mode;
      int run = mt.x + min(mt.y, quota);      // first position of the chunk
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2)
        if (w2 < wave) run += (int)wcnt[0][i][w2];
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const bool take = (int)((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu) < lim;
        const uint64_t m = __ballot(take);
        if (m) {
          if (take) sink(run + lanes_below(m), (int32_t)(tw + 64 * j));
          run += __popcll(m);
        }
      }
    } else {
      int run_lt = mt.x, run_eq = mt.y;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        if (w2 < wave) {
          run_lt += (int)wcnt[0][i][w2];
          run_eq += (int)wcnt[1][i][w2];
        }
      }
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int d = (int)((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu);
        const uint64_t blt = __ballot(d < T), beq = __ballot(d == T);
        if (blt | beq) {
          if (d <= T) {
            const int lt_rank = run_lt + lanes_below(blt);
            const int eq_rank = run_eq + lanes_below(beq);
            int pos = -1;
            if (d < T) pos = lt_rank + min(eq_rank, quota);
            else if (eq_rank < quota) pos = lt_rank + eq_rank;
            if (pos >= 0) sink(pos, (int32_t)(tw + 64 * j));
          }
          run_lt += __popcll(blt);
          run_eq += __popcll(beq);
        }
      }
    }
  }
}

}  // namespace hk
