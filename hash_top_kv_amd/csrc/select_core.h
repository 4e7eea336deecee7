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

// Threads of a workgroup that computes a head threshold.
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

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts within rows of 16 lanes,
// then the row totals broadcast to the following rows (DPP row_shr, row_bcast:15/31).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The threshold of one head, computed by one workgroup of kThrThreads threads, one thread
// per chunk (tiles of kThrThreads chunks).  A two-level radix select over the chunk
// histograms hb[S][BINS + BINS/8]:
//   1. superbin totals over all chunks -> the superbin holding T (or T = BINS when the
//      histogrammed distances hold fewer than k_eff candidates);
//   2. that superbin's 8 bins, totalled over the chunks -> T and the tie quota;
//   3. per chunk, #(D < T) (its superbins below T's plus its bins of T's superbin below
//      T) and #(D == T), then an exclusive prefix of both over chunks: sink(c, meta) is
//      called by the thread of chunk c with meta = (below T before c, at T before c,
//      below T in c, at T in c).
// T = -1 when k_eff = 0.  Every thread returns T and the tie quota.  For up to
// kThrThreads chunks per head every value is read once and kept in registers.
//
// Each level is one exchange through LDS: the wavefronts' partial totals go to LDS, and
// after one barrier every wavefront adds them up itself and finds the bin that reaches
// k_eff with an inclusive scan over its lanes and a ballot (the same answer in every
// wavefront), so no thread walks the totals serially and no result is broadcast.
template <int BINS, class Sink>
__device__ __forceinline__ void head_threshold(const uint32_t *__restrict__ hb, int S, int64_t C,
                                               int CH, int keff, int &T_out, int &quota_out,
                                               Sink sink) {
  constexpr int NSB = BINS / 8;                // 16 or 8 superbins
  constexpr int ROW = BINS + NSB;
  constexpr int NT = kThrThreads;
  constexpr int NW = NT / 64;
  __shared__ uint32_t red1[NW][16];            // per-wavefront superbin totals
  __shared__ uint32_t red2[NW][8];             // per-wavefront bin totals of T's superbin
  __shared__ uint2 part[2][NW];                // per-wavefront (below, at) totals, per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  auto row = [&](int c) { return hb + (int64_t)(c < S ? c : S - 1) * ROW; };

  uint32_t sb0[NSB], bb0[8];                   // the first tile's values, kept
  int T = -1, quota = 0;
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
    const uint32_t r1 = wave_transpose_sum<NSB>(acc);
    if (lane < NSB) red1[wave][bitrev_k<NSB>(lane)] = r1;
    __syncthreads();
    uint32_t tot = 0;
    if (lane < NSB) {
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += red1[w][lane];
    }
    const uint32_t inc = wave_incl_scan_dpp(tot);                 // lanes >= NSB add 0
    const uint64_t reach = __ballot(lane < NSB && inc >= (uint32_t)keff);
    const int Ts = reach ? (int)__builtin_ctzll(reach) : NSB;
    const uint32_t below = Ts == 0 ? 0u : (uint32_t)__shfl((int)inc, Ts - 1, 64);
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
      const uint32_t r2 = wave_transpose_sum<8>(bacc);
      if (lane < 8) red2[wave][bitrev_k<8>(lane)] = r2;
      __syncthreads();
      uint32_t bt = 0;
      if (lane < 8) {
#pragma unroll
        for (int w = 0; w < NW; ++w) bt += red2[w][lane];
      }
      const uint32_t binc = wave_incl_scan_dpp(bt) + below;
      // the superbin holds the k_eff-th distance, so one of its 8 bins reaches k_eff
      const uint64_t reach2 = __ballot(lane < 8 && binc >= (uint32_t)keff);
      const int b = (int)__builtin_ctzll(reach2);
      const uint32_t bbelow = b == 0 ? below : (uint32_t)__shfl((int)binc, b - 1, 64);
      T = 8 * Ts + b;
      quota = keff - (int)bbelow;
    } else {
      T = BINS;
      quota = keff - (int)below;
    }
  }
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
    // Exclusive prefix over the tile's chunks: scans within each wavefront, then the
    // wavefront totals through LDS (double-buffered across tiles, one barrier per tile).
    const uint32_t lt_inc = wave_incl_scan_dpp(lt), eq_inc = wave_incl_scan_dpp(eq);
    uint2 *pt = part[(c0 / NT) & 1];
    if (lane == 63) pt[wave] = make_uint2(lt_inc, eq_inc);
    __syncthreads();
    uint32_t off_lt = 0, off_eq = 0, tl = 0, te = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint2 x = pt[w];
      off_lt += (w < wave) ? x.x : 0u;
      off_eq += (w < wave) ? x.y : 0u;
      tl += x.x;
      te += x.y;
    }
    if (c < S)
      sink(c, make_int4((int)(carry_lt + off_lt + lt_inc - lt),
                        (int)(carry_eq + off_eq + eq_inc - eq), (int)lt, (int)eq));
    carry_lt += tl;
    carry_eq += te;
  }
  T_out = T;
  quota_out = quota;
}

// Words of chunk histograms a workgroup can hold in LDS (the selection list's space,
// which is unused while the threshold is derived).
constexpr int kHistLdsWords = 4096;

// head_threshold for a head whose chunk histograms fit in LDS: hl[S][BINS] holds the bin
// counts of its S chunks (S * BINS <= kHistLdsWords), copied there by the caller in one
// round trip together with its other loads, so that no step waits on memory.  Gives the
// same T, tie quota and sink calls as head_threshold (kThrThreads threads):
//   1. bin totals over the chunks (wavefront w adds chunks w, w + 4, ...), exchanged
//      through LDS; every wavefront then scans the totals and takes the first bin whose
//      inclusive count reaches k_eff (T = BINS when none does);
//   2. per chunk, #(D < T) and #(D == T) from TPC threads that each add BPT bins, and the
//      exclusive prefix of both over the chunks.
template <int BINS, class Sink>
__device__ __forceinline__ void head_threshold_lds(const uint32_t *hl, int S, int64_t C, int CH,
                                                   int keff, int &T_out, int &quota_out,
                                                   Sink sink) {
  constexpr int NT = kThrThreads, NW = NT / 64;
  constexpr int NJ = BINS / 64;                // 64-bin blocks: one per lane each
  constexpr int SMAX = kHistLdsWords / BINS;   // 32 or 64 chunks
  constexpr int TPC = NT / SMAX;               // threads per chunk: 8 or 4
  constexpr int BPT = BINS / TPC;              // bins per thread: 16
  static_assert(NT % SMAX == 0 && BINS % TPC == 0 && (BPT & (BPT - 1)) == 0, "layout");
  __shared__ uint32_t red[NW][BINS];
  __shared__ uint2 part[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int T = -1, quota = 0;
  if (keff > 0) {
    uint32_t p[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) p[j] = 0u;
    for (int c = wave; c < S; c += NW)
#pragma unroll
      for (int j = 0; j < NJ; ++j) p[j] += hl[c * BINS + 64 * j + lane];
#pragma unroll
    for (int j = 0; j < NJ; ++j) red[wave][64 * j + lane] = p[j];
    __syncthreads();
    uint32_t run = 0, below = 0;               // run: count of the bins before block j
    int found = -1;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint32_t tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += red[w][64 * j + lane];
      const uint32_t inc = wave_incl_scan_dpp(tot) + run;
      const uint64_t reach = __ballot(inc >= (uint32_t)keff);
      if (found < 0 && reach) {
        const int b = (int)__builtin_ctzll(reach);
        found = 64 * j + b;
        below = b == 0 ? run : (uint32_t)__shfl((int)inc, b - 1, 64);
      }
      run = (uint32_t)__shfl((int)inc, 63, 64);
    }
    T = found < 0 ? BINS : found;
    quota = keff - (int)(found < 0 ? run : below);
  }
  if (T >= 0) {
    const int c = tid / TPC, pp = tid - c * TPC;
    uint32_t lt = 0, eq = 0;
    if (c < S) {
      const uint32_t *hc = hl + c * BINS + pp * BPT;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        const int ii = (i + c) & (BPT - 1);    // rotated by chunk: fewer LDS bank conflicts
        const int b = pp * BPT + ii;
        const uint32_t v = hc[ii];
        lt += b < T ? v : 0u;
        eq += b == T ? v : 0u;
      }
    }
#pragma unroll
    for (int o = 1; o < TPC; o <<= 1) {
      lt += (uint32_t)__shfl_xor((int)lt, o, 64);
      eq += (uint32_t)__shfl_xor((int)eq, o, 64);
    }
    if (T == BINS && c < S) {                  // distance BINS is not in the histogram
      const int64_t n = C - (int64_t)c * CH;
      eq = (uint32_t)(n < CH ? n : CH) - lt;
    }
    const bool lead = pp == 0 && c < S;
    const uint32_t lt_inc = wave_incl_scan_dpp(lead ? lt : 0u);
    const uint32_t eq_inc = wave_incl_scan_dpp(lead ? eq : 0u);
    if (lane == 63) part[wave] = make_uint2(lt_inc, eq_inc);
    __syncthreads();
    uint32_t off_lt = 0, off_eq = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint2 x = part[w];
      off_lt += (w < wave) ? x.x : 0u;
      off_eq += (w < wave) ? x.y : 0u;
    }
    if (lead)
      sink(c, make_int4((int)(off_lt + lt_inc - lt), (int)(off_eq + eq_inc - eq), (int)lt, (int)eq));
  }
  T_out = T;
  quota_out = quota;
}

// Writes the selected tokens of nch consecutive chunks (nch uniform, at most MAXC) into
// list[position - first], where first is the head-list position of the first chunk's
// first selected token.  The chunks' distance stashes are in LDS (sw[chunk][word][thread]
// as written by the scan), their counts in smt[chunk]; chunk i starts at token
// tok0 + i*CH.  Called by all threads of the workgroup; ends with the list complete.
//
// Thread t takes the LPT consecutive tokens LPT*t .. LPT*t + LPT-1 of every chunk, so
// tokens ascend with (chunk, thread, bit).  It reads their distances from the stash
// (they were stashed by LPT different scan threads), and keeps two bit masks per chunk:
// tokens below the threshold and tokens at it.  One block-wide exclusive scan of the
// packed per-thread counts (below | at << 16) gives every thread the number of tokens
// below / at the threshold before its own in the head; a token below the threshold goes
// to position (below before) + min(at before, quota), a tie with (at before) < quota to
// (below before) + (at before).  Each thread then visits only its set mask bits.
template <int LPT, int MAXC>
__device__ __forceinline__ void emit_chunks_lanes(const uint32_t (*sw)[LPT / 4][kScanThreads],
                                                  const int4 *smt, int nch, int T, int quota,
                                                  int64_t tok0, int first, int32_t *list) {
  constexpr int NW = kScanThreads / 64;
  constexpr int CH = kScanThreads * LPT;
  constexpr int TPR = 64 / LPT;                // threads per 64-token row of a wavefront
  __shared__ uint32_t wtot[NW][MAXC];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  // Scan thread of this thread's first token, and the item (byte) that holds it.
  const int s0 = (t & ~63) + LPT * (t % TPR);
  const int item = (t / TPR) % LPT;
  const int sh = 8 * (item & 3);
  // All MAXC chunks of sw are read (unused ones hold a copy of a used chunk) so that the
  // reads issue together; the masks of unused chunks are cleared.
  uint4 wr[MAXC][LPT / 4];
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int q4 = 0; q4 < LPT / 4; ++q4)
      wr[i][q4] = *reinterpret_cast<const uint4 *>(&sw[i][item >> 2][s0 + 4 * q4]);
  uint32_t masks[MAXC], cnt[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    uint32_t mlt = 0, meq = 0;
#pragma unroll
    for (int q4 = 0; q4 < LPT / 4; ++q4) {
      const uint32_t wv[4] = {wr[i][q4].x, wr[i][q4].y, wr[i][q4].z, wr[i][q4].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = (int)((wv[e] >> sh) & 0xFFu);
        mlt |= (d < T ? 1u : 0u) << (4 * q4 + e);
        meq |= (d == T ? 1u : 0u) << (4 * q4 + e);
      }
    }
    const uint32_t live = i < nch ? 0xFFFFFFFFu : 0u;
    mlt &= live;
    meq &= live;
    masks[i] = mlt | (meq << 16);
    cnt[i] = (uint32_t)__popc(mlt) | ((uint32_t)__popc(meq) << 16);
  }
  // Block-wide exclusive scan of the packed counts (each half stays below 2^16).
  uint32_t inc[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) inc[i] = wave_incl_scan_dpp(cnt[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) wtot[wave][i] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (i >= nch) break;
    uint32_t before = inc[i] - cnt[i];
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) before += wtot[w][i];
    const int4 mt = smt[i];
    const int lt0 = mt.x + (int)(before & 0xFFFFu);
    const int eq0 = mt.y + (int)(before >> 16);
    const uint32_t mlt = masks[i] & 0xFFFFu, meq = masks[i] >> 16;
    uint32_t all = mlt | meq;
    const int32_t tokb = (int32_t)(tok0 + (int64_t)i * CH) + LPT * t;
    while (all) {
      const int j = __builtin_ctz(all);
      all &= all - 1;
      const uint32_t below = (1u << j) - 1u;
      const int ltb = lt0 + __popc(mlt & below);
      const int eqb = eq0 + __popc(meq & below);
      int pos = -1;
      if ((mlt >> j) & 1u) pos = ltb + min(eqb, quota);
      else if (eqb < quota) pos = ltb + eqb;
      if (pos >= 0) list[pos - first] = tokb + j;
    }
  }
  __syncthreads();
}

}  // namespace hk
