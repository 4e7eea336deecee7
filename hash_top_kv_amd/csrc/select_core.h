// Device core of the top-k selection shared by the emit kernel and the fused
// retrieve-and-attend kernel.
#pragma once

#include "hk_internal.h"

namespace hk {

constexpr int kScanThreads = 256;

// Token order within a chunk: wavefront w owns tokens [w*64*LPT, (w+1)*64*LPT), and its
// item i covers tokens w*64*LPT + 64*i + lane, so every load instruction of a wavefront
// reads 64 consecutive codes.  The distances are stored in token order: byte p of a
// head's distance bytes is candidate p's distance (255 past the last candidate, never
// selected), so each item is one coalesced 64-byte store per wavefront and a reader finds
// any run of consecutive tokens in consecutive bytes.

// Bits 8, 9, 24, 25 of the result flag the bytes 0, 1, 2, 3 of w (four consecutive tokens)
// whose value is >= t, for 0 <= t <= 256 given as tt = t | t << 16.  Each byte x sits in a
// 16-bit field as 0x100 | x, from which t is subtracted: bit 8 of the field survives exactly
// when x >= t, and no borrow leaves the field (0x100 + x - t >= 0).
constexpr uint32_t kByteFlags = 0x03000300u;
__device__ __forceinline__ uint32_t bytes_ge(uint32_t w, uint32_t tt) {
  const uint32_t ev = (w & 0x00FF00FFu) | 0x01000100u;
  const uint32_t od = ((w >> 8) & 0x00FF00FFu) | 0x01000100u;
  return ((ev - tt) & 0x01000100u) | (((od - tt) & 0x01000100u) << 1);
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

// Exclusive prefix over the 256 threads of a workgroup: DPP scans within the wavefronts,
// the wavefront totals through lds[4].  Returns the prefix and sets total.  Called by all
// threads; lds may be reused after the caller's next barrier.
__device__ __forceinline__ uint32_t block_excl_scan_dpp(uint32_t v, uint32_t *lds,
                                                        uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan_dpp(v);
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const uint32_t x = lds[w];
    off += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  return off + inc - v;
}

// Flags at bit 7 of each byte of w (four consecutive tokens) for the bytes >= t, for
// 0 <= t <= 127 given as t4 = t * 0x01010101: a byte of 128 or more (distance 128 of
// 128-bit codes, 255 past the last candidate) carries bit 7 itself, and for the others
// (x | 0x80) - t keeps bit 7 exactly when x >= t, with no borrow out of the byte.
constexpr uint32_t kByteHigh = 0x80808080u;
__device__ __forceinline__ uint32_t bytes_ge7(uint32_t w, uint32_t t4) {
  return (((w | kByteHigh) - t4) | w) & kByteHigh;
}
// The flags (bit 7 of each byte) of two words as 8 bits in token order: byte b of fa at
// bit b, byte b of fb at bit 4 + b.  x holds fa's flags at bits 0, 8, 16, 24 and fb's at
// 4, 12, 20, 28; the multiply by 2^21 + 2^14 + 2^7 + 1 adds four shifted copies of x whose
// bits differ mod 4, so no two bits meet (no carries), and bits 21 .. 28 of the product
// are the eight flags in order.
__device__ __forceinline__ uint32_t high_pair_to_byte(uint32_t fa, uint32_t fb) {
  return (((fa >> 7) | (fb >> 3)) * 0x00204081u >> 21) & 0xFFu;
}
// Bits 8, 9, 24, 25 (the flags of bytes_ge) moved to bits 0..3.
__device__ __forceinline__ uint32_t spread_to_nibble(uint32_t f) {
  return ((f >> 8) & 3u) | ((f >> 22) & 0xCu);
}
// The lowest n set bits of m (all of them when n >= popcount(m)).
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, int n) {
  if (n <= 0) return 0u;
  uint32_t rest = m;
  for (int i = 0; i < n && rest; ++i) rest &= rest - 1u;
  return m & ~rest;
}

// The selected tokens of a run of a head's candidates, with TPT consecutive tokens per
// thread of a 256-thread workgroup (TPT a multiple of 4, at most 64).  Selected are the
// tokens with D < T and the first `quota` tokens of the head with D == T in token order.
//   build(): from this thread's distance bytes w (bytes past the run set to 255) and the
//     head's counts below and at T before the run: one block-wide scan of the packed
//     counts below / at T gives the counts before this thread's first token, hence its
//     share of the tie quota; then this thread's mask of selected tokens (bit j = token j)
//     and the number of the head's selected tokens before its first one;
//   emit(): sink(position - first, token offset in the thread's run) for every selected
//     token whose list position p - first lies in [lo, hi), visiting only the set bits.
// The top-k list is written in token order, so a selected token's position is the number
// of selected tokens before it: (below before) + min(at before, quota) for the thread,
// plus its rank among the thread's own.
template <int TPT>
struct RunSelect {
  static_assert(TPT % 4 == 0 && TPT <= 64, "4 .. 64 tokens per thread");
  static constexpr int NWD = TPT / 4;
  static constexpr int NH = (TPT + 31) / 32;   // 32-bit mask words
  uint32_t sel[NH];
  int selb, total, first;

  __device__ void build(const uint32_t (&w)[NWD], int T, int quota, int lt_before, int eq_before,
                        uint32_t *lds) {
    uint32_t lt[NH], eq[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) lt[h] = eq[h] = 0u;
    if (T <= 126) {                            // uniform
      const uint32_t t0 = (uint32_t)T * 0x01010101u, t1 = t0 + 0x01010101u;
      uint32_t fl[NWD], fe[NWD];
#pragma unroll
      for (int k = 0; k < NWD; ++k) {
        const uint32_t ge0 = bytes_ge7(w[k], t0), ge1 = bytes_ge7(w[k], t1);
        fl[k] = ~ge0 & kByteHigh;
        fe[k] = ge0 & ~ge1;
      }
#pragma unroll
      for (int k = 0; k < NWD; k += 2) {
        const uint32_t bl = high_pair_to_byte(fl[k], k + 1 < NWD ? fl[k + 1] : 0u);
        const uint32_t be = high_pair_to_byte(fe[k], k + 1 < NWD ? fe[k + 1] : 0u);
        lt[k / 8] |= bl << (4 * (k % 8));
        eq[k / 8] |= be << (4 * (k % 8));
      }
    } else {
      const uint32_t t0 = (uint32_t)T | ((uint32_t)T << 16), t1 = t0 + 0x00010001u;
#pragma unroll
      for (int k = 0; k < NWD; ++k) {
        const uint32_t ge0 = bytes_ge(w[k], t0), ge1 = bytes_ge(w[k], t1);
        lt[k / 8] |= spread_to_nibble(~ge0 & kByteFlags) << (4 * (k % 8));
        eq[k / 8] |= spread_to_nibble(ge0 & ~ge1) << (4 * (k % 8));
      }
    }
    uint32_t n = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) n += (uint32_t)__popc(lt[h]) | ((uint32_t)__popc(eq[h]) << 16);
    uint32_t tot;
    const uint32_t before = block_excl_scan_dpp(n, lds, tot);
    const int ltb = lt_before + (int)(before & 0xFFFFu);
    const int eqb = eq_before + (int)(before >> 16);
    // this thread's ties within the quota: the first quota - eqb of them
    int take = quota - eqb;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int c = __popc(eq[h]);
      sel[h] = lt[h] | (take >= c ? eq[h] : lowest_bits(eq[h], take));
      take -= c;
    }
    const int tl = (int)(tot & 0xFFFFu), te = (int)(tot >> 16);
    const int ties = quota - eq_before;
    total = tl + (ties <= 0 ? 0 : (ties < te ? ties : te));
    first = lt_before + min(eq_before, quota);
    selb = ltb + min(eqb, quota) - first;      // run position of this thread's first selected
  }

  template <class Sink>
  __device__ void emit(int lo, int hi, Sink sink) const {
    int r = selb;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      uint32_t m = sel[h];
      while (m) {
        const int bb = __builtin_ctz(m);
        const int pos = r + __popc(sel[h] & ((1u << bb) - 1u));
        m &= m - 1u;
        if (pos >= lo && pos < hi) sink(pos, 32 * h + bb);
      }
      r += __popc(sel[h]);
    }
  }
};

// Loads the TPT distance bytes of tokens [p, p + TPT) from a head's distance bytes d (16-
// byte aligned runs), or 255s when ok is false.
template <int TPT>
__device__ __forceinline__ void load_run(const uint8_t *d, int64_t p, bool ok,
                                         uint32_t (&w)[TPT / 4]) {
  if constexpr (TPT % 16 == 0) {
#pragma unroll
    for (int i = 0; i < TPT / 16; ++i) {
      const uint4 v = ok ? reinterpret_cast<const uint4 *>(d + p)[i]
                         : make_uint4(~0u, ~0u, ~0u, ~0u);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (TPT == 8) {
    const uint2 v = ok ? *reinterpret_cast<const uint2 *>(d + p) : make_uint2(~0u, ~0u);
    w[0] = v.x; w[1] = v.y;
  } else {
    static_assert(TPT == 4, "4, 8 or a multiple of 16 tokens per thread");
    w[0] = ok ? *reinterpret_cast<const uint32_t *>(d + p) : ~0u;
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

// The threshold of one head together with the counts of the head's tokens below / at it
// before the first chunk of each of NG groups, by one workgroup of kThrThreads threads
// (one thread per chunk, tiles of kThrThreads chunks) from the chunk histograms
// hb[S][BINS + BINS/8].  Level 1 is head_threshold's: the superbin totals give the
// superbin Ts holding T.  Level 2 reads that superbin's 8 bins of every chunk once and
// reduces, in one exchange, both the 8 bin totals (which give T and the tie quota) and,
// for every group g, the sums over the chunks c < gs[g] of (c's superbins below Ts) and of
// its 8 bins; the counts below / at T before the group follow from prefix sums over
// those totals, whatever bin of Ts holds T.  T = -1 when k_eff = 0 (the counts are then
// left unset); T = BINS when the histogrammed distances hold fewer than k_eff candidates
// (distance BINS is not in the histogram: its count is the chunk size minus the others).
// Every thread returns the same T, quota and counts.
template <int BINS, int NG>
__device__ __forceinline__ void head_threshold_groups(const uint32_t *__restrict__ hb, int S,
                                                      int CH, int keff, const int (&gs)[NG],
                                                      int &T_out, int &quota_out,
                                                      int (&lt_before)[NG], int (&eq_before)[NG]) {
  constexpr int NSB = BINS / 8;
  constexpr int ROW = BINS + NSB;
  constexpr int NT = kThrThreads;
  constexpr int NW = NT / 64;
  constexpr int NV = 8 + 9 * NG;               // reduced values of level 2
  constexpr int K = NV <= 16 ? 16 : 32;
  static_assert(NV <= 32, "at most 2 groups");
  __shared__ uint32_t red1[NW][16];
  __shared__ uint32_t red2[NW][K];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  auto row = [&](int c) { return hb + (int64_t)(c < S ? c : S - 1) * ROW; };
  int T = -1, quota = 0;
  if (keff > 0) {
    // level 1: superbin totals
    uint32_t sb0[NSB], acc[NSB];
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
    // level 2: T's superbin, and the sums before every group
    uint32_t a[K];
#pragma unroll
    for (int v = 0; v < K; ++v) a[v] = 0u;
    for (int c0 = 0; c0 < S; c0 += NT) {
      const int c = c0 + tid;
      uint32_t sbv[NSB], bb[8];
      if (c0 == 0) {
#pragma unroll
        for (int i = 0; i < NSB; ++i) sbv[i] = sb0[i];
      } else {
        load_u32x<NSB>(row(c) + BINS, sbv);
      }
      if (Ts < NSB) {
        load_u32x<8>(row(c) + 8 * Ts, bb);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) bb[j] = 0u;
      }
      const bool ok = c < S;
      uint32_t sbelow = 0;
#pragma unroll
      for (int i = 0; i < NSB; ++i) sbelow += i < Ts ? sbv[i] : 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] += ok ? bb[j] : 0u;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const bool m = ok && c < gs[g];
        a[8 + 9 * g] += m ? sbelow : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) a[9 + 9 * g + j] += m ? bb[j] : 0u;
      }
    }
    const uint32_t r2 = wave_transpose_sum<K>(a);
    if (lane < K) red2[wave][bitrev_k<K>(lane)] = r2;
    __syncthreads();
    uint32_t t2 = 0;
    if (lane < NV) {
#pragma unroll
      for (int w = 0; w < NW; ++w) t2 += red2[w][lane];
    }
    // inclusive prefix over the NV values: bins of Ts in lanes 0..7, then per group its
    // below-superbin sum and its 8 bins
    const uint32_t p2 = wave_incl_scan_dpp(t2);
    auto pre = [&](int l) { return l < 0 ? 0u : (uint32_t)__shfl((int)p2, l, 64); };
    int b = 0;
    if (Ts < NSB) {
      const uint64_t reach2 = __ballot(lane < 8 && p2 + below >= (uint32_t)keff);
      b = (int)__builtin_ctzll(reach2);        // the superbin holds the k_eff-th distance
      T = 8 * Ts + b;
      quota = keff - (int)(below + pre(b - 1));
    } else {
      T = BINS;
      quota = keff - (int)below;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int a0 = 8 + 9 * g;                // the group's below-superbin sum
      if (Ts < NSB) {
        lt_before[g] = (int)(pre(a0 + b) - pre(a0 - 1));
        eq_before[g] = (int)(pre(a0 + 1 + b) - pre(a0 + b));
      } else {
        lt_before[g] = (int)(pre(a0) - pre(a0 - 1));   // every histogrammed distance is below T
        eq_before[g] = gs[g] * CH - lt_before[g];      // chunks before a group are whole
      }
    }
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

}  // namespace hk
