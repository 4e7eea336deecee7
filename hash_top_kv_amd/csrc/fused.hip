// Fused top-k select + exact attention over the selected tokens, for one decode step.
//
// After the Hamming scan, each chunk workgroup derives its head's distance threshold
// from the chunk histograms, compacts its selected tokens (writing them to the head's
// ascending index list, as hk_topk_select does, and to LDS), gathers their K/V rows and
// computes the partial attention of the G query heads of its KV head over them.  Window
// workgroups do the same over slices of the static sink + local window.  The partials of
// a head -- disjoint token sets -- are then merged by log-sum-exp rescaling
// (RetrievalAttention, atlas summary: Approach), which gives attention over the selected
// tokens and the window together.
//
// Compared with threshold -> emit -> sparse decode -> merge, this saves two kernels and
// their dependent memory round trips (the threshold's outputs, the index list) on the
// decode step's critical path.
#include "attend_core.h"
#include "select_core.h"

namespace hk {
namespace {

// An argument used where the attention needs it: the empty asm keeps the compiler from
// hoisting its first use (and so the wait for its scalar load) into the kernel's entry.
template <class T>
__device__ __forceinline__ T at_use(T v) {
  asm volatile("" : "+s"(v));
  return v;
}

// grid (Sc + Sw, B*Hkv), after the Hamming scan.  Block c < Sc covers chunk group c (and
// c + Sc when REPS = 2) of the head, a group being chunks [g*CPB, (g+1)*CPB); blocks
// c >= Sc cover window slice c - Sc.  Block c writes the normalised partial of part c.
// A chunk block compacts its chunks' selected tokens into an LDS list (and into the
// head's index list) and attends over the list; when a list would overflow LDS it is
// attended and emptied first, so any selection size works.
constexpr int kListMax = 4096;
constexpr int kMaxCpb = 8;                 // chunks per workgroup, bounded by registers
// Workgroups resident at once at this kernel's register use (3 per CU).  Beyond that,
// fewer and longer workgroups amortise each one's serial phases (stash read,
// compaction, first gather, combine) over more rows.
constexpr int64_t kResidentBlocks = 768;

// The parameters that the first memory requests need come first (16 dwords, preloaded
// into SGPRs at launch), so the distance bytes and histograms are requested without
// waiting for a scalar load of the arguments.
template <int LPT, bool BF16, int G, int MAXC, int REPS>
__device__ __forceinline__ void emit_attend_body(
    const uint8_t *__restrict__ stash, const uint32_t *__restrict__ hist,
    const int32_t *__restrict__ ctx_len, int keff, int bins, int S, int CPB, int Sc, int Hkv,
    int64_t C, int64_t lo, int32_t *__restrict__ count, int k, int32_t *__restrict__ idx,
    const void *__restrict__ q, const void *__restrict__ kc, const void *__restrict__ vc,
    int Hq, int64_t cap, float scale_log2, int win_sinks, int64_t win_local0, int n_win,
    int win_rows, float *__restrict__ part_o, float *__restrict__ part_lse, int64_t rows,
    int64_t n_local, int64_t max_ctx) {
  constexpr int CH = kScanThreads * LPT;
  static_assert(kHistLdsWords <= kListMax, "the chunk histograms are staged in the list");
  __shared__ __attribute__((aligned(16))) int32_t sel[kListMax];
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int hkv = bh - b * Hkv;
  const int t = threadIdx.x;
  // Query rows and the head's K/V rows; these use arguments past the preloaded ones and
  // are computed where the attention needs them.
  auto row0 = [&]() { return (int64_t)b * at_use(Hq) + (int64_t)hkv * G; };
  auto head_row0 = [&]() { return (size_t)bh * (size_t)at_use(cap); };
  // Sequences of their own lengths: the head's candidates, chunks, budget and window
  // follow its n_b; S stays the launch's chunk stride (sized for the longest).
  int Sb = S;
  if (ctx_len) {
    C = head_candidates(ctx_len, b, max_ctx, lo, n_local);
    Sb = (int)((C + CH - 1) / CH);
    keff = (int)(k < C ? k : C);
  }

  // The query fragment is loaded after the chunks are compacted: its load then issues
  // with the first K/V rows and does not hold registers through the compaction.
  typename AttentionCore<BF16, G>::type ga;
  bool ga_ready = false;
  auto attend_list = [&](int len) {
    if (!ga_ready) {
      ga.init(at_use(q), row0(), scale_log2);
      ga_ready = true;
    }
    ga.run_block(at_use(kc), at_use(vc), head_row0(), len, [&](int r) { return sel[r]; });
  };
  if (c < Sc) {
    // Chunk workgroup c covers chunk groups c and, when REPS = 2, c + Sc of its head, one
    // after the other: the head's threshold is derived once for both, and the two
    // groups' tokens go into one online softmax (one partial per workgroup).  A group is
    // CPB chunks; a shorter sequence spreads its Sb chunks over all Sc * REPS groups of
    // its head (Sb <= S <= Sc * REPS * CPB, so at most CPB each).
    const int ngroups = Sc * REPS;
    const int cpb = ctx_len ? (Sb + ngroups - 1) / ngroups : CPB;
    // chunks [g0(r), g1(r)) of group r; uniform over the workgroup
    auto g0 = [&](int r) { return (c + r * Sc) * cpb; };
    auto g1 = [&](int r) { return min(Sb, g0(r) + cpb); };
    // A group's candidates are one run of the head's distance bytes (token order); thread
    // t holds tokens [t*TPT, (t+1)*TPT) of the run.  The first group's bytes are requested
    // before the threshold is derived, and arrive while it is.
    constexpr int TPT = MAXC * LPT;
    const uint8_t *dh = stash + (int64_t)bh * S * CH;
    auto load_group = [&](int r, uint32_t(&w)[TPT / 4]) {
      const bool ok = (int64_t)t * TPT < (int64_t)(g1(r) - g0(r)) * CH;
      load_run<TPT>(dh, (int64_t)g0(r) * CH + (int64_t)t * TPT, ok, w);
    };
    __shared__ int2 gbase[REPS];               // head counts below / at T before group r
    __shared__ uint32_t scan_lds[kScanThreads / 64];
    uint32_t w[TPT / 4];
    // The head's threshold, tie quota and the counts before each group, from the chunk
    // histograms, derived by every workgroup of the head, which saves a kernel and its
    // dependent round trip: two reads of the histograms (superbins, then the bins of the
    // superbin holding T) and two exchanges.  When the head's bin counts fit in LDS
    // (Sb * bins <= kHistLdsWords: up to 32 chunks of 128-bit codes), they are requested
    // together with the distance bytes and the threshold is derived from LDS, one round
    // trip to memory instead of two.
    int T, quota;
    {
      const int roww = bins + bins / 8;
      const uint32_t *hh = hist + (int64_t)bh * S * roww;
      const bool hist_lds = keff > 0 && Sb * bins <= kHistLdsWords;   // uniform
      constexpr int HV = kHistLdsWords / 4 / kScanThreads;
      const int qpr = bins / 4;                // 16-byte vectors per chunk row
      uint4 hv[HV];
      if (hist_lds) {
#pragma unroll
        for (int i = 0; i < HV; ++i) {
          const int v = t + kScanThreads * i;
          const int cc = bins == 128 ? v >> 5 : v >> 4;     // v / qpr
          hv[i] = cc < Sb ? *reinterpret_cast<const uint4 *>(hh + (int64_t)cc * roww + 4 * (v - cc * qpr))
                          : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      load_group(0, w);
      auto sink = [&](int cc, const int4 &m) {
#pragma unroll
        for (int r = 0; r < REPS; ++r)
          if (cc == g0(r)) gbase[r] = make_int2(m.x, m.y);
      };
      if (hist_lds) {
        uint32_t *hl = reinterpret_cast<uint32_t *>(sel);
#pragma unroll
        for (int i = 0; i < HV; ++i) {
          const int v = t + kScanThreads * i;
          if (v < Sb * qpr) reinterpret_cast<uint4 *>(hl)[v] = hv[i];
        }
        __syncthreads();
        if (bins == 128)
          head_threshold_lds<128>(hl, Sb, C, CH, keff, T, quota, sink);
        else
          head_threshold_lds<64>(hl, Sb, C, CH, keff, T, quota, sink);
      } else {
        int gs[REPS], lb[REPS], eb[REPS];
#pragma unroll
        for (int r = 0; r < REPS; ++r) gs[r] = g0(r);
        if (bins == 128)
          head_threshold_groups<128, REPS>(hh, Sb, CH, keff, gs, T, quota, lb, eb);
        else
          head_threshold_groups<64, REPS>(hh, Sb, CH, keff, gs, T, quota, lb, eb);
        if (t == 0 && T >= 0) {
#pragma unroll
          for (int r = 0; r < REPS; ++r) gbase[r] = make_int2(lb[r], eb[r]);
        }
      }
      if (c == 0 && t == 0) count[bh] = keff;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < REPS; ++r) {
      if (T < 0 || g0(r) >= g1(r)) break;      // uniform: nothing selected, or no chunks
      if (r > 0) load_group(r, w);
      const int2 gb = gbase[r];
      const int64_t tok_t = lo + (int64_t)g0(r) * CH + (int64_t)t * TPT;   // thread's first token
      RunSelect<TPT> rs;
      rs.build(w, T, quota, gb.x, gb.y, scan_lds);
      const int total = rs.total, first = rs.first;
      // The group's selected tokens occupy positions [first, first + total) of the head's
      // list.  They go to the LDS list first and to the index list afterwards, in
      // coalesced stores; the workgroup attends over the LDS list.
      const int n0 = min(total, kListMax);
      if (n0 > 0) {
        rs.emit(0, n0, [&](int pos, int off) { sel[pos] = (int32_t)(tok_t + off); });
        __syncthreads();
        int32_t *out = idx + (int64_t)bh * k + first;
        for (int rr = t; rr < n0; rr += kScanThreads) out[rr] = sel[rr];
        attend_list(n0);
      }
      // More than the list holds (a budget of thousands of tokens per group): further
      // rounds of kListMax positions, each rebuilding the masks from the distance bytes
      // so that no mask stays live through the attention.
      for (int base = kListMax; base < total; base += kListMax) {
        __syncthreads();                       // every wavefront is done with the list
        uint32_t w2[TPT / 4];
        load_group(r, w2);
        RunSelect<TPT> rs2;
        rs2.build(w2, T, quota, gb.x, gb.y, scan_lds);
        const int n = min(total - base, kListMax);
        rs2.emit(base, base + n, [&](int pos, int off) { sel[pos - base] = (int32_t)(tok_t + off); });
        __syncthreads();
        int32_t *out = idx + (int64_t)bh * k + first + base;
        for (int rr = t; rr < n; rr += kScanThreads) out[rr] = sel[rr];
        attend_list(n);
      }
      __syncthreads();                         // the list and scan_lds are reused
    }
    if (!ga_ready) ga.init(at_use(q), row0(), scale_log2);
  } else {
    if (ctx_len) {                             // the sequence's own window
      int64_t n = ctx_len[b];
      n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
      win_sinks = (int)(lo < n ? lo : n);
      win_local0 = (n - n_local) > lo ? (n - n_local) : lo;
      n_win = win_sinks + (int)(n > win_local0 ? n - win_local0 : 0);
    }
    ga.init(at_use(q), row0(), scale_log2);
    const int r0 = (c - Sc) * win_rows;
    const int r1 = min(n_win, r0 + win_rows);
    ga.run_block(at_use(kc), at_use(vc), head_row0(), r1 > r0 ? r1 - r0 : 0, [&](int rr) {
      const int r = r0 + rr;
      return r < win_sinks ? r : (int)(win_local0 + (r - win_sinks));
    });
  }
  ga.combine_store(part_o + ((int64_t)c * rows + row0()) * kHeadDim, part_lse + (int64_t)c * rows + row0());
}

#define HK_EMIT_ATTEND_PARAMS                                                                 \
  const uint8_t *__restrict__ stash, const uint32_t *__restrict__ hist,                       \
      const int32_t *__restrict__ ctx_len, int keff, int bins, int S, int CPB, int Sc, int Hkv, \
      int64_t C, int64_t lo, int32_t *__restrict__ count, int k, int32_t *__restrict__ idx,   \
      const void *__restrict__ q, const void *__restrict__ kc, const void *__restrict__ vc,   \
      int Hq, int64_t cap, float scale_log2, int win_sinks, int64_t win_local0, int n_win,    \
      int win_rows, float *__restrict__ part_o, float *__restrict__ part_lse, int64_t rows,   \
      int64_t n_local, int64_t max_ctx
#define HK_EMIT_ATTEND_ARGS                                                                   \
  stash, hist, ctx_len, keff, bins, S, CPB, Sc, Hkv, C, lo, count, k, idx, q, kc, vc, Hq, cap, \
      scale_log2, win_sinks, win_local0, n_win, win_rows, part_o, part_lse, rows, n_local,    \
      max_ctx

// bf16 (matrix cores): held to 168 VGPRs, three workgroups per CU.  fp32 (VALU) keeps
// the compiler's choice: its accumulators would spill under that limit.  MAXC (8, or 4
// when the plan puts at most 4 chunks in a workgroup) sizes the run of distance bytes a
// thread holds (MAXC * LPT tokens) and selects from.  REPS (1 or 2) chunk groups per
// chunk workgroup: 2 when one group of 8 chunks per workgroup would need more workgroups
// than are resident at once.
template <int LPT, int G, int MAXC, int REPS>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(3))) void
emit_attend_bf16_kernel(HK_EMIT_ATTEND_PARAMS) {
  emit_attend_body<LPT, true, G, MAXC, REPS>(HK_EMIT_ATTEND_ARGS);
}
template <int LPT, int G, int MAXC, int REPS>
__global__ __launch_bounds__(kScanThreads) void emit_attend_f32_kernel(HK_EMIT_ATTEND_PARAMS) {
  emit_attend_body<LPT, false, G, MAXC, REPS>(HK_EMIT_ATTEND_ARGS);
}
#undef HK_EMIT_ATTEND_PARAMS
#undef HK_EMIT_ATTEND_ARGS

template <int LPT, bool BF16, int G, int MAXC, int REPS>
void fused_launch_c(const FusedPlan &p, const uint8_t *stash, const uint32_t *hist,
                  int32_t *count, int k, int32_t *idx, const void *q, const void *kc,
                  const void *vc, int Hq, int Hkv, int64_t cap, float scale_log2, float *po,
                  float *pl, int64_t rows, const int32_t *ctx_len, hipStream_t st) {
  if constexpr (BF16)
    hipLaunchKernelGGL((emit_attend_bf16_kernel<LPT, G, MAXC, REPS>), dim3(p.parts, p.r.BH),
                       dim3(kScanThreads), 0, st, stash, hist, ctx_len, p.r.keff, p.r.BINS, p.r.S,
                       p.cpb, p.Sc, Hkv, p.r.C, p.r.lo, count, k, idx, q, kc, vc, Hq, cap,
                       scale_log2, p.win_sinks, p.win_local0, p.n_win, p.win_rows, po, pl, rows,
                       p.n_local, p.max_ctx);
  else
    hipLaunchKernelGGL((emit_attend_f32_kernel<LPT, G, MAXC, REPS>), dim3(p.parts, p.r.BH),
                       dim3(kScanThreads), 0, st, stash, hist, ctx_len, p.r.keff, p.r.BINS, p.r.S,
                       p.cpb, p.Sc, Hkv, p.r.C, p.r.lo, count, k, idx, q, kc, vc, Hq, cap,
                       scale_log2, p.win_sinks, p.win_local0, p.n_win, p.win_rows, po, pl, rows,
                       p.n_local, p.max_ctx);
}

template <int LPT, bool BF16, int G>
void fused_launch(const FusedPlan &p, const uint8_t *stash, const uint32_t *hist,
                  int32_t *count, int k, int32_t *idx, const void *q, const void *kc,
                  const void *vc, int Hq, int Hkv, int64_t cap, float scale_log2, float *po,
                  float *pl, int64_t rows, const int32_t *ctx_len, hipStream_t st) {
  if (p.cpb <= 4)
    fused_launch_c<LPT, BF16, G, 4, 1>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv, cap,
                                       scale_log2, po, pl, rows, ctx_len, st);
  else if (p.reps == 2)
    fused_launch_c<LPT, BF16, G, kMaxCpb, 2>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv,
                                             cap, scale_log2, po, pl, rows, ctx_len, st);
  else
    fused_launch_c<LPT, BF16, G, kMaxCpb, 1>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv,
                                             cap, scale_log2, po, pl, rows, ctx_len, st);
}

template <int LPT, bool BF16>
void fused_dispatch_g(const FusedPlan &p, const uint8_t *stash, const uint32_t *hist,
                      int32_t *count, int k, int32_t *idx, const void *q, const void *kc,
                      const void *vc, int Hq, int Hkv, int64_t cap, float sl2, float *po,
                      float *pl, int64_t rows, const int32_t *ctx_len, hipStream_t st) {
#define HK_FUSED_CASE(GG)                                                                   \
  case GG:                                                                                  \
    fused_launch<LPT, BF16, GG>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv, cap,    \
                                sl2, po, pl, rows, ctx_len, st);                            \
    break;
  switch (p.G) {
    HK_FUSED_CASE(1) HK_FUSED_CASE(2) HK_FUSED_CASE(3) HK_FUSED_CASE(4)
    HK_FUSED_CASE(5) HK_FUSED_CASE(6) HK_FUSED_CASE(7) HK_FUSED_CASE(8)
    default: break;
  }
#undef HK_FUSED_CASE
}

}  // namespace

FusedPlan plan_fused(int bits, int B, int Hq, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                     int k) {
  FusedPlan p;
  p.r = plan_retrieve(bits, B, Hkv, n_ctx, n_sink, n_local, k);
  p.G = Hkv > 0 ? Hq / Hkv : 1;
  const int64_t sinks = n_sink < n_ctx ? n_sink : n_ctx;
  const int64_t local0 = (n_ctx - n_local) > n_sink ? (n_ctx - n_local) : n_sink;
  p.win_sinks = (int)sinks;
  p.win_local0 = local0;
  p.n_local = n_local;
  p.max_ctx = n_ctx;
  p.n_win = (int)(sinks + (n_ctx > local0 ? n_ctx - local0 : 0));
  // Chunks per workgroup: at least two 16-row tiles of selected rows per workgroup and no
  // more workgroups than are resident at once, while keeping at least 128 workgroups.
  // Every workgroup derives its head's threshold (a fixed cost per workgroup), so when
  // the selection is small fewer, larger workgroups win: on 8 heads x 524288 codes with
  // top-1024, 8 chunks (32 rows) per workgroup take the step from 30.0 to 28.4 us against
  // 4 chunks (16 rows); with thousands of rows per head the resident-workgroup bound
  // decides as before.  (Each chunk adds compaction work for all of its tokens, so chunks
  // are not merged just to give every wavefront a tile: that lengthens the serial phase.)
  const int64_t chunks = (int64_t)p.r.BH * p.r.S;
  const int64_t per_chunk = p.r.S > 0 ? (p.r.keff + p.r.S - 1) / p.r.S : 1;
  int cpb = 1;
  while (cpb < kMaxCpb && chunks / (2 * cpb) >= 128 &&
         (per_chunk * cpb < 32 || chunks / cpb > kResidentBlocks))
    cpb *= 2;
  p.cpb = cpb;
  p.Sc = (p.r.S + cpb - 1) / cpb;
  p.reps = 1;
  // Window slices of about as many rows as a chunk workgroup attends (at least 64), of
  // equal size.
  const int64_t target = per_chunk * cpb > 64 ? per_chunk * cpb : 64;
  p.Sw = (int)((p.n_win + target - 1) / target);
  p.win_rows = p.Sw > 0 ? (int)((p.n_win + p.Sw - 1) / p.Sw) : 64;
  // Two groups of 8 chunks per chunk workgroup when one would need more workgroups than
  // are resident at once: the head's threshold is derived once for both groups, and the
  // serial phase is not paid again by a second round of workgroups (16 x 131072 tokens,
  // 8 KV heads: 768 workgroups in one round instead of 1280, select+attend 65 -> 58 us).
  if (p.cpb == kMaxCpb && p.Sc >= 2 && (int64_t)p.r.BH * (p.Sc + p.Sw) > kResidentBlocks) {
    p.reps = 2;
    p.Sc = (p.Sc + 1) / 2;
  }
  p.parts = p.Sc + p.Sw;
  size_t off = p.r.total;
  const size_t rows = (size_t)B * Hq;
  p.off_o = off;
  off = align_up(off + (size_t)p.parts * rows * kHeadDim * sizeof(float), 256);
  p.off_lse = off;
  off = align_up(off + (size_t)p.parts * rows * sizeof(float), 256);
  p.total = off;
  return p;
}

hipError_t launch_fused_attend(const FusedPlan &p, const void *q, const void *kc,
                               const void *vc, int dtype, int B, int Hq, int Hkv, int64_t cap,
                               float scale, int k, int32_t *idx, int32_t *count, float *o,
                               float *lse, void *ws, hipStream_t st, const int32_t *ctx_len) {
  const int64_t rows = (int64_t)B * Hq;
  if (rows == 0) return hipSuccess;
  // Without candidate chunks no workgroup derives the threshold: the threshold kernel
  // writes the counts (k_eff = 0) instead.
  if (p.Sc == 0) {
    hipError_t e = launch_topk_threshold(p.r, count, ws, st);
    if (e != hipSuccess) return e;
  }
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  float *po = reinterpret_cast<float *>(w8 + p.off_o);
  float *pl = reinterpret_cast<float *>(w8 + p.off_lse);
  if (p.parts > 0) {
    const uint8_t *stash = w8 + p.r.off_stash;
    const uint32_t *hist = reinterpret_cast<const uint32_t *>(w8 + p.r.off_hist);
    const float sl2 = scale * kLog2e;
    const bool bf = dtype == HK_BF16;
#define HK_LPT(L)                                                                            \
  if (bf) fused_dispatch_g<L, true>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv, cap,  \
                                    sl2, po, pl, rows, ctx_len, st);                         \
  else fused_dispatch_g<L, false>(p, stash, hist, count, k, idx, q, kc, vc, Hq, Hkv, cap,    \
                                  sl2, po, pl, rows, ctx_len, st);
    if (p.r.lpt == 8) { HK_LPT(8) }
    else { HK_LPT(4) }
#undef HK_LPT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_lse_merge_parts(po, pl, p.parts, rows, kHeadDim, o, lse, st);
}

}  // namespace hk
