// Internal declarations shared by the HIP translation units of libhk.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hk.h"

namespace hk {

constexpr int kHeadDim = 128;
constexpr int kHidden = 256;
constexpr int kMaxGroup = 8;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Candidates [lo, n - n_local) of sequence b whose context length is ctx_len[b],
// clamped to [0, max_ctx].
__device__ __forceinline__ int64_t head_candidates(const int32_t *ctx_len, int b, int64_t max_ctx,
                                                   int64_t lo, int64_t n_local) {
  int64_t n = ctx_len[b];
  n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
  const int64_t hi = n - n_local;
  return hi > lo ? hi - lo : 0;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One packed code of W words as a vector load, and its Hamming distance to a query code.
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

// ---------------------------------------------------------------- retrieval plan
// Candidate tokens of each (b, KV head) are cut into S chunks of `ch` tokens; one
// workgroup scans one chunk.  The workspace holds
//   stash  [BH][S*ch] uint8     per-token Hamming distance (255 past the last candidate)
//   hist   [BH][S][BINS + BINS/8] uint32 per-chunk histogram of distances 0 .. BINS-1
//                               (BINS = bits), then counts of 8 consecutive distances
//   meta   [BH][S] int4        (#dist<T before chunk, #dist==T before chunk, #<T, #==T)
//   params [BH] int2           (threshold T or -1, tie quota)
struct RetrievePlan {
  int W = 0, BINS = 0, lpt = 0, ch = 0, S = 0, BH = 0, keff = 0;
  int64_t lo = 0, C = 0;
  size_t off_stash = 0, off_hist = 0, off_meta = 0, off_params = 0, total = 0;
};
RetrievePlan plan_retrieve(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                           int k);
hipError_t launch_hamming_scan(const RetrievePlan &p, const uint32_t *codes,
                               const uint32_t *qcodes, int64_t cap, void *ws, hipStream_t st,
                               const int32_t *ctx_len = nullptr, int Hkv = 1,
                               int64_t n_local = 0, int64_t max_ctx = 0);
// Per-query-head retrieval: p planned with B*Hq heads; each code is read once and
// compared with the G query codes of its KV head.
// The whole step of small heads in one workgroup each (tiny.hip): one query head per
// KV head, at most kTinyC candidates and kTinyList selected + window rows per head, at
// most kTinyMaxHeads heads.
constexpr int kTinyC = 4096;
constexpr int kTinyList = 1024;
constexpr int kTinyMaxHeads = 256;
bool tiny_step_fits(int B, int Hq, int Hkv, int64_t C, int keff, int n_win);
hipError_t launch_tiny_step(const hk_hash &h, const RetrievePlan &p, const void *q,
                            const uint32_t *codes, const void *kc, const void *vc, int B,
                            int Hq, int Hkv, int64_t cap, int k, float scale, int win_sinks,
                            int64_t win_local0, int n_win, uint32_t *qcodes, int32_t *idx,
                            int32_t *count, float *o, float *lse, hipStream_t st);
// The scan with the query hash computed inside it (one code per KV head from the group
// mean of q, fp32 arithmetic; chunk 0 writes it to qcodes), for plans that
// scan_hashes_query accepts: sign codes, and hashes with weights at most
// kScanQueryMaxBlocks workgroups with ordinary stores.
constexpr int64_t kScanQueryMaxBlocks = 512;
bool scan_hashes_query(const RetrievePlan &p, const hk_hash &h);
hipError_t launch_hamming_scan_query(const RetrievePlan &p, const hk_hash &h, const void *q,
                                     int Hq, int Hkv, const uint32_t *codes, int64_t cap,
                                     uint32_t *qcodes, void *ws, hipStream_t st);
hipError_t launch_hamming_scan_qheads(const RetrievePlan &p, int G, const uint32_t *codes,
                                      const uint32_t *qcodes, int64_t cap, void *ws,
                                      hipStream_t st);
hipError_t launch_topk_select(const RetrievePlan &p, int k, int32_t *idx, int32_t *count,
                              void *ws, hipStream_t st);
hipError_t launch_topk_threshold(const RetrievePlan &p, int32_t *count, void *ws,
                                 hipStream_t st);
hipError_t launch_window_indices(int64_t n_ctx, int n_sink, int n_local, int32_t *idx,
                                 hipStream_t st);

// ---------------------------------------------------------------- attention plan
// The token list of each (b, KV head) is split into P slices; one workgroup gathers a
// slice for all G query heads of the group.  With P > 1 the workspace holds normalised
// partials o [P][B*Hq][d] and lse [P][B*Hq], merged by the log-sum-exp kernel.
struct DecodePlan {
  int P = 1, rows_per_split = 0, G = 1;
  size_t off_o = 0, off_lse = 0, total = 0;
};
DecodePlan plan_decode(int B, int Hq, int Hkv, int max_count);
hipError_t launch_sparse_decode(const DecodePlan &p, const void *q, const void *k,
                                const void *v, int dtype, int B, int Hq, int Hkv,
                                int64_t cap, const int32_t *idx, int64_t idx_stride,
                                const int32_t *count, int max_count, float scale, float *o,
                                float *lse, void *ws, hipStream_t st, int kv_group = 1);
hipError_t launch_lse_merge(const float *o_parts, const float *lse_parts, int P,
                            int64_t rows, int d, float *o, float *lse, hipStream_t st);
// As launch_lse_merge for P >= 1.  P == 0 (no partial written, none reserved) writes
// o = 0, lse = -inf to every row without reading o_parts or lse_parts.
hipError_t launch_lse_merge_parts(const float *o_parts, const float *lse_parts, int P,
                                  int64_t rows, int d, float *o, float *lse, hipStream_t st);

// ---------------------------------------------------------------- fused step
// hk_retrieve_attend: the retrieval workspace (RetrievePlan) followed by one normalised
// partial per group of `cpb` chunks of each head and per window slice: o [parts][B*Hq][d],
// lse [parts][B*Hq], parts = Sc + Sw.
struct FusedPlan {
  RetrievePlan r;
  int win_sinks = 0, n_win = 0, win_rows = 64, Sw = 0, parts = 0, G = 1, cpb = 1, Sc = 0;
  int reps = 1;                  // chunk groups per chunk workgroup (1 or 2)
  int64_t win_local0 = 0, n_local = 0, max_ctx = 0;
  size_t off_o = 0, off_lse = 0, total = 0;
};
FusedPlan plan_fused(int bits, int B, int Hq, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                     int k);
hipError_t launch_fused_attend(const FusedPlan &p, const void *q, const void *kc,
                               const void *vc, int dtype, int B, int Hq, int Hkv, int64_t cap,
                               float scale, int k, int32_t *idx, int32_t *count, float *o,
                               float *lse, void *ws, hipStream_t st,
                               const int32_t *ctx_len = nullptr);

// ---------------------------------------------------------------- encoders
hipError_t launch_encode_keys(const hk_hash &h, const void *k, int B, int Hkv, int64_t cap,
                              int64_t t0, int64_t t1, uint32_t *codes, hipStream_t st);
hipError_t launch_encode_query(const hk_hash &h, const void *q, int B, int Hq, int Hkv,
                               uint32_t *qcodes, hipStream_t st);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Sums each of K per-lane values (K = 8, 16 or 32) over the 64 lanes of a wavefront, by a
// butterfly that halves the values held per lane at every exchange, then adds across the
// remaining lane bits.  Returns, in lane l, the total of value bitrev(l mod K), where
// bitrev reverses log2(K) bits.
template <int M>
__device__ __forceinline__ uint32_t swizzle_xor(uint32_t v) {     // lane ^ M, M < 32
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
}
template <int K, int M>
__device__ __forceinline__ void transpose_sum_step(uint32_t (&x)[K], int lane) {
  constexpr int H = K / (2 * M);
  // Lanes with bit M set keep the upper half and send the lower; the choice is made with
  // masks, not with a select between elements (which the compiler turns into a dynamic
  // index into the array and so into scratch memory).
  const uint32_t up = (lane & M) ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const uint32_t d = (x[i] ^ x[i + H]) & up;
    const uint32_t send = x[i + H] ^ d;
    const uint32_t keep = x[i] ^ d;
    x[i] = keep + swizzle_xor<M>(send);
  }
}
template <int K>
__device__ __forceinline__ int bitrev_k(int l) {
  int r = 0;
#pragma unroll
  for (int b = 1; b < K; b <<= 1) r = (r << 1) | ((l & b) ? 1 : 0);
  return r;
}
template <int K>
__device__ __forceinline__ uint32_t wave_transpose_sum(uint32_t (&x)[K]) {
  static_assert(K == 8 || K == 16 || K == 32, "8, 16 or 32 values");
  const int lane = threadIdx.x & 63;
  transpose_sum_step<K, 1>(x, lane);
  transpose_sum_step<K, 2>(x, lane);
  transpose_sum_step<K, 4>(x, lane);
  if constexpr (K >= 16) transpose_sum_step<K, 8>(x, lane);
  if constexpr (K == 32) transpose_sum_step<K, 16>(x, lane);
  uint32_t r = x[0];
  if constexpr (K == 8) r += swizzle_xor<8>(r);
  if constexpr (K <= 16) r += swizzle_xor<16>(r);
  r += (uint32_t)__shfl_xor((int)r, 32, 64);
  return r;
}

// Exclusive scan over a workgroup of NT threads (NT multiple of 64).  `lds` holds
// NT/64 entries.  Returns this thread's exclusive prefix and sets `total`.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t *lds,
                                                        uint32_t &total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t x = lds[w];
    off += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// ---------------------------------------------------------------- eviction
// HashEvict's victim per head: the candidate [n_sink, n_ctx - n_local) with the largest
// Hamming distance to the query code, ties to the lowest token.  The workspace holds
// one 64-bit key (distance << 32 | ~token) per chunk of 2048 candidates.
struct EvictPlan {
  int W = 0, BH = 0, S = 0;
  int64_t lo = 0, C = 0;
  size_t total = 0;
};
EvictPlan plan_evict(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local);
hipError_t launch_evict_select(const EvictPlan &p, const uint32_t *codes, const uint32_t *qcodes,
                               int64_t cap, int32_t *victim, void *ws, hipStream_t st);
hipError_t launch_evict_replace(const void *k_new, const void *v_new, const uint32_t *code_new,
                                int elem_bytes, int W, int BH, int64_t cap, const int32_t *victim,
                                void *kc, void *vc, uint32_t *codes, hipStream_t st);

// ---------------------------------------------------------------- exact top-k
// Candidates cut into S chunks of 1024.  Workspace: keys [BH][S*1024] uint32 (logit order
// keys), hist [BH][S][256] uint32, cnt [BH][S] uint2, meta [BH][S] int4, state [BH] uint2.
struct ExactPlan {
  int BH = 0, S = 0, keff = 0;
  int64_t lo = 0, C = 0;
  size_t off_keys = 0, off_hist = 0, off_cnt = 0, off_meta = 0, off_state = 0, total = 0;
};
ExactPlan plan_exact(int B, int Hkv, int64_t n_ctx, int n_sink, int n_local, int k);
hipError_t launch_exact_topk(const ExactPlan &p, const void *q, const void *kc, int dtype, int Hq,
                             int Hkv, int64_t cap, int k, int32_t *idx, int32_t *count, void *ws,
                             hipStream_t st);
hipError_t launch_intersect(const int32_t *a, const int32_t *ca, int64_t sa, const int32_t *b,
                            const int32_t *cb, int64_t sb, int n_lists, int32_t *inter,
                            hipStream_t st);

}  // namespace hk
