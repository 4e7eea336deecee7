// Exact top-k by attention logit -- the pages' "oracle top-k" (Spotlight Attention:
// Key results, the baseline its retrieval IoU is measured against) and exact Flat
// search (RetrievalAttention, atlas summary: Results) -- and the overlap of two
// ascending token lists, from which the retrieval IoU |A n B| / |A u B| follows.
//
// Per (batch, KV head) the candidates [n_sink, n_ctx - n_local) are ranked by the
// group's summed logit sum_g q_g . k_j (the ranking of the group-mean query, as the hash
// retrieval uses), largest first, ties to the lower token; the first k_eff are returned
// in ascending token order.
//
//   exact_scan    grid (S, B*Hkv), 1024 candidates per workgroup: every K row is read
//                 once (16 lanes x 16 bytes per bf16 row), its fp32 logit becomes a
//                 32-bit key that orders logits descending, and the chunk's histogram
//                 of the key's top byte is written.  Bound by HBM bandwidth (d*e bytes
//                 per candidate).
//   exact_pick    one workgroup per head, once per key byte: the byte value that holds
//                 the k-th key among the keys matching the bytes found so far.
//   exact_hist    grid (S, B*Hkv): histogram of the next key byte among the keys that
//                 match the bytes found so far (4 bytes read per candidate).
//   exact_count   grid (S, B*Hkv): per chunk, the keys below and equal to the threshold.
//   exact_prefix  one workgroup per head: exclusive prefix of those counts over chunks.
//   exact_emit    grid (S, B*Hkv): writes the selected tokens at their final positions.
// Deterministic: LDS histograms only, no ordering of results by atomics.
#include "select_core.h"

namespace hk {
namespace {

constexpr int kExThreads = 256;
constexpr int kExChunk = 1024;               // candidates per workgroup
constexpr int kExPerThread = kExChunk / kExThreads;
constexpr int kExUnroll = 8;

// A 32-bit key that orders finite logits descending: larger logit, smaller key.
__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ void write_hist(uint32_t (*h)[256], uint32_t *out) {
  __syncthreads();
  const int t = threadIdx.x;
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < kExThreads / 64; ++w) s += h[w][t];
  out[t] = s;
}

template <bool BF16>
__global__ __launch_bounds__(kExThreads) void exact_scan_kernel(
    const void *__restrict__ q, const void *__restrict__ kc, int Hq, int Hkv, int64_t cap,
    int64_t lo, int64_t C, int S, uint32_t *__restrict__ keys, uint32_t *__restrict__ hist) {
  constexpr int LPR = BF16 ? 16 : 32;        // lanes per K row, 16 bytes each
  constexpr int RPI = 64 / LPR;              // rows per wavefront load
  constexpr int EPL = BF16 ? 8 : 4;          // elements per lane
  constexpr int ITERS = kExChunk / 4 / RPI;  // loads per wavefront
  __shared__ uint32_t h[kExThreads / 64][256];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = bh / Hkv, hkv = bh - b * Hkv, G = Hq / Hkv;
  for (int i = t; i < (kExThreads / 64) * 256; i += kExThreads) (&h[0][0])[i] = 0u;
  // This lane's elements e0 .. e0 + EPL - 1 of the group's summed query.
  const int e0 = EPL * (lane % LPR);
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
  for (int g = 0; g < G; ++g) {
    const size_t row = ((size_t)b * Hq + (size_t)hkv * G + g) * kHeadDim + e0;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      qs[e] += BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t *>(q)[row + e] << 16)
                    : static_cast<const float *>(q)[row + e];
  }
  __syncthreads();
  const int64_t p_wave = (int64_t)c * kExChunk + wave * (kExChunk / 4) + lane / LPR;
  const u32x4 *kb = reinterpret_cast<const u32x4 *>(kc);
  const size_t head = (size_t)bh * (size_t)cap + (size_t)lo;
  uint32_t *kout = keys + (int64_t)bh * S * kExChunk;
#pragma unroll 1
  for (int it0 = 0; it0 < ITERS; it0 += kExUnroll) {
    u32x4 v[kExUnroll];
#pragma unroll
    for (int u = 0; u < kExUnroll; ++u) {
      const int64_t p = p_wave + (int64_t)(it0 + u) * RPI;
      v[u] = p < C ? __builtin_nontemporal_load(kb + ((head + (size_t)p) * kHeadDim + e0) / EPL)
                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kExUnroll; ++u) {
      const int64_t p = p_wave + (int64_t)(it0 + u) * RPI;
      const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
      float s = 0.f;
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = fmaf(qs[2 * e], __uint_as_float(w[e] << 16), s);
          s = fmaf(qs[2 * e + 1], __uint_as_float(w[e] & 0xFFFF0000u), s);
        }
        s = row16_sum(s);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(qs[e], __uint_as_float(w[e]), s);
        s = row16_sum(s);
        s += __shfl_xor(s, 16);
      }
      if (lane % LPR == 0 && p < (int64_t)S * kExChunk) {
        const bool live = p < C;
        const uint32_t key = live ? desc_key(s) : 0xFFFFFFFFu;
        kout[p] = key;
        if (live) atomicAdd(&h[wave][key >> 24], 1u);
      }
    }
  }
  write_hist(h, hist + ((int64_t)bh * S + c) * 256);
}

// state[bh] = (key bytes found so far, rank still needed among the keys matching them)
__global__ __launch_bounds__(kExThreads) void exact_pick_kernel(const uint32_t *__restrict__ hist,
                                                               int S, int r, int keff,
                                                               uint2 *__restrict__ state) {
  __shared__ uint32_t lds[kExThreads / 64];
  const int bh = blockIdx.x, t = threadIdx.x;
  // Sixteen chunk histograms in flight at a time: the sum is a run of independent loads.
  const uint32_t *hp = hist + (int64_t)bh * S * 256 + t;
  uint32_t n = 0;
  int c = 0;
  for (; c + 16 <= S; c += 16) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = hp[(int64_t)(c + u) * 256];
#pragma unroll
    for (int u = 0; u < 16; ++u) n += v[u];
  }
  for (; c < S; ++c) n += hp[(int64_t)c * 256];
  const uint2 st = r == 0 ? make_uint2(0u, (uint32_t)keff) : state[bh];
  uint32_t total;
  const uint32_t below = block_excl_scan_u32<kExThreads>(n, lds, total);
  if (below < st.y && st.y <= below + n)
    state[bh] = make_uint2(st.x | ((uint32_t)t << (24 - 8 * r)), st.y - below);
}

__global__ __launch_bounds__(kExThreads) void exact_hist_kernel(const uint32_t *__restrict__ keys,
                                                               const uint2 *__restrict__ state,
                                                               int S, int64_t C, int r,
                                                               uint32_t *__restrict__ hist) {
  __shared__ uint32_t h[kExThreads / 64][256];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, wave = t >> 6;
  for (int i = t; i < (kExThreads / 64) * 256; i += kExThreads) (&h[0][0])[i] = 0u;
  const uint32_t prefix = state[bh].x >> (32 - 8 * r);
  __syncthreads();
  const int64_t p0 = (int64_t)c * kExChunk + kExPerThread * t;
  const uint4 k4 = *reinterpret_cast<const uint4 *>(keys + (int64_t)bh * S * kExChunk + p0);
  const uint32_t kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (p0 + j < C && (kv[j] >> (32 - 8 * r)) == prefix)
      atomicAdd(&h[wave][(kv[j] >> (24 - 8 * r)) & 0xFFu], 1u);
  write_hist(h, hist + ((int64_t)bh * S + c) * 256);
}

__global__ __launch_bounds__(kExThreads) void exact_count_kernel(const uint32_t *__restrict__ keys,
                                                                const uint2 *__restrict__ state,
                                                                int S, int64_t C,
                                                                uint2 *__restrict__ cnt) {
  __shared__ uint32_t red[2][kExThreads / 64];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const uint32_t T = state[bh].x;
  const int64_t p0 = (int64_t)c * kExChunk + kExPerThread * t;
  const uint4 k4 = *reinterpret_cast<const uint4 *>(keys + (int64_t)bh * S * kExChunk + p0);
  const uint32_t kv[4] = {k4.x, k4.y, k4.z, k4.w};
  uint32_t lt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (p0 + j < C) {
      lt += kv[j] < T ? 1u : 0u;
      eq += kv[j] == T ? 1u : 0u;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lt += __shfl_xor(lt, o);
    eq += __shfl_xor(eq, o);
  }
  if ((t & 63) == 0) {
    red[0][t >> 6] = lt;
    red[1][t >> 6] = eq;
  }
  __syncthreads();
  if (t == 0) {
    uint2 s = make_uint2(0u, 0u);
#pragma unroll
    for (int w = 0; w < kExThreads / 64; ++w) {
      s.x += red[0][w];
      s.y += red[1][w];
    }
    cnt[(int64_t)bh * S + c] = s;
  }
}

// meta[bh][c] = (below T before chunk c, at T before it, below T in it, at T in it)
__global__ __launch_bounds__(kExThreads) void exact_prefix_kernel(const uint2 *__restrict__ cnt,
                                                                 int S, int keff,
                                                                 int4 *__restrict__ meta,
                                                                 int32_t *__restrict__ count) {
  __shared__ uint32_t lds[2][kExThreads / 64];
  const int bh = blockIdx.x, t = threadIdx.x;
  uint32_t run_lt = 0, run_eq = 0;
  for (int c0 = 0; c0 < S; c0 += kExThreads) {
    const int c = c0 + t;
    const uint2 v = c < S ? cnt[(int64_t)bh * S + c] : make_uint2(0u, 0u);
    uint32_t tot_lt, tot_eq;
    const uint32_t ex_lt = block_excl_scan_u32<kExThreads>(v.x, lds[0], tot_lt);
    const uint32_t ex_eq = block_excl_scan_u32<kExThreads>(v.y, lds[1], tot_eq);
    if (c < S)
      meta[(int64_t)bh * S + c] = make_int4((int)(run_lt + ex_lt), (int)(run_eq + ex_eq), (int)v.x, (int)v.y);
    run_lt += tot_lt;
    run_eq += tot_eq;
  }
  if (t == 0) count[bh] = keff;
}

// Thread t takes candidates 4t .. 4t+3 of the chunk: masks of keys below / at T, one
// block-wide scan of the packed counts, then each set bit is written at its position
// (below: (below before) + min(at before, quota); at: (below before) + (at before)
// while (at before) < quota).
__global__ __launch_bounds__(kExThreads) void exact_emit_kernel(const uint32_t *__restrict__ keys,
                                                               const uint2 *__restrict__ state,
                                                               const int4 *__restrict__ meta,
                                                               int S, int64_t C, int64_t lo, int k,
                                                               int32_t *__restrict__ idx) {
  __shared__ uint32_t wtot[kExThreads / 64];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint2 st = state[bh];
  const uint32_t T = st.x;
  const int quota = (int)st.y;
  const int4 mt = meta[(int64_t)bh * S + c];
  const int64_t p0 = (int64_t)c * kExChunk + kExPerThread * t;
  const uint4 k4 = *reinterpret_cast<const uint4 *>(keys + (int64_t)bh * S * kExChunk + p0);
  const uint32_t kv[4] = {k4.x, k4.y, k4.z, k4.w};
  uint32_t mlt = 0, meq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (p0 + j < C) {
      mlt |= (kv[j] < T ? 1u : 0u) << j;
      meq |= (kv[j] == T ? 1u : 0u) << j;
    }
  }
  const uint32_t cntp = (uint32_t)__popc(mlt) | ((uint32_t)__popc(meq) << 16);
  const uint32_t inc = wave_incl_scan_dpp(cntp);
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  uint32_t before = inc - cntp;
#pragma unroll
  for (int w = 0; w < kExThreads / 64; ++w)
    if (w < wave) before += wtot[w];
  const int lt0 = mt.x + (int)(before & 0xFFFFu);
  const int eq0 = mt.y + (int)(before >> 16);
  int32_t *out = idx + (int64_t)bh * k;
  uint32_t all = mlt | meq;
  while (all) {
    const int j = __builtin_ctz(all);
    all &= all - 1;
    const uint32_t below = (1u << j) - 1u;
    const int ltb = lt0 + __popc(mlt & below);
    const int eqb = eq0 + __popc(meq & below);
    int pos = -1;
    if ((mlt >> j) & 1u) pos = ltb + min(eqb, quota);
    else if (eqb < quota) pos = ltb + eqb;
    if (pos >= 0) out[pos] = (int32_t)(lo + p0 + j);
  }
}

__global__ __launch_bounds__(kExThreads) void count_fill_kernel(int32_t *count, int n, int v) {
  const int i = blockIdx.x * kExThreads + threadIdx.x;
  if (i < n) count[i] = v;
}

// inter[l] = |A_l n B_l| for ascending lists A_l, B_l: each entry of A binary-searched
// in B.
__global__ __launch_bounds__(kExThreads) void intersect_kernel(
    const int32_t *__restrict__ a, const int32_t *__restrict__ ca, int64_t sa,
    const int32_t *__restrict__ b, const int32_t *__restrict__ cb, int64_t sb,
    int32_t *__restrict__ inter) {
  __shared__ uint32_t red[kExThreads / 64];
  const int l = blockIdx.x, t = threadIdx.x;
  const int na = (int)min((int64_t)max(ca[l], 0), sa);
  const int nb = (int)min((int64_t)max(cb[l], 0), sb);
  const int32_t *A = a + (int64_t)l * sa;
  const int32_t *Bl = b + (int64_t)l * sb;
  uint32_t n = 0;
  for (int i = t; i < na; i += kExThreads) {
    const int32_t x = A[i];
    int lo = 0, hi = nb;                        // first entry >= x in [lo, hi)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (Bl[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    n += (lo < nb && Bl[lo] == x) ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  if ((t & 63) == 0) red[t >> 6] = n;
  __syncthreads();
  if (t == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kExThreads / 64; ++w) s += red[w];
    inter[l] = (int32_t)s;
  }
}

}  // namespace

ExactPlan plan_exact(int B, int Hkv, int64_t n_ctx, int n_sink, int n_local, int k) {
  ExactPlan p;
  p.BH = B * Hkv;
  p.lo = n_sink;
  const int64_t hi = n_ctx - n_local;
  p.C = hi > p.lo ? hi - p.lo : 0;
  p.keff = (int)(k < p.C ? k : p.C);
  if (p.keff < 0) p.keff = 0;
  p.S = (int)((p.C + kExChunk - 1) / kExChunk);
  const size_t bhs = (size_t)p.BH * (size_t)p.S;
  size_t off = 0;
  p.off_keys = off;
  off = align_up(off + bhs * kExChunk * sizeof(uint32_t), 256);
  p.off_hist = off;
  off = align_up(off + bhs * 256 * sizeof(uint32_t), 256);
  p.off_cnt = off;
  off = align_up(off + bhs * sizeof(uint2), 256);
  p.off_meta = off;
  off = align_up(off + bhs * sizeof(int4), 256);
  p.off_state = off;
  off = align_up(off + (size_t)p.BH * sizeof(uint2), 256);
  p.total = off;
  return p;
}

hipError_t launch_exact_topk(const ExactPlan &p, const void *q, const void *kc, int dtype, int Hq,
                             int Hkv, int64_t cap, int k, int32_t *idx, int32_t *count, void *ws,
                             hipStream_t st) {
  if (p.BH == 0) return hipSuccess;
  if (p.keff == 0) {
    hipLaunchKernelGGL(count_fill_kernel, dim3((p.BH + kExThreads - 1) / kExThreads),
                       dim3(kExThreads), 0, st, count, p.BH, 0);
    return hipGetLastError();
  }
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  uint32_t *keys = reinterpret_cast<uint32_t *>(w8 + p.off_keys);
  uint32_t *hist = reinterpret_cast<uint32_t *>(w8 + p.off_hist);
  uint2 *cnt = reinterpret_cast<uint2 *>(w8 + p.off_cnt);
  int4 *meta = reinterpret_cast<int4 *>(w8 + p.off_meta);
  uint2 *state = reinterpret_cast<uint2 *>(w8 + p.off_state);
  const dim3 grid(p.S, p.BH), blk(kExThreads);
  if (dtype == HK_BF16)
    hipLaunchKernelGGL(exact_scan_kernel<true>, grid, blk, 0, st, q, kc, Hq, Hkv, cap, p.lo, p.C,
                       p.S, keys, hist);
  else
    hipLaunchKernelGGL(exact_scan_kernel<false>, grid, blk, 0, st, q, kc, Hq, Hkv, cap, p.lo, p.C,
                       p.S, keys, hist);
  for (int r = 0; r < 4; ++r) {
    if (r > 0)
      hipLaunchKernelGGL(exact_hist_kernel, grid, blk, 0, st, keys, state, p.S, p.C, r, hist);
    hipLaunchKernelGGL(exact_pick_kernel, dim3(p.BH), blk, 0, st, hist, p.S, r, p.keff, state);
  }
  hipLaunchKernelGGL(exact_count_kernel, grid, blk, 0, st, keys, state, p.S, p.C, cnt);
  hipLaunchKernelGGL(exact_prefix_kernel, dim3(p.BH), blk, 0, st, cnt, p.S, p.keff, meta, count);
  hipLaunchKernelGGL(exact_emit_kernel, grid, blk, 0, st, keys, state, meta, p.S, p.C, p.lo, k,
                     idx);
  return hipGetLastError();
}

hipError_t launch_intersect(const int32_t *a, const int32_t *ca, int64_t sa, const int32_t *b,
                            const int32_t *cb, int64_t sb, int n_lists, int32_t *inter,
                            hipStream_t st) {
  hipLaunchKernelGGL(intersect_kernel, dim3(n_lists), dim3(kExThreads), 0, st, a, ca, sa, b, cb, sb,
                     inter);
  return hipGetLastError();
}

}  // namespace hk
