// Exact softmax attention restricted to a token list, and the log-sum-exp merge.
//
// Attention over the retrieved tokens only ("partial attention": RetrievalAttention,
// elamur summary: Summary; Spotlight Attention: summary) and over the static sink +
// local window, combined by exact log-sum-exp rescaling (RetrievalAttention, atlas
// summary: Approach).
//
// sparse_decode: one workgroup gathers one slice of one (batch, KV head)'s token list for
// all G query heads of the group (see attend_core.h); with several slices per list the
// normalised partials are merged by the log-sum-exp kernel.  Both are bound by HBM
// bandwidth or, for short lists, by memory latency: 2*d*sizeof(elem) bytes per row
// against 4*d*G flops.
#include "attend_core.h"

namespace hk {
namespace {

constexpr int kMaxSliceRows = 256;         // rows_per_split never exceeds this

// grid (P, B*Hkv).  Writes either the final (o, lse) of its query heads (P == 1) or the
// normalised partial of slice p into out_o + p*rows*d, out_lse + p*rows.
// kv_group: 1 for lists per KV head; G for lists per query head, where the launch's
// "KV heads" are the query heads (Hkv = Hq, G = 1 here) and list bh reads the rows of KV
// head bh / kv_group.
template <bool BF16, int G>
__global__ __launch_bounds__(kAttThreads) void sparse_decode_kernel(
    const void *__restrict__ q, const void *__restrict__ kc, const void *__restrict__ vc,
    int Hq, int Hkv, int64_t cap, const int32_t *__restrict__ idx, int64_t idx_stride,
    const int32_t *__restrict__ count, int max_count, int rows_per_split, float scale_log2,
    float *__restrict__ out_o, float *__restrict__ out_lse, int64_t rows, int kv_group) {
  const int p = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int hkv = bh - b * Hkv;
  const int64_t row0 = (int64_t)b * Hq + (int64_t)hkv * G;

  // The slice's token indices are staged in LDS first (one coalesced read), so the
  // row gathers never wait on an index load.
  __shared__ int32_t s_idx[kMaxSliceRows];
  int n = count ? count[bh] : max_count;
  n = n < 0 ? 0 : (n > max_count ? max_count : n);
  const int r0 = p * rows_per_split;
  const int r1 = min(n, r0 + rows_per_split);
  const int len = r1 > r0 ? r1 - r0 : 0;
  const int32_t *ilist = idx + (int64_t)bh * idx_stride + r0;
  for (int r = threadIdx.x; r < len; r += kAttThreads) s_idx[r] = ilist[r];
  typename AttentionCore<BF16, G>::type ga;
  ga.init(q, row0, scale_log2);
  __syncthreads();
  ga.run_block(kc, vc, (size_t)(bh / kv_group) * (size_t)cap, len, [&](int r) { return s_idx[r]; });
  ga.combine_store(out_o + ((int64_t)p * rows + row0) * kHeadDim, out_lse + (int64_t)p * rows + row0);
}

// Up to 64 parts of d = 128: one workgroup per output row.  Wavefront w merges parts
// w, w+4, ... (up to 16, every load in flight at once: the lse of each part and two
// columns per lane); the four wavefront results combine through LDS.
constexpr int kMergeSmallParts = 64;

__global__ __launch_bounds__(256) void lse_merge_small_kernel(
    const float *__restrict__ o_parts, const float *__restrict__ lse_parts, int P,
    int64_t rows, float *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = kHeadDim;
  constexpr int PW = kMergeSmallParts / 4;     // parts per wavefront
  __shared__ float s_m[4], s_s[4];
  __shared__ float s_acc[4][D];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float x[PW], va[PW], vb[PW];
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int p = wave + 4 * j;
    x[j] = -INFINITY;
    va[j] = vb[j] = 0.f;
    if (p < P) {                               // parts past P are never read
      x[j] = lse_parts[(int64_t)p * rows + row];
      const float *op = o_parts + ((int64_t)p * rows + row) * D;
      va[j] = op[lane];
      vb[j] = op[lane + 64];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < PW; ++j) M = fmaxf(M, x[j]);
  float S = 0.f, acc_a = 0.f, acc_b = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const float wgt = __expf(x[j] - M);      // 0 for parts past P and empty parts
      S += wgt;
      acc_a = fmaf(wgt, va[j], acc_a);
      acc_b = fmaf(wgt, vb[j], acc_b);
    }
  }
  if (lane == 0) {
    s_m[wave] = M;
    s_s[wave] = S;
  }
  s_acc[wave][lane] = acc_a;
  s_acc[wave][lane + 64] = acc_b;
  __syncthreads();
  if (threadIdx.x < D) {
    const int e = threadIdx.x;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, s_m[w]);
    float St = 0.f, at = 0.f;
    if (Mt != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = s_m[w] == -INFINITY ? 0.f : __expf(s_m[w] - Mt);
        St += s_s[w] * f;
        at += s_acc[w][e] * f;
      }
    }
    o[row * D + e] = Mt == -INFINITY ? 0.f : at / St;
    if (e == 0) lse[row] = Mt == -INFINITY ? -INFINITY : Mt + __logf(St);
  }
}

// One workgroup per output row.  The row's P log-sum-exps and P x d partial outputs are
// requested together (one memory round trip for up to 128 parts per column block):
// thread (pg, c) of the 8 x 32 layout reads columns c, c+32, c+64, c+96 of parts
// pg, pg+8, ...; the parts' weights come from a workgroup max / sum of the lse's.
constexpr int kMergeThreads = 256;
constexpr int kMergeLse = 1024;            // lse's kept in LDS; later ones re-read

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const float *__restrict__ o_parts, const float *__restrict__ lse_parts, int P,
    int64_t rows, int d, float *__restrict__ o, float *__restrict__ lse) {
  __shared__ float s_lse[kMergeLse];
  __shared__ float s_red[kMergeThreads];
  __shared__ float s_acc[8][128];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int pg = t >> 5, c = t & 31;
  constexpr int PJ = 16;                   // parts per thread per pass

  // Issue the first pass of partial-output loads before reducing the lse's.
  float v[PJ][4];
  auto load_pass = [&](int pass, int e0) {
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      const int pp = pass * 8 * PJ + pg + 8 * j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + c + 32 * i;
        v[j][i] = (pp < P && e < d) ? o_parts[((int64_t)pp * rows + row) * d + e] : 0.f;
      }
    }
  };
  load_pass(0, 0);
  float m = -INFINITY;
  for (int pp = t; pp < P; pp += kMergeThreads) {
    const float x = lse_parts[(int64_t)pp * rows + row];
    if (pp < kMergeLse) s_lse[pp] = x;
    m = fmaxf(m, x);
  }
  s_red[t] = m;
  __syncthreads();
  for (int s = kMergeThreads / 2; s > 0; s >>= 1) {
    if (t < s) s_red[t] = fmaxf(s_red[t], s_red[t + s]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();
  float sum = 0.f;
  if (M != -INFINITY)
    for (int pp = t; pp < P; pp += kMergeThreads)
      sum += expf((pp < kMergeLse ? s_lse[pp] : lse_parts[(int64_t)pp * rows + row]) - M);
  s_red[t] = sum;
  __syncthreads();
  for (int s = kMergeThreads / 2; s > 0; s >>= 1) {
    if (t < s) s_red[t] += s_red[t + s];
    __syncthreads();
  }
  const float S = s_red[0];
  auto weight = [&](int pp) -> float {
    if (pp >= P || M == -INFINITY) return 0.f;
    const float x = pp < kMergeLse ? s_lse[pp] : lse_parts[(int64_t)pp * rows + row];
    return expf(x - M);
  };
  const int passes = (P + 8 * PJ - 1) / (8 * PJ);
  for (int e0 = 0; e0 < d; e0 += 128) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int pass = 0; pass < passes; ++pass) {
      if (pass > 0 || e0 > 0) load_pass(pass, e0);
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        const float w = weight(pass * 8 * PJ + pg + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, v[j][i], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[pg][c + 32 * i] = acc[i];
    __syncthreads();
    if (t < 128 && e0 + t < d) {
      float a = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) a += s_acc[g][t];
      o[row * d + e0 + t] = M == -INFINITY ? 0.f : a / S;
    }
    __syncthreads();
  }
  if (t == 0) lse[row] = M == -INFINITY ? -INFINITY : M + logf(S);
}

// Attention over empty sets: o = 0, lse = -inf for every row (reads nothing).
__global__ __launch_bounds__(256) void empty_rows_kernel(int64_t rows, int d, float *__restrict__ o,
                                                         float *__restrict__ lse) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < rows * d) o[i] = 0.f;
  if (i < rows) lse[i] = -INFINITY;
}

template <bool BF16, int G>
void decode_launch(const DecodePlan &pl, const void *q, const void *k, const void *v, int B,
                   int Hq, int Hkv, int64_t cap, const int32_t *idx, int64_t idx_stride,
                   const int32_t *count, int max_count, float scale_log2, float *o_dst,
                   float *lse_dst, int kv_group, hipStream_t st) {
  hipLaunchKernelGGL((sparse_decode_kernel<BF16, G>), dim3(pl.P, B * Hkv), dim3(kAttThreads),
                     0, st, q, k, v, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                     pl.rows_per_split, scale_log2, o_dst, lse_dst, (int64_t)B * Hq, kv_group);
}

template <bool BF16>
void decode_dispatch(const DecodePlan &pl, const void *q, const void *k, const void *v, int B,
                     int Hq, int Hkv, int64_t cap, const int32_t *idx, int64_t idx_stride,
                     const int32_t *count, int max_count, float scale_log2, float *o_dst,
                     float *lse_dst, int kv_group, hipStream_t st) {
#define HK_DEC_CASE(GG)                                                                    \
  case GG:                                                                                 \
    decode_launch<BF16, GG>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count,          \
                            max_count, scale_log2, o_dst, lse_dst, kv_group, st);          \
    break;
  switch (pl.G) {
    HK_DEC_CASE(1) HK_DEC_CASE(2) HK_DEC_CASE(3) HK_DEC_CASE(4)
    HK_DEC_CASE(5) HK_DEC_CASE(6) HK_DEC_CASE(7) HK_DEC_CASE(8)
    default: break;
  }
#undef HK_DEC_CASE
}

}  // namespace

DecodePlan plan_decode(int B, int Hq, int Hkv, int max_count) {
  DecodePlan p;
  p.G = Hkv > 0 ? Hq / Hkv : 1;
  const int64_t BH = (int64_t)B * Hkv;
  const int mc = max_count > 0 ? max_count : 1;
  // Slices of 64, 128 or 256 rows: the smallest that keeps the grid near 1024
  // workgroups.  Short slices finish in two memory round trips (indices, then rows);
  // long ones amortise the (G x d) partial each slice writes.
  int rps = 256;
  for (int cand : {64, 128, 256}) {
    if (BH * ((mc + cand - 1) / cand) <= 1024) {
      rps = cand;
      break;
    }
  }
  p.rows_per_split = rps < mc ? rps : mc;
  p.P = (mc + p.rows_per_split - 1) / p.rows_per_split;
  size_t off = 0;
  if (p.P > 1) {
    const size_t rows = (size_t)B * Hq;
    p.off_o = off;
    off = align_up(off + (size_t)p.P * rows * kHeadDim * sizeof(float), 256);
    p.off_lse = off;
    off = align_up(off + (size_t)p.P * rows * sizeof(float), 256);
  }
  p.total = off;
  return p;
}

hipError_t launch_sparse_decode(const DecodePlan &pl, const void *q, const void *k,
                                const void *v, int dtype, int B, int Hq, int Hkv,
                                int64_t cap, const int32_t *idx, int64_t idx_stride,
                                const int32_t *count, int max_count, float scale, float *o,
                                float *lse, void *ws, hipStream_t st, int kv_group) {
  if ((int64_t)B * Hq == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  float *o_dst = pl.P > 1 ? reinterpret_cast<float *>(w8 + pl.off_o) : o;
  float *lse_dst = pl.P > 1 ? reinterpret_cast<float *>(w8 + pl.off_lse) : lse;
  if (dtype == HK_BF16)
    decode_dispatch<true>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                          scale_log2, o_dst, lse_dst, kv_group, st);
  else
    decode_dispatch<false>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                           scale_log2, o_dst, lse_dst, kv_group, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.P == 1) return e;
  return launch_lse_merge(o_dst, lse_dst, pl.P, (int64_t)B * Hq, kHeadDim, o, lse, st);
}

hipError_t launch_lse_merge_parts(const float *o_parts, const float *lse_parts, int P,
                                  int64_t rows, int d, float *o, float *lse, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (P == 0) {
    // No partial exists (and no partial space was reserved): every row is the empty set.
    hipLaunchKernelGGL(empty_rows_kernel, dim3((unsigned)((rows * d + 255) / 256)), dim3(256), 0,
                       st, rows, d, o, lse);
    return hipGetLastError();
  }
  return launch_lse_merge(o_parts, lse_parts, P, rows, d, o, lse, st);
}

hipError_t launch_lse_merge(const float *o_parts, const float *lse_parts, int P,
                            int64_t rows, int d, float *o, float *lse, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (P < 1) return hipErrorInvalidValue;      // the merge kernels read part 0 .. P-1
  if (P <= kMergeSmallParts && d == kHeadDim) {
    hipLaunchKernelGGL(lse_merge_small_kernel, dim3((unsigned)rows), dim3(256), 0, st,
                       o_parts, lse_parts, P, rows, o, lse);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, st,
                     o_parts, lse_parts, P, rows, d, o, lse);
  return hipGetLastError();
}

}  // namespace hk
