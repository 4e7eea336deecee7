// Exact softmax attention restricted to a token list, and the log-sum-exp merge.
//
// Attention over the retrieved tokens only ("partial attention": RetrievalAttention,
// elamur summary: Summary; Spotlight Attention: summary) and over the static sink +
// local window, combined by exact log-sum-exp rescaling (RetrievalAttention, atlas
// summary: Approach).
//
// sparse_decode: one workgroup gathers one slice of one (batch, KV head)'s token list.
// A 16-lane quarter-wave owns one K/V row at a time: each lane loads 8 consecutive
// elements (16 bytes of bf16, 32 bytes of fp32), so a row of 128 is one coalesced
// 256- or 512-byte read.  The row is loaded once and scored against all G query heads
// of the GQA group (the K/V bytes are shared across the group).  Scores reduce across
// the 16 lanes with DPP row rotations; softmax is online in fp32 with base-2
// exponentials; each quarter-wave keeps its own running (max, sum, output) and the 16
// quarter-waves of the workgroup combine at the end.  Rows are independent, so several
// are kept in flight per quarter-wave to cover HBM latency.  The kernel is bound by HBM
// bandwidth: 2*d*sizeof(elem) bytes per row against 4*d*G flops.
#include "hk_internal.h"

namespace hk {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;           // rows in flight per quarter-wave
constexpr int kQuarterWaves = kDecThreads / 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ __forceinline__ float row_rotate(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += row_rotate<0x128>(v);  // row_ror:8
  v += row_rotate<0x124>(v);  // row_ror:4
  v += row_rotate<0x122>(v);  // row_ror:2
  v += row_rotate<0x121>(v);  // row_ror:1
  return v;
}

template <bool BF16> struct Row8;
template <> struct Row8<true> {       // 8 bf16 = 16 bytes
  using Raw = uint4;
  __device__ static Raw load(const void *base, size_t elem) {
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
  }
  __device__ static Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
  __device__ static void widen(const Raw &r, float *f) {
    f[0] = __uint_as_float(r.x << 16); f[1] = __uint_as_float(r.x & 0xFFFF0000u);
    f[2] = __uint_as_float(r.y << 16); f[3] = __uint_as_float(r.y & 0xFFFF0000u);
    f[4] = __uint_as_float(r.z << 16); f[5] = __uint_as_float(r.z & 0xFFFF0000u);
    f[6] = __uint_as_float(r.w << 16); f[7] = __uint_as_float(r.w & 0xFFFF0000u);
  }
};
template <> struct Row8<false> {      // 8 fp32 = 32 bytes
  struct Raw { float4 a, b; };
  __device__ static Raw load(const void *base, size_t elem) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
    return Raw{p[0], p[1]};
  }
  __device__ static Raw zero() { return Raw{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)}; }
  __device__ static void widen(const Raw &r, float *f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
    f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
};

// grid (P, B*Hkv).  Writes either the final (o, lse) of its query heads (P == 1) or the
// normalised partial of slice p into out_o + p*rows*d, out_lse + p*rows.
template <bool BF16, int G>
__global__ __launch_bounds__(kDecThreads) void sparse_decode_kernel(
    const void *__restrict__ q, const void *__restrict__ kc, const void *__restrict__ vc,
    int Hq, int Hkv, int64_t cap, const int32_t *__restrict__ idx, int64_t idx_stride,
    const int32_t *__restrict__ count, int max_count, int rows_per_split, float scale_log2,
    float *__restrict__ out_o, float *__restrict__ out_lse, int64_t rows) {
  using RL = Row8<BF16>;
  constexpr int D = kHeadDim;
  __shared__ float s_m[kDecThreads / 64][G];
  __shared__ float s_l[kDecThreads / 64][G];
  __shared__ float s_o[kDecThreads / 64][G][D];

  const int p = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int hkv = bh - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int qw = wave * 4 + (lane >> 4);

  int n = count ? count[bh] : max_count;
  n = n < 0 ? 0 : (n > max_count ? max_count : n);
  const int r0 = p * rows_per_split;
  const int r1 = min(n, r0 + rows_per_split);

  float qf[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t qe = ((size_t)b * Hq + (size_t)hkv * G + g) * D + col * 8;
    RL::widen(RL::load(q, qe), qf[g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[g][e] *= scale_log2;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // Rows of this quarter-wave: r0 + qw + 16*j.  Lane col of the quarter-wave fetches the
  // token index of row j = 16*blk + col for a block of 16 rows at a time, and the rows'
  // indices are then broadcast within the quarter-wave.  K/V rows are loaded four at a
  // time, one group ahead of the group being reduced.
  const int32_t *ilist = idx + (int64_t)bh * idx_stride;
  const size_t head_row0 = (size_t)bh * (size_t)cap;
  const int nrows = r1 > r0 + qw ? (r1 - r0 - qw + kQuarterWaves - 1) / kQuarterWaves : 0;
  const int qlane0 = lane & ~15;
  auto fetch_tokens = [&](int blk) -> int {
    const int j = blk * 16 + col;
    return j < nrows ? ilist[r0 + qw + kQuarterWaves * j] : 0;
  };
  auto load_group = [&](int grp, int toks, typename RL::Raw *kr, typename RL::Raw *vr) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = grp * kDecUnroll + u;
      const int tok = __shfl(toks, qlane0 + (j & 15));
      const bool ok = j < nrows;
      const size_t e0 = (head_row0 + (size_t)(ok ? tok : 0)) * D + col * 8;
      kr[u] = ok ? RL::load(kc, e0) : RL::zero();
      vr[u] = ok ? RL::load(vc, e0) : RL::zero();
    }
  };
  const int ngroups = (nrows + kDecUnroll - 1) / kDecUnroll;
  int toks = fetch_tokens(0);
  typename RL::Raw kr[kDecUnroll], vr[kDecUnroll];
  if (ngroups > 0) load_group(0, toks, kr, vr);
  for (int grp = 0; grp < ngroups; ++grp) {
    // Prefetch the next group (and the next 16 indices when this block of 16 is used up).
    typename RL::Raw kn[kDecUnroll], vn[kDecUnroll];
    const int ngrp = grp + 1;
    int toks_n = toks;
    if ((ngrp & 3) == 0 && ngrp < ngroups) toks_n = fetch_tokens(ngrp >> 2);
    if (ngrp < ngroups) load_group(ngrp, toks_n, kn, vn);

    float s[G][kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float kf[8];
      RL::widen(kr[u], kf);
      const bool ok = grp * kDecUnroll + u < nrows;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qf[g][e], kf[e], a);
        a = row16_sum(a);
        s[g][u] = ok ? a : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = s[g][0];
#pragma unroll
      for (int u = 1; u < kDecUnroll; ++u) mx = fmaxf(mx, s[g][u]);
      const float mn = fmaxf(m[g], mx);        // finite: row 0 of a group is always valid
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        s[g][u] = __builtin_amdgcn_exp2f(s[g][u] - mn);   // now the weight of row u
        psum += s[g][u];
      }
      l[g] = l[g] * alpha + psum;
      m[g] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float vf[8];
      RL::widen(vr[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(s[g][u], vf[e], acc[g][e]);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      kr[u] = kn[u];
      vr[u] = vn[u];
    }
    toks = toks_n;
  }

  // Combine the four quarter-waves of this wave (lanes col, col+16, col+32, col+48).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mw = fmaxf(m[g], __shfl_xor(m[g], 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - mw);
    float lw = l[g] * f;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc[g][e] * f;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[g][e] = a;
    }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][g][col * 8 + e] = acc[g][e];
    }
    if (lane == 0) {
      s_m[wave][g] = mw;
      s_l[wave][g] = lw;
    }
  }
  __syncthreads();

  // Combine the waves; thread t handles output elements t, t + 256, ... of G*D.
  for (int i = threadIdx.x; i < G * D; i += kDecThreads) {
    const int g = i / D, e = i - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecThreads / 64; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
        L += s_l[w][g] * f;
        O += s_o[w][g][e] * f;
      }
    }
    const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
    const int64_t prow = (int64_t)p * rows + row;
    const bool empty = !(L > 0.f);
    out_o[prow * D + e] = empty ? 0.f : O / L;
    if (e == 0) out_lse[prow] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
  }
}

// One wavefront per row.  Phase 1: the lanes read the P log-sum-exps at once (max and
// normaliser by wavefront reductions).  Phase 2: each lane accumulates its output
// elements over the parts, eight parts of loads in flight at a time.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float *__restrict__ o_parts, const float *__restrict__ lse_parts, int P,
    int64_t rows, int d, float *__restrict__ o, float *__restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int p = lane; p < P; p += 64) m = fmaxf(m, lse_parts[(int64_t)p * rows + row]);
  m = wave_max(m);
  if (m == -INFINITY) {
    for (int e = lane; e < d; e += 64) o[row * d + e] = 0.f;
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float ssum = 0.f;
  for (int p = lane; p < P; p += 64) ssum += expf(lse_parts[(int64_t)p * rows + row] - m);
  ssum = wave_sum(ssum);
  const float inv = 1.f / ssum;
  constexpr int PB = 8;
  for (int e0 = 0; e0 < d; e0 += 128) {
    const int ea = e0 + lane, eb = e0 + 64 + lane;
    float acc_a = 0.f, acc_b = 0.f;
    for (int p0 = 0; p0 < P; p0 += PB) {
      float la[PB], va[PB], vb[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int p = p0 + j;
        const bool ok = p < P;
        const float *op = o_parts + ((int64_t)(ok ? p : 0) * rows + row) * d;
        la[j] = ok ? lse_parts[(int64_t)p * rows + row] : -INFINITY;
        va[j] = (ok && ea < d) ? op[ea] : 0.f;
        vb[j] = (ok && eb < d) ? op[eb] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const float w = expf(la[j] - m);
        acc_a = fmaf(w, va[j], acc_a);
        acc_b = fmaf(w, vb[j], acc_b);
      }
    }
    if (ea < d) o[row * d + ea] = acc_a * inv;
    if (eb < d) o[row * d + eb] = acc_b * inv;
  }
  if (lane == 0) lse[row] = m + logf(ssum);
}

template <bool BF16, int G>
void decode_launch(const DecodePlan &pl, const void *q, const void *k, const void *v, int B,
                   int Hq, int Hkv, int64_t cap, const int32_t *idx, int64_t idx_stride,
                   const int32_t *count, int max_count, float scale_log2, float *o_dst,
                   float *lse_dst, hipStream_t st) {
  hipLaunchKernelGGL((sparse_decode_kernel<BF16, G>), dim3(pl.P, B * Hkv), dim3(kDecThreads),
                     0, st, q, k, v, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                     pl.rows_per_split, scale_log2, o_dst, lse_dst, (int64_t)B * Hq);
}

template <bool BF16>
void decode_dispatch(const DecodePlan &pl, const void *q, const void *k, const void *v, int B,
                     int Hq, int Hkv, int64_t cap, const int32_t *idx, int64_t idx_stride,
                     const int32_t *count, int max_count, float scale_log2, float *o_dst,
                     float *lse_dst, hipStream_t st) {
#define HK_DEC_CASE(GG)                                                                    \
  case GG:                                                                                 \
    decode_launch<BF16, GG>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count,          \
                            max_count, scale_log2, o_dst, lse_dst, st);                    \
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
                                float *lse, void *ws, hipStream_t st) {
  if ((int64_t)B * Hq == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  float *o_dst = pl.P > 1 ? reinterpret_cast<float *>(w8 + pl.off_o) : o;
  float *lse_dst = pl.P > 1 ? reinterpret_cast<float *>(w8 + pl.off_lse) : lse;
  if (dtype == HK_BF16)
    decode_dispatch<true>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                          scale_log2, o_dst, lse_dst, st);
  else
    decode_dispatch<false>(pl, q, k, v, B, Hq, Hkv, cap, idx, idx_stride, count, max_count,
                           scale_log2, o_dst, lse_dst, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.P == 1) return e;
  return launch_lse_merge(o_dst, lse_dst, pl.P, (int64_t)B * Hq, kHeadDim, o, lse, st);
}

hipError_t launch_lse_merge(const float *o_parts, const float *lse_parts, int P,
                            int64_t rows, int d, float *o, float *lse, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     o_parts, lse_parts, P, rows, d, o, lse);
  return hipGetLastError();
}

}  // namespace hk
