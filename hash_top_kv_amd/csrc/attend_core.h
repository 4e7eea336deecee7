// Device core of exact softmax attention over a token list, shared by the sparse-decode
// kernel and the fused retrieve-and-attend kernel.
//
// A workgroup of 256 threads is 16 quarter-waves of 16 lanes.  A quarter-wave owns one
// K/V row at a time: each lane holds 8 consecutive elements (16 bytes of bf16 or 32 of
// fp32), so a row of 128 is one coalesced read.  Each row is scored against all G query
// heads of the GQA group (its bytes are shared by the group); scores reduce across the
// 16 lanes with DPP row rotations; softmax is online in fp32 with base-2 exponentials.
// Rows are loaded four at a time, one group of four ahead of the group being reduced,
// and token indices arrive 16 at a time (one per lane) and are broadcast in the
// quarter-wave.  At the end the 16 quarter-wave states of the workgroup combine into one
// normalised (o, lse) per query head.
#pragma once

#include "hk_internal.h"

namespace hk {

constexpr int kAttThreads = 256;
constexpr int kAttUnroll = 4;                       // rows in flight per quarter-wave
constexpr int kQuarterWaves = kAttThreads / 16;
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

// Per-lane state of the G query heads of one group.
template <bool BF16, int G>
struct GroupAttention {
  using RL = Row8<BF16>;
  static constexpr int D = kHeadDim;
  float qf[G][8];
  float m[G], l[G], acc[G][8];

  // q [B][Hq][D]; query heads row0 .. row0 + G - 1 (row0 = b*Hq + hkv*G).
  __device__ void init(const void *q, int64_t row0, float scale_log2) {
    const int col = threadIdx.x & 15;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      RL::widen(RL::load(q, (size_t)(row0 + g) * D + col * 8), qf[g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[g][e] *= scale_log2;
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }
  }

  // This quarter-wave's rows j = 0 .. nrows-1; fetch(j) returns the token of row j and
  // is called by lane (j % 16) of the quarter-wave for each block of 16 rows.  Rows of
  // head `head_row0` (= b*Hkv + hkv) * cap) of kc / vc.
  template <class Fetch>
  __device__ void run(const void *kc, const void *vc, size_t head_row0, int nrows, Fetch fetch) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int qlane0 = lane & ~15;
    auto fetch_block = [&](int blk) -> int {
      const int j = blk * 16 + col;
      return j < nrows ? fetch(j) : 0;
    };
    auto load_group = [&](int grp, int toks, typename RL::Raw *kr, typename RL::Raw *vr) {
#pragma unroll
      for (int u = 0; u < kAttUnroll; ++u) {
        const int j = grp * kAttUnroll + u;
        const int tok = __shfl(toks, qlane0 + (j & 15));
        const bool ok = j < nrows;
        const size_t e0 = (head_row0 + (size_t)(ok ? tok : 0)) * D + col * 8;
        kr[u] = ok ? RL::load(kc, e0) : RL::zero();
        vr[u] = ok ? RL::load(vc, e0) : RL::zero();
      }
    };
    const int ngroups = (nrows + kAttUnroll - 1) / kAttUnroll;
    int toks = fetch_block(0);
    typename RL::Raw kr[kAttUnroll], vr[kAttUnroll];
    if (ngroups > 0) load_group(0, toks, kr, vr);
    for (int grp = 0; grp < ngroups; ++grp) {
      typename RL::Raw kn[kAttUnroll], vn[kAttUnroll];
      const int ngrp = grp + 1;
      int toks_n = toks;
      if ((ngrp & 3) == 0 && ngrp < ngroups) toks_n = fetch_block(ngrp >> 2);
      if (ngrp < ngroups) load_group(ngrp, toks_n, kn, vn);

      float s[G][kAttUnroll];
#pragma unroll
      for (int u = 0; u < kAttUnroll; ++u) {
        float kf[8];
        RL::widen(kr[u], kf);
        const bool ok = grp * kAttUnroll + u < nrows;
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
        for (int u = 1; u < kAttUnroll; ++u) mx = fmaxf(mx, s[g][u]);
        const float mn = fmaxf(m[g], mx);      // finite: row 0 of a group is always valid
        const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < kAttUnroll; ++u) {
          s[g][u] = __builtin_amdgcn_exp2f(s[g][u] - mn);   // now the weight of row u
          psum += s[g][u];
        }
        l[g] = l[g] * alpha + psum;
        m[g] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < kAttUnroll; ++u) {
        float vf[8];
        RL::widen(vr[u], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(s[g][u], vf[e], acc[g][e]);
        }
      }
#pragma unroll
      for (int u = 0; u < kAttUnroll; ++u) {
        kr[u] = kn[u];
        vr[u] = vn[u];
      }
      toks = toks_n;
    }
  }

  // Combine the 16 quarter-waves and store the normalised o (G rows of D at out_o) and
  // natural-log lse (G values at out_lse).  An empty set stores o = 0, lse = -inf.
  // Called by all 256 threads of the workgroup.
  __device__ void combine_store(float *out_o, float *out_lse) {
    __shared__ float s_m[kAttThreads / 64][G];
    __shared__ float s_l[kAttThreads / 64][G];
    __shared__ float s_o[kAttThreads / 64][G][D];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
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
    for (int i = threadIdx.x; i < G * D; i += kAttThreads) {
      const int g = i / D, e = i - g * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttThreads / 64; ++w) M = fmaxf(M, s_m[w][g]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAttThreads / 64; ++w) {
          const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
          L += s_l[w][g] * f;
          O += s_o[w][g][e] * f;
        }
      }
      const bool empty = !(L > 0.f);
      out_o[(size_t)g * D + e] = empty ? 0.f : O / L;
      if (e == 0) out_lse[g] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
  }
};

}  // namespace hk
