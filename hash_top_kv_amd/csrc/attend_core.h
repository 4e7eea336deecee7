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

// Query fragments and partial dot products.  bf16: the query stays packed (its values
// are exact in bf16) and each lane's 8-element partial dot product is four
// v_dot2c_f32_bf16 (exact products, fp32 accumulation) on the raw K words; fp32: the
// query and the row are fp32.  The softmax scale is applied to the reduced dot product.
template <bool BF16, int G> struct QueryFrag;
template <int G> struct QueryFrag<true, G> {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  uint32_t qp[G][4];
  __device__ void load(const void *q, int64_t row0, int col) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 r = Row8<true>::load(q, (size_t)(row0 + g) * kHeadDim + col * 8);
      qp[g][0] = r.x; qp[g][1] = r.y; qp[g][2] = r.z; qp[g][3] = r.w;
    }
  }
  __device__ float dot(int g, const uint4 &k) const {
    float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[g][0]),
                                              __builtin_bit_cast(bf16x2, k.x), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[g][1]),
                                        __builtin_bit_cast(bf16x2, k.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[g][2]),
                                        __builtin_bit_cast(bf16x2, k.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[g][3]),
                                        __builtin_bit_cast(bf16x2, k.w), a, false);
    return a;
  }
};
template <int G> struct QueryFrag<false, G> {
  float qf[G][8];
  __device__ void load(const void *q, int64_t row0, int col) {
#pragma unroll
    for (int g = 0; g < G; ++g) Row8<false>::widen(Row8<false>::load(q, (size_t)(row0 + g) * kHeadDim + col * 8), qf[g]);
  }
  __device__ float dot(int g, const Row8<false>::Raw &k) const {
    float kf[8];
    Row8<false>::widen(k, kf);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf(qf[g][e], kf[e], a);
    return a;
  }
};

// The last step of both cores' combine_store.  s_m, s_l and s_o hold each wavefront's
// running maximum (base 2), normaliser and unnormalised output per query head.  For each
// output element: M = max over wavefronts, weights 2^(m_w - M), o = (sum over
// wavefronts, in order, of weight * o_w) / L, lse = (M + log2 L) ln 2; an empty set
// gives o = 0, lse = -inf.  When the G x D outputs fit in one pass of the workgroup
// (G <= 2) each thread takes one element; for larger groups each thread takes four
// consecutive dims of one head, read from LDS and stored to out_o 16 bytes at a time
// (element by element when out_o is not 16-byte aligned), which needs a quarter of the
// passes and of the LDS reads of the weights.  Both give the same values.
template <int G>
__device__ __forceinline__ void combine_waves(const float (*s_m)[G], const float (*s_l)[G],
                                              const float (*s_o)[G][kHeadDim], float *out_o,
                                              float *out_lse) {
  constexpr int D = kHeadDim, NW = kAttThreads / 64, V = D / 4;
  if constexpr (G * D <= kAttThreads) {
    const int i = threadIdx.x;
    if (i < G * D) {
      const int h = i / D, e = i - h * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
          L += s_l[w][h] * f;
          O += s_o[w][h][e] * f;
        }
      }
      const bool empty = !(L > 0.f);
      out_o[(size_t)h * D + e] = empty ? 0.f : O / L;
      if (e == 0) out_lse[h] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
  } else {
    const bool vec = (reinterpret_cast<uintptr_t>(out_o) & 15u) == 0;
    for (int i = threadIdx.x; i < G * V; i += kAttThreads) {
      const int h = i / V, e = 4 * (i - h * V);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
      float L = 0.f;
      float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
          L += s_l[w][h] * f;
          const float4 v = *reinterpret_cast<const float4 *>(&s_o[w][h][e]);
          O.x += v.x * f;
          O.y += v.y * f;
          O.z += v.z * f;
          O.w += v.w * f;
        }
      }
      const bool empty = !(L > 0.f);
      const float4 r = empty ? make_float4(0.f, 0.f, 0.f, 0.f)
                             : make_float4(O.x / L, O.y / L, O.z / L, O.w / L);
      float *dst = out_o + (size_t)h * D + e;
      if (vec) {
        *reinterpret_cast<float4 *>(dst) = r;
      } else {
        dst[0] = r.x;
        dst[1] = r.y;
        dst[2] = r.z;
        dst[3] = r.w;
      }
      if (e == 0) out_lse[h] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
  }
}

// Per-lane state of the G query heads of one group.
template <bool BF16, int G>
struct GroupAttention {
  using RL = Row8<BF16>;
  static constexpr int D = kHeadDim;
  QueryFrag<BF16, G> qfrag;
  float scale_log2;
  float m[G], l[G], acc[G][8];

  // q [B][Hq][D]; query heads row0 .. row0 + G - 1 (row0 = b*Hq + hkv*G).
  __device__ void init(const void *q, int64_t row0, float sl2) {
    const int col = threadIdx.x & 15;
    qfrag.load(q, row0, col);
    scale_log2 = sl2;
#pragma unroll
    for (int g = 0; g < G; ++g) {
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
        const bool ok = grp * kAttUnroll + u < nrows;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float a = row16_sum(qfrag.dot(g, kr[u])) * scale_log2;
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

  // The workgroup's rows 0 .. len-1, fetch_row(r) giving the token of row r: quarter-wave
  // qw takes rows qw, qw + 16, ...
  template <class FetchRow>
  __device__ void run_block(const void *kc, const void *vc, size_t head_row0, int len,
                            FetchRow fetch_row) {
    const int qw = threadIdx.x >> 4;
    const int nrows = len > qw ? (len - qw + kQuarterWaves - 1) / kQuarterWaves : 0;
    run(kc, vc, head_row0, nrows, [&](int j) { return fetch_row(qw + kQuarterWaves * j); });
  }

  // Combine the 16 quarter-waves and store the normalised o (G rows of D at out_o) and
  // natural-log lse (G values at out_lse).  An empty set stores o = 0, lse = -inf.
  // Called by all 256 threads of the workgroup.
  __device__ void combine_store(float *out_o, float *out_lse) {
    __shared__ float s_m[kAttThreads / 64][G];
    __shared__ float s_l[kAttThreads / 64][G];
    __shared__ __attribute__((aligned(16))) float s_o[kAttThreads / 64][G][D];
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
        float4 *dst = reinterpret_cast<float4 *>(&s_o[wave][g][col * 8]);
        dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
        dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
      }
      if (lane == 0) {
        s_m[wave][g] = mw;
        s_l[wave][g] = lw;
      }
    }
    __syncthreads();
    combine_waves<G>(s_m, s_l, s_o, out_o, out_lse);
  }
};

// ------------------------------------------------------------------ matrix-core variant
// bf16 rows, G <= 16 query heads: per wavefront, tiles of 16 rows.
//   scores  S^T[16 rows][16 heads] = K_tile . Q^T with four v_mfma_f32_16x16x32_bf16; lane l
//           loads 16 bytes of row (l % 16) per k-step (dims 32*ks + 8*(l/16) .., so the four
//           lanes of a row read 64 contiguous bytes per load instruction), and holds
//           the scores of head l % 16 for rows 4*(l/16) .. +3 -- which is already the
//           A-operand layout of P for the second product, so no transpose is needed.
//   output  O[16 heads][dims] += P . V_tile with eight v_mfma_f32_16x16x16_bf16, one per
//           output dim t of 8*(l % 16) + t: lane l loads bytes 16*(l % 16) .. +15 of rows
//           4*(l/16) .. +3 (each row read whole and coalesced by 16 lanes), and v_perm
//           pairs element t of two rows into the B operand.
// Softmax is online in base 2 with a lazy maximum: the running max moves (and O is
// rescaled) only when a tile's max exceeds it by more than 8, so weights stay <= 2^8.
// P enters the product rounded to bf16 and the normaliser sums the same rounded values.
template <int G>
struct GroupAttentionMfma {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  static constexpr int D = kHeadDim;
  static constexpr float kLazy = 8.f;
  bf16x8 qb[4];
  float scale_log2, m, l;
  f32x4 o[8];

  __device__ void init(const void *q, int64_t row0, float sl2) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    const uint16_t *qp = static_cast<const uint16_t *>(q) + (size_t)(row0 + n) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = n < G ? *reinterpret_cast<const uint4 *>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
      qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
    scale_log2 = sl2;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct Tile {
    uint4 k[4], v[4];
  };

  template <class FetchRow>
  __device__ void run_block(const void *kc, const void *vc, size_t head_row0, int len,
                            FetchRow fetch_row) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int ntiles = (len + 15) >> 4;
    const uint16_t *kb = static_cast<const uint16_t *>(kc);
    const uint16_t *vb = static_cast<const uint16_t *>(vc);
    auto load_tile = [&](int tile, Tile &T) {
      const int r0 = tile * 16;
      const int tok = r0 + n < len ? fetch_row(r0 + n) : 0;
      const bool okk = r0 + n < len;
      const uint16_t *kp = kb + (head_row0 + (size_t)tok) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        T.k[ks] = okk ? *reinterpret_cast<const uint4 *>(kp + 32 * ks) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tv = __shfl(tok, 4 * g + j);
        const bool okv = r0 + 4 * g + j < len;
        T.v[j] = okv ? *reinterpret_cast<const uint4 *>(vb + (head_row0 + (size_t)tv) * D + 8 * n)
                     : make_uint4(0, 0, 0, 0);
      }
    };
    Tile cur, nxt;
    if (wave < ntiles) load_tile(wave, cur);
    for (int tile = wave; tile < ntiles; tile += kAttThreads / 64) {
      if (tile + kAttThreads / 64 < ntiles) load_tile(tile + kAttThreads / 64, nxt);
      // scores of head n, rows 4g .. 4g+3 of the tile
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[ks]), qb[ks], sc, 0, 0, 0);
      float s[4];
      const int rb = tile * 16 + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = rb + j < len ? sc[j] * scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m + kLazy;                 // also the first valid tile
      if (__ballot(need)) {
        const float mn = need ? mx : m;
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
        l *= alpha;
        m = mn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * g + j);     // alpha of head 4g + j
#pragma unroll
          for (int t = 0; t < 8; ++t) o[t][j] *= aj;
        }
      }
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = s[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[j] - m);
      const bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]};
      const bf16x2 p23 = {(__bf16)p[2], (__bf16)p[3]};
      const uint32_t w01 = __builtin_bit_cast(uint32_t, p01), w23 = __builtin_bit_cast(uint32_t, p23);
      l += __uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xFFFF0000u) +
           __uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xFFFF0000u);
      const s16x4 pa = __builtin_bit_cast(s16x4, uint2{w01, w23});
      const uint32_t *v0 = reinterpret_cast<const uint32_t *>(&cur.v[0]);
      const uint32_t *v1 = reinterpret_cast<const uint32_t *>(&cur.v[1]);
      const uint32_t *v2 = reinterpret_cast<const uint32_t *>(&cur.v[2]);
      const uint32_t *v3 = reinterpret_cast<const uint32_t *>(&cur.v[3]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t a = __builtin_amdgcn_perm(v1[t >> 1], v0[t >> 1], sel);
        const uint32_t b = __builtin_amdgcn_perm(v3[t >> 1], v2[t >> 1], sel);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, uint2{a, b}), o[t], 0, 0, 0);
      }
      cur = nxt;
    }
  }

  __device__ void combine_store(float *out_o, float *out_lse) {
    __shared__ float s_m[kAttThreads / 64][G];
    __shared__ float s_l[kAttThreads / 64][G];
    __shared__ __attribute__((aligned(16))) float s_o[kAttThreads / 64][G][D];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0 && n < G) {
      s_m[wave][n] = m;
      s_l[wave][n] = lt;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * g + j;
      if (h < G) {
        float4 *dst = reinterpret_cast<float4 *>(&s_o[wave][h][8 * n]);
        dst[0] = make_float4(o[0][j], o[1][j], o[2][j], o[3][j]);
        dst[1] = make_float4(o[4][j], o[5][j], o[6][j], o[7][j]);
      }
    }
    __syncthreads();
    combine_waves<G>(s_m, s_l, s_o, out_o, out_lse);
  }
};

// The attention core used for an element type: matrix cores for bf16, VALU for fp32.
template <bool BF16, int G> struct AttentionCore { using type = GroupAttention<false, G>; };
template <int G> struct AttentionCore<true, G> { using type = GroupAttentionMfma<G>; };

}  // namespace hk
