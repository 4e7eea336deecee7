// Encoder arithmetic shared by the key and query encoders (encode.hip) and by the scan
// that hashes its head's query itself (retrieve.hip): element loads, the GELU, bf16
// rounding, and the group-mean query code computed by one 256-thread workgroup.
#pragma once
#include "hk_internal.h"

namespace hk {
namespace enc {

// GELU(a) = a Phi(a) = max(a, 0) - x Phi(-x) with x = |a|, and Phi(-x) = 2^R(x): R is a
// degree-5 polynomial fitted to log2 Phi(-x) (a weighted minimax fit that bounds the
// absolute error of x 2^R(x), not of R).  Evaluated in fp32 (Horner, then one base-2
// exponential), |GELU - exact| <= 4.6e-7 above fp32 rounding of the result, for every
// finite a.  R's leading coefficient is negative, so R falls without bound: from x ~ 12
// on, 2^R is below 2^-140 and GELU(a) = max(a, 0) to fp32 precision, with no clamp; for
// very large x the Horner sum reaches -inf and the exponential 0 (never NaN).  Five
// fused multiply-adds, one exponential, one integer max (a negative float, -0 included,
// is a negative integer) and one fused multiply-add: eight vector instructions, one of
// them transcendental.  The fit is written out, with its check, in gelu_fit.py.
constexpr float kGelu0 = -1.000037722e+00f, kGelu1 = -1.150787181e+00f,
                kGelu2 = -4.599939130e-01f, kGelu3 = -5.182606418e-02f,
                kGelu4 = 7.084052480e-03f, kGelu5 = -4.732408280e-04f;
__device__ __forceinline__ float gelu(float a) {
  const float x = fabsf(a);
  float r = fmaf(kGelu5, x, kGelu4);
  r = fmaf(r, x, kGelu3);
  r = fmaf(r, x, kGelu2);
  r = fmaf(r, x, kGelu1);
  r = fmaf(r, x, kGelu0);
  const float g = __builtin_amdgcn_exp2f(r);
  return fmaf(-x, g, __int_as_float(max(__float_as_int(a), 0)));   // max(a, 0)
}

// Round to the nearest bf16 (ties to even); finite inputs.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(bf16_bits(f) << 16);
}

template <bool BF16>
__device__ __forceinline__ float elem(const void *p, size_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
  else
    return static_cast<const float *>(p)[i];
}

struct HashPtrs {
  const void *R, *W1, *b1, *W2, *b2;
};

// The code of the group-mean query of (batch b, KV head hg), computed by the 256
// threads of one workgroup in fp32 with the arithmetic of the fp32 query encoder, step
// for step: the mean sums the G query rows in order (zeros padding to 8 rows) and
// divides by G; a projection or hidden unit is one fused multiply-add chain over the
// 128 dimensions in order; the MLP's hidden activation is GELU(a + b1), rounded to bf16
// for bf16 hashes; an MLP output sums each half of its 256 hidden units in order, the
// halves then added as (first + (second + b2)).  LSH: bit j = [R_j . x > 0]; SIGN: bit
// j = [x_j > 0].  The words go to qw[BITS / 32] in LDS, valid for every thread when the
// function returns.  xs [128] and hid [256] are LDS scratch.  Uses every thread of the
// workgroup and ends with a barrier.
enum { kLsh = HK_HASH_LSH, kMlp = HK_HASH_MLP, kSign = HK_HASH_SIGN };
template <bool BF16, int KIND, int BITS>
__device__ __forceinline__ void wg_query_code(const HashPtrs &hp, const void *__restrict__ q,
                                              int64_t b, int hg, int Hq, int Hkv, float *xs,
                                              float *hid, uint32_t *qw) {
  constexpr int D = kHeadDim, NH = kHidden, W = BITS / 32;
  constexpr int EPV = BF16 ? 8 : 4;            // elements per 16-byte vector
  constexpr int V1 = D / EPV;                  // vectors per first-product row
  constexpr int V2 = (NH / 2) / EPV;           // vectors per half second-product row
  constexpr size_t ES = BF16 ? 2 : 4;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  auto unpack = [&](const uint4 &v, float *f) {
    if constexpr (BF16) {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
      f[0] = __uint_as_float(v.x);
      f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z);
      f[3] = __uint_as_float(v.w);
    }
  };
  // The group's query rows and the MLP biases are requested first, all at once, and the
  // weight rows right after them: memory waits count requests in issue order, so the mean
  // then waits for the query rows alone and its round trip overlaps the stream of weight
  // rows.  None of these loads sits under a branch (the compiler waits for a load at the
  // end of the branch that holds it): every thread reads column t mod D of the rows,
  // rows past the group read the group's last row and add zero to the mean, and a
  // missing bias reads a weight instead and is replaced by zero.  (Workgroups of 256
  // threads: t indexes the 256 hidden units.)
  const int G = Hq / Hkv;
  float qv[kMaxGroup];
  {
    const size_t r0 = (size_t)(b * Hq + (int64_t)hg * G) * D + (size_t)(t & (D - 1));
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) qv[j] = elem<BF16>(q, r0 + (size_t)(j < G ? j : G - 1) * D);
  }
  float bias1 = 0.f, bias2 = 0.f;
  if constexpr (KIND == kMlp) {
    const float v1 = elem<BF16>(hp.b1 ? hp.b1 : hp.W1, (size_t)t);
    const float v2 = elem<BF16>(hp.b2 ? hp.b2 : hp.W2, (size_t)((t >> 1) & (BITS - 1)));
    bias1 = hp.b1 ? v1 : 0.f;
    bias2 = (hp.b2 && t < 2 * BITS) ? v2 : 0.f;
  }
  const bool has1 = KIND == kMlp || (KIND == kLsh && t < BITS);
  uint4 w1[KIND == kSign ? 1 : V1];
  uint4 w2[KIND == kMlp ? V2 : 1];
  // bf16 MLP weights are copied into LDS by direct-to-LDS 16-byte loads, each wavefront
  // instruction moving 64 consecutive vectors of a padded row layout (rows of D + 8 and
  // NH + 8 elements, against bank conflicts; a pad slot reads its row's last vector
  // again), and each thread then reads its own row from LDS.  Reading the rows straight
  // from memory (every load instruction touching 64 rows) keeps one CU's load path busy
  // several times longer, and these loads hold no registers while in flight.  The
  // products are the same either way.
  constexpr bool kStage = BF16 && KIND == kMlp;
  constexpr int R1 = D / 8 + 1, R2 = NH / 8 + 1;     // padded row lengths in 16-byte vectors
  if constexpr (kStage) {
    __shared__ __attribute__((aligned(16))) uint4 w1s[NH * R1];
    __shared__ __attribute__((aligned(16))) uint4 w2s[BITS * R2];
    typedef const __attribute__((address_space(1))) void *gvp;
    typedef __attribute__((address_space(3))) void *lvp;
    const uint4 *s1 = static_cast<const uint4 *>(hp.W1);
    const uint4 *s2 = static_cast<const uint4 *>(hp.W2);
    constexpr int N1 = NH * R1 / 64, N2 = BITS * R2 / 64;   // instructions (64 vectors each)
    static_assert(NH * R1 % 64 == 0 && BITS * R2 % 64 == 0, "whole instructions");
    for (int k = wave; k < N1; k += 4) {
      const int v = 64 * k + lane, row = v / R1, pc = v - row * R1;
      __builtin_amdgcn_global_load_lds((gvp)(s1 + row * (D / 8) + (pc < D / 8 ? pc : D / 8 - 1)),
                                       (lvp)&w1s[64 * k], 16, 0, 0);
    }
    for (int k = wave; k < N2; k += 4) {
      const int v = 64 * k + lane, row = v / R2, pc = v - row * R2;
      __builtin_amdgcn_global_load_lds((gvp)(s2 + row * (NH / 8) + (pc < NH / 8 ? pc : NH / 8 - 1)),
                                       (lvp)&w2s[64 * k], 16, 0, 0);
    }
    if (t < D) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) sum += j < G ? qv[j] : 0.f;
      xs[t] = sum / (float)G;
    }
    __builtin_amdgcn_s_waitcnt(0);             // this wavefront's copies have landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < V1; ++i) w1[i] = w1s[t * R1 + i];
    if (t < 2 * BITS) {
#pragma unroll
      for (int i = 0; i < V2; ++i) w2[i] = w2s[(t >> 1) * R2 + (NH / 16) * (t & 1) + i];
    }
  } else {
    if (has1) {
      const uint4 *p = reinterpret_cast<const uint4 *>(
          static_cast<const char *>(KIND == kMlp ? hp.W1 : hp.R) + (size_t)t * D * ES);
#pragma unroll
      for (int i = 0; i < V1; ++i) w1[i] = p[i];
    }
    if (KIND == kMlp && t < 2 * BITS) {
      const uint4 *p = reinterpret_cast<const uint4 *>(
          static_cast<const char *>(hp.W2) + ((size_t)(t >> 1) * NH + (NH / 2) * (t & 1)) * ES);
#pragma unroll
      for (int i = 0; i < V2; ++i) w2[i] = p[i];
    }
    if (t < D) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) sum += j < G ? qv[j] : 0.f;
      xs[t] = sum / (float)G;
    }
    __syncthreads();
  }
  uint64_t m = 0;
  if constexpr (KIND == kSign) {
    m = __ballot(t < BITS && xs[t < D ? t : 0] > 0.f);
  } else {
    float a = 0.f;
    if (has1) {
#pragma unroll
      for (int i = 0; i < V1; ++i) {
        float f[EPV];
        unpack(w1[i], f);
#pragma unroll
        for (int k = 0; k < EPV; ++k) a = fmaf(f[k], xs[i * EPV + k], a);
      }
    }
    if constexpr (KIND == kMlp) {
      float h = gelu(a + bias1);
      if constexpr (BF16) h = round_bf16(h);
      hid[t] = h;
      __syncthreads();
      float y = 0.f;
      if (t < 2 * BITS) {
        const int e0 = (NH / 2) * (t & 1);
#pragma unroll
        for (int i = 0; i < V2; ++i) {
          float f[EPV];
          unpack(w2[i], f);
#pragma unroll
          for (int k = 0; k < EPV; ++k) y = fmaf(f[k], hid[e0 + i * EPV + k], y);
        }
      }
      y += __shfl_xor(y, 1) + bias2;
      m = __ballot(t < 2 * BITS && y > 0.f);
    } else {
      m = __ballot(t < BITS && a > 0.f);
    }
  }
  if (lane == 0) {
    if constexpr (KIND == kMlp) {
      // lanes 2j and 2j+1 both hold bit 32*wave + j: the even lanes' bits
      if (wave < W) {
        uint64_t x = m & 0x5555555555555555ull;
        x = (x | (x >> 1)) & 0x3333333333333333ull;
        x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
        x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
        x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
        x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
        qw[wave] = (uint32_t)x;
      }
    } else if (2 * wave < W) {                 // lane l of wave w holds bit 64 w + l
      qw[2 * wave] = (uint32_t)m;
      qw[2 * wave + 1] = (uint32_t)(m >> 32);
    }
  }
  __syncthreads();
}

}  // namespace enc
}  // namespace hk
