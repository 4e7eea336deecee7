// Hash encoders: keys and queries to packed sign-bit codes.
//
// LSH (HashEvict: Abstract): y = R x with R a Gaussian projection [bits][d].
// MLP (Spotlight Attention: Approach): y = W2 rho(GELU(W1 x + b1)) + b2, with rho the
// bf16 rounding (nearest-even) of the hidden activation when the hash is bf16.
// Bit j of a code is [y_j > 0], stored at bit j%32 of word j/32.
//
// bf16 keys (prefill of a whole cache, or one appended token) run on the matrix cores:
// each wavefront encodes 64 tokens per tile with v_mfma_f32_32x32x16_bf16.
//   GEMM1   H^T = W1 . X^T   A = W1 fragments from LDS, B = the tokens' rows loaded
//                            straight from HBM (each lane reads 128 contiguous bytes)
//   GELU    on the fp32 accumulators, bias, rounding to bf16 -- the accumulator layout
//           of H^T (one token column per lane) is already the B-operand layout of the
//           second GEMM once W2's hidden index is permuted the same way in LDS, so the
//           hidden activations never leave registers
//   GEMM2   Y^T = W2 . H^T
//   pack    lane m (+32) holds 16 of the 32 bits of token m for each 32-bit output
//           tile; the two halves are OR-ed across lanes m and m+32 and stored as one
//           16-byte code per token.
// Weights are staged in LDS once per workgroup in fragment order (64 lanes x 16 bytes
// per fragment), so every fragment read is one conflict-free ds_read_b128.
// Query codes (B*Hkv rows) and fp32 keys use a plain VALU kernel, one row per
// workgroup.
//
// The erf of GELU uses the Chebyshev fit of erfc from Numerical Recipes (Press et al.,
// section 6.2, "erfcc"), fractional error below 1.2e-7 everywhere: branch-free, one
// reciprocal and one exponential.
#include "hk_internal.h"

namespace hk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kRsqrt2 = 0.70710678118654752f;

// erfc(z) for z >= 0 (Numerical Recipes "erfcc").
__device__ __forceinline__ float erfc_nonneg(float z) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float arg = fmaf(-z, z, p);
  return t * __expf(arg);
}

// GELU(a) = a * Phi(a), Phi(a) = erfc(-a / sqrt 2) / 2.
__device__ __forceinline__ float gelu(float a) {
  const float e = 0.5f * erfc_nonneg(fabsf(a) * kRsqrt2);  // Phi(-|a|)
  return a >= 0.f ? fmaf(-a, e, a) : a * e;
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

// ------------------------------------------------------------------ VALU kernel
// mode 0: row r = (bh, t0 + j) of the key cache; mode 1: row r = (b, KV head), the
// input is the fp32 mean of the group's G query vectors.
template <bool BF16, bool MLP, int BITS>
__global__ __launch_bounds__(256) void encode_valu_kernel(HashPtrs hp, const void *__restrict__ x,
                                                          int mode, int64_t nt, int64_t cap,
                                                          int64_t t0, int Hq, int Hkv,
                                                          uint32_t *__restrict__ out) {
  constexpr int W = BITS / 32;
  __shared__ float xs[kHeadDim];
  __shared__ float hid[kHidden];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  uint32_t *dst;
  if (mode == 0) {
    const int64_t bh = r / nt, tok = t0 + (r - bh * nt);
    if (t < kHeadDim) xs[t] = elem<BF16>(x, (size_t)(bh * cap + tok) * kHeadDim + t);
    dst = out + (bh * cap + tok) * W;
  } else {
    const int64_t b = r / Hkv, g = r - b * Hkv;
    const int G = Hq / Hkv;
    if (t < kHeadDim) {
      float s = 0.f;
      for (int j = 0; j < G; ++j) s += elem<BF16>(x, (size_t)((b * Hq + g * G + j) * kHeadDim + t));
      xs[t] = s / (float)G;
    }
    dst = out + r * W;
  }
  __syncthreads();
  float y = 0.f;
  if constexpr (MLP) {
    float a = 0.f;
    for (int e = 0; e < kHeadDim; ++e) a = fmaf(elem<BF16>(hp.W1, (size_t)t * kHeadDim + e), xs[e], a);
    if (hp.b1) a += elem<BF16>(hp.b1, t);
    float h = gelu(a);
    if constexpr (BF16) h = round_bf16(h);
    hid[t] = h;
    __syncthreads();
    if (t < BITS) {
      for (int e = 0; e < kHidden; ++e) y = fmaf(elem<BF16>(hp.W2, (size_t)t * kHidden + e), hid[e], y);
      if (hp.b2) y += elem<BF16>(hp.b2, t);
    }
  } else {
    if (t < BITS)
      for (int e = 0; e < kHeadDim; ++e) y = fmaf(elem<BF16>(hp.R, (size_t)t * kHeadDim + e), xs[e], y);
  }
  const uint64_t mask = __ballot(t < BITS && y > 0.f);
  const int wave = t >> 6;
  if ((t & 63) == 0 && wave * 64 < BITS) {
    dst[2 * wave] = (uint32_t)mask;
    if (2 * wave + 1 < W) dst[2 * wave + 1] = (uint32_t)(mask >> 32);
  }
}

// ------------------------------------------------------------------ MFMA kernel
constexpr int kEncWaves = 4;

template <bool MLP, int BITS> struct EncLayout {
  static constexpr int JT = BITS / 32;                // 32-bit output tiles
  static constexpr int F1 = MLP ? 8 * 8 : JT * 8;     // first-GEMM fragments
  static constexpr int F2 = MLP ? JT * 16 : 0;        // second-GEMM fragments
  static constexpr int NB1 = MLP ? kHidden : 0;       // b1 floats
  static constexpr int NB2 = MLP ? BITS : 0;          // b2 floats
  static constexpr size_t bytes = (size_t)(F1 + F2) * 64 * 16 + (NB1 + NB2) * 4;
};

// Bit position, inside its 32-bit tile, of accumulator register r of lane group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

template <bool MLP, int BITS>
__global__ __launch_bounds__(kEncWaves * 64) void encode_keys_mfma_kernel(
    HashPtrs hp, const uint16_t *__restrict__ K, int64_t nt, int64_t cap, int64_t t0,
    int64_t total_rows, int64_t n_tiles, uint32_t *__restrict__ codes) {
  using L = EncLayout<MLP, BITS>;
  constexpr int JT = L::JT;
  constexpr int W = BITS / 32;
  __shared__ u32x4 frag[L::F1 + L::F2][64];
  __shared__ float bias[L::NB1 + L::NB2 + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int lg = lane >> 5;

  // Stage the weights in fragment order.
  const uint16_t *A1 = static_cast<const uint16_t *>(MLP ? hp.W1 : hp.R);
  for (int f = tid; f < L::F1 * 64; f += kEncWaves * 64) {
    const int fi = f >> 6, fl = f & 63, i = fl & 31, g = fl >> 5;
    const int tile = fi >> 3, ks = fi & 7;      // (hidden or bit tile, k-step)
    const uint16_t *src = A1 + (size_t)(32 * tile + i) * kHeadDim + 64 * g + 8 * ks;
    frag[fi][fl] = *reinterpret_cast<const u32x4 *>(src);
  }
  if constexpr (MLP) {
    const uint16_t *A2 = static_cast<const uint16_t *>(hp.W2);
    for (int f = tid; f < L::F2 * 64; f += kEncWaves * 64) {
      const int fi = f >> 6, fl = f & 63, i = fl & 31, g = fl >> 5;
      const int jt = fi >> 4, ks2 = fi & 15, ht = ks2 >> 1, half = ks2 & 1;
      const uint16_t *row = A2 + (size_t)(32 * jt + i) * kHidden + 32 * ht + 16 * half + 4 * g;
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(row);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 8);
      frag[L::F1 + fi][fl] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    for (int j = tid; j < L::NB1 + L::NB2; j += kEncWaves * 64) {
      const void *bp = j < L::NB1 ? hp.b1 : hp.b2;
      const int jj = j < L::NB1 ? j : j - L::NB1;
      bias[j] = bp ? elem<true>(bp, jj) : 0.f;
    }
  }
  __syncthreads();

  for (int64_t tile = (int64_t)blockIdx.x * kEncWaves + wave; tile < n_tiles;
       tile += (int64_t)gridDim.x * kEncWaves) {
    // X^T fragments of the two 32-token column tiles: lane (i, g) holds token
    // 64*tile + 32*n + i, elements 64*g .. 64*g + 63 (8 per k-step).
    bf16x8 xf[2][8];
    int64_t mem[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t row = tile * 64 + 32 * n + li;
      const bool ok = row < total_rows;
      const int64_t bh = ok ? row / nt : 0;
      mem[n] = ok ? bh * cap + t0 + (row - bh * nt) : -1;
      const uint16_t *src = K + (size_t)(ok ? mem[n] : 0) * kHeadDim + 64 * lg;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 v = ok ? *reinterpret_cast<const u32x4 *>(src + 8 * ks) : u32x4{0u, 0u, 0u, 0u};
        xf[n][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    f32x16 yacc[2][JT];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < JT; ++j) yacc[n][j] = f32x16{};

    if constexpr (MLP) {
#pragma unroll 1
      for (int ht = 0; ht < 8; ++ht) {
        f32x16 hacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, frag[ht * 8 + ks][lane]);
          hacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[0][ks], hacc[0], 0, 0, 0);
          hacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[1][ks], hacc[1], 0, 0, 0);
        }
        // GELU + bias + bf16 rounding; register r of lane group g is hidden unit
        // 32*ht + acc_row(r, g).  k-step half h of the second GEMM takes r = 8h .. 8h+7.
        bf16x8 hb[2][2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              const int r0 = 8 * half + 2 * s2, r1 = r0 + 1;
              const float h0 = gelu(hacc[n][r0] + bias[32 * ht + acc_row(r0, lg)]);
              const float h1 = gelu(hacc[n][r1] + bias[32 * ht + acc_row(r1, lg)]);
              w[s2] = bf16_bits(h0) | (bf16_bits(h1) << 16);
            }
            hb[n][half] = __builtin_bit_cast(bf16x8, w);
          }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int j = 0; j < JT; ++j) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, frag[L::F1 + j * 16 + 2 * ht + half][lane]);
            yacc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hb[0][half], yacc[0][j], 0, 0, 0);
            yacc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hb[1][half], yacc[1][j], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < JT; ++j) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, frag[j * 8 + ks][lane]);
          yacc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[0][ks], yacc[0][j], 0, 0, 0);
          yacc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[1][ks], yacc[1][j], 0, 0, 0);
        }
      }
    }

    // Sign bits.  Lanes li and li+32 hold complementary halves of each word of token
    // 32*n + li; OR them, then lane (li, lg) stores token 32*lg + li.
    uint32_t words[2][JT];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float y = yacc[n][j][r];
          if constexpr (MLP) y += bias[L::NB1 + 32 * j + acc_row(r, lg)];
          w |= (y > 0.f ? 1u : 0u) << acc_row(r, lg);
        }
        words[n][j] = w | __shfl_xor(w, 32);
      }
    }
    const int64_t dst_row = lg ? mem[1] : mem[0];
    if (dst_row >= 0) {
      uint32_t *dst = codes + (size_t)dst_row * W;
      if constexpr (W == 4) {
        *reinterpret_cast<u32x4 *>(dst) = lg ? u32x4{words[1][0], words[1][1], words[1][2], words[1][3]}
                                             : u32x4{words[0][0], words[0][1], words[0][2], words[0][3]};
      } else {
        *reinterpret_cast<u32x2 *>(dst) = lg ? u32x2{words[1][0], words[1][1]} : u32x2{words[0][0], words[0][1]};
      }
    }
  }
}

template <bool MLP, int BITS>
hipError_t mfma_launch(const HashPtrs &hp, const void *k, int64_t nt, int64_t cap, int64_t t0,
                       int64_t total, uint32_t *codes, hipStream_t st) {
  const int64_t n_tiles = (total + 63) / 64;
  // One workgroup per CU when the weights fill LDS; more when they are small.
  const int64_t per_cu = MLP ? 1 : 4;
  int64_t grid = (n_tiles + kEncWaves - 1) / kEncWaves;
  if (grid > 256 * per_cu) grid = 256 * per_cu;
  hipLaunchKernelGGL((encode_keys_mfma_kernel<MLP, BITS>), dim3((unsigned)grid),
                     dim3(kEncWaves * 64), 0, st, hp, static_cast<const uint16_t *>(k), nt, cap,
                     t0, total, n_tiles, codes);
  return hipGetLastError();
}

template <bool BF16, bool MLP, int BITS>
hipError_t valu_launch(const HashPtrs &hp, const void *x, int mode, int64_t rows, int64_t nt,
                       int64_t cap, int64_t t0, int Hq, int Hkv, uint32_t *out, hipStream_t st) {
  hipLaunchKernelGGL((encode_valu_kernel<BF16, MLP, BITS>), dim3((unsigned)rows), dim3(256), 0,
                     st, hp, x, mode, nt, cap, t0, Hq, Hkv, out);
  return hipGetLastError();
}

template <bool BF16>
hipError_t valu_dispatch(const hk_hash &h, const void *x, int mode, int64_t rows, int64_t nt,
                         int64_t cap, int64_t t0, int Hq, int Hkv, uint32_t *out, hipStream_t st) {
  const HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const bool mlp = h.kind == HK_HASH_MLP;
  if (mlp && h.bits == 128) return valu_launch<BF16, true, 128>(hp, x, mode, rows, nt, cap, t0, Hq, Hkv, out, st);
  if (mlp) return valu_launch<BF16, true, 64>(hp, x, mode, rows, nt, cap, t0, Hq, Hkv, out, st);
  if (h.bits == 128) return valu_launch<BF16, false, 128>(hp, x, mode, rows, nt, cap, t0, Hq, Hkv, out, st);
  return valu_launch<BF16, false, 64>(hp, x, mode, rows, nt, cap, t0, Hq, Hkv, out, st);
}

}  // namespace

hipError_t launch_encode_keys(const hk_hash &h, const void *k, int B, int Hkv, int64_t cap,
                              int64_t t0, int64_t t1, uint32_t *codes, hipStream_t st) {
  const int64_t nt = t1 - t0;
  const int64_t total = (int64_t)B * Hkv * nt;
  if (total == 0) return hipSuccess;
  if (h.dtype == HK_F32) return valu_dispatch<false>(h, k, 0, total, nt, cap, t0, 0, 1, codes, st);
  const HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const bool mlp = h.kind == HK_HASH_MLP;
  if (mlp && h.bits == 128) return mfma_launch<true, 128>(hp, k, nt, cap, t0, total, codes, st);
  if (mlp) return mfma_launch<true, 64>(hp, k, nt, cap, t0, total, codes, st);
  if (h.bits == 128) return mfma_launch<false, 128>(hp, k, nt, cap, t0, total, codes, st);
  return mfma_launch<false, 64>(hp, k, nt, cap, t0, total, codes, st);
}

hipError_t launch_encode_query(const hk_hash &h, const void *q, int B, int Hq, int Hkv,
                               uint32_t *qcodes, hipStream_t st) {
  const int64_t rows = (int64_t)B * Hkv;
  if (rows == 0) return hipSuccess;
  if (h.dtype == HK_F32) return valu_dispatch<false>(h, q, 1, rows, 1, 0, 0, Hq, Hkv, qcodes, st);
  return valu_dispatch<true>(h, q, 1, rows, 1, 0, 0, Hq, Hkv, qcodes, st);
}

}  // namespace hk
