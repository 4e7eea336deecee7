// Hash encoders: keys and queries to packed sign-bit codes.
//
// LSH (HashEvict: Abstract): y = R x with R a Gaussian projection [bits][d].
// MLP (Spotlight Attention: Approach): y = W2 rho(GELU(W1 x + b1)) + b2, with rho the
// bf16 rounding (nearest-even) of the hidden activation when the hash is bf16.
// Bit j of a code is [y_j > 0], stored at bit j%32 of word j/32.
//
// bf16 keys (prefill of a whole cache, or one appended token) run on the matrix cores:
// each wavefront encodes 32 tokens per tile with v_mfma_f32_32x32x16_bf16.
//   GEMM1   H^T = W1 . X^T   A = W1 fragments from LDS, B = the tokens' rows loaded
//                            straight from HBM (each lane reads 128 contiguous bytes)
//   GELU    on the fp32 accumulators, bias, rounding to bf16 -- the accumulator layout
//           of H^T (one token column per lane) is already the B-operand layout of the
//           second GEMM once W2's hidden index is permuted the same way in LDS, so the
//           hidden activations never leave registers.
//   GEMM2   Y^T = W2 . H^T
//   pack    lane i (+32) holds 16 of the 32 bits of token i for each 32-bit output
//           tile; the two halves are OR-ed across lanes i and i+32, and each lane of
//           the pair stores half of the token's code.
// The GELU's vector instructions (eight per hidden unit) and the matrix-core products
// take comparable time; two wavefronts per SIMD overlap one's GELU with the other's
// products.
// Weights are staged in LDS once per workgroup in fragment order (64 lanes x 16 bytes
// per fragment), so every fragment read is one conflict-free ds_read_b128.
// Query codes (B*Hkv rows) and fp32 keys use a plain VALU kernel, one row per
// workgroup.
//
// GELU's normal tail is one polynomial under one exponential (no reciprocal, no
// branch), with absolute error below 4.6e-7.
#include "encode_core.h"

namespace hk {
namespace {
using namespace enc;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ VALU kernel
// fp32 keys: row r = (bh, t0 + j) of the key cache, one workgroup per key.
template <bool BF16, bool MLP, int BITS>
__global__ __launch_bounds__(256) void encode_valu_kernel(HashPtrs hp, const void *__restrict__ x,
                                                          int64_t nt, int64_t cap, int64_t t0,
                                                          uint32_t *__restrict__ out) {
  constexpr int W = BITS / 32;
  __shared__ float xs[kHeadDim];
  __shared__ float hid[kHidden];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t bh = r / nt, tok = t0 + (r - bh * nt);
  if (t < kHeadDim) xs[t] = elem<BF16>(x, (size_t)(bh * cap + tok) * kHeadDim + t);
  uint32_t *dst = out + (bh * cap + tok) * W;
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

// ------------------------------------------------------------------ query kernel (fp32)
// The query code of each (b, KV head) for fp32 hashes: the fp32 mean of the group's G
// query vectors, hashed in fp32 arithmetic.  kQRows rows per workgroup.  Every thread requests its
// whole weight rows at the start (row t of W1 or R; for the MLP also one half of row t/2
// of W2), so the kernel makes one memory round trip before the arithmetic; the two
// halves of a W2 row are summed by neighbouring lanes.
constexpr int kQRows = 2;

template <bool BF16, bool MLP, int BITS>
__global__ __launch_bounds__(256) void encode_query_kernel(HashPtrs hp, const void *__restrict__ q,
                                                           int64_t rows, int Hq, int Hkv,
                                                           uint32_t *__restrict__ out) {
  constexpr int D = kHeadDim, NH = kHidden, W = BITS / 32;
  constexpr int EPV = BF16 ? 8 : 4;            // elements per 16-byte vector
  constexpr int V1 = D / EPV;                  // vectors per GEMM1 row
  constexpr int V2 = (NH / 2) / EPV;           // vectors per half GEMM2 row
  __shared__ float xs[kQRows][D];
  __shared__ float hid[kQRows][NH];
  const int64_t r0 = (int64_t)blockIdx.x * kQRows;
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
  constexpr size_t ES = BF16 ? 2 : 4;
  const bool has1 = MLP || t < BITS;
  uint4 w1[V1];
  if (has1) {
    const uint4 *p = reinterpret_cast<const uint4 *>(
        static_cast<const char *>(MLP ? hp.W1 : hp.R) + (size_t)t * D * ES);
#pragma unroll
    for (int i = 0; i < V1; ++i) w1[i] = p[i];
  }
  uint4 w2[MLP ? V2 : 1];
  auto load_w2 = [&]() {
    if (t < 2 * BITS) {
      const uint4 *p = reinterpret_cast<const uint4 *>(
          static_cast<const char *>(hp.W2) + ((size_t)(t >> 1) * NH + (NH / 2) * (t & 1)) * ES);
#pragma unroll
      for (int i = 0; i < V2; ++i) w2[i] = p[i];
    }
  };
  // bf16 weights: both rows in flight at once.  fp32 rows are twice as large; their W2
  // half is requested after the first product so that the registers suffice.
  if constexpr (MLP && BF16) load_w2();
  const int G = Hq / Hkv;
  for (int i = t; i < kQRows * D; i += 256) {
    const int rr = i / D, e = i - rr * D;
    const int64_t r = r0 + rr;
    float sum = 0.f;
    if (r < rows) {
      const int64_t b = r / Hkv, g = r - b * Hkv;
      float v[kMaxGroup];                      // all loads issued before any is summed
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j)
        v[j] = j < G ? elem<BF16>(q, (size_t)((b * Hq + g * G + j) * D + e)) : 0.f;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) sum += v[j];
    }
    xs[rr][e] = sum / (float)G;
  }
  __syncthreads();
  float a[kQRows];
#pragma unroll
  for (int rr = 0; rr < kQRows; ++rr) a[rr] = 0.f;
  if (has1) {
#pragma unroll
    for (int i = 0; i < V1; ++i) {
      float f[EPV];
      unpack(w1[i], f);
#pragma unroll
      for (int rr = 0; rr < kQRows; ++rr)
#pragma unroll
        for (int k = 0; k < EPV; ++k) a[rr] = fmaf(f[k], xs[rr][i * EPV + k], a[rr]);
    }
  }
  float y[kQRows];
  if constexpr (MLP) {
    if constexpr (!BF16) load_w2();
    const float bias1 = hp.b1 ? elem<BF16>(hp.b1, t) : 0.f;
#pragma unroll
    for (int rr = 0; rr < kQRows; ++rr) {
      float h = gelu(a[rr] + bias1);
      if constexpr (BF16) h = round_bf16(h);
      hid[rr][t] = h;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < kQRows; ++rr) y[rr] = 0.f;
    if (t < 2 * BITS) {
      const int e0 = (NH / 2) * (t & 1);
#pragma unroll
      for (int i = 0; i < V2; ++i) {
        float f[EPV];
        unpack(w2[i], f);
#pragma unroll
        for (int rr = 0; rr < kQRows; ++rr)
#pragma unroll
          for (int k = 0; k < EPV; ++k) y[rr] = fmaf(f[k], hid[rr][e0 + i * EPV + k], y[rr]);
      }
    }
    const float bias2 = (hp.b2 && t < 2 * BITS) ? elem<BF16>(hp.b2, t >> 1) : 0.f;
#pragma unroll
    for (int rr = 0; rr < kQRows; ++rr) y[rr] += __shfl_xor(y[rr], 1) + bias2;
  } else {
#pragma unroll
    for (int rr = 0; rr < kQRows; ++rr) y[rr] = a[rr];
  }
  // Sign bits.  MLP: lanes 2j and 2j+1 both hold bit 32*wave + j; LSH: lane l holds bit
  // 64*wave + l.
#pragma unroll
  for (int rr = 0; rr < kQRows; ++rr) {
    const int64_t r = r0 + rr;
    const bool valid = MLP ? (t < 2 * BITS) : (t < BITS);
    const uint64_t m = __ballot(valid && y[rr] > 0.f);
    if (r >= rows || lane != 0) continue;
    if constexpr (MLP) {
      if (wave < W) {
        uint64_t x = m & 0x5555555555555555ull;            // even lanes -> 32 bits
        x = (x | (x >> 1)) & 0x3333333333333333ull;
        x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
        x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
        x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
        x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
        out[r * W + wave] = (uint32_t)x;
      }
    } else {
      if (2 * wave < W) {
        out[r * W + 2 * wave] = (uint32_t)m;
        out[r * W + 2 * wave + 1] = (uint32_t)(m >> 32);
      }
    }
  }
}

// ------------------------------------------------------------------ query kernel (bf16)
// bf16 hashes on the matrix cores: 16 query rows per workgroup (one 16-row tile), one
// 16-column tile of each product per wavefront (16 wavefronts, so the weight fragments,
// the products and the GELUs are spread over as many SIMD slots as there are tiles).  The fp32 group mean x is split exactly into
// three bf16 parts (x = hi + mid + lo to 24 bits), so x . w accumulates in fp32 from
// exact products, as an fp32 dot product would.  The MLP's hidden activation is bf16 by
// definition (rounded after GELU), so the second product needs no split.
//   A operand (16 x 32): lane l holds row l%16, k = 8*(l/16) .. +7 of a 32-wide k-step;
//   B operand (32 x 16): lane l holds column l%16, the same 8 k's;
//   result: lane l holds column l%16 of rows 4*(l/16) .. +3.
constexpr int kQTile = 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool MLP, int BITS>
__global__ __launch_bounds__(1024) void encode_query_mfma_kernel(HashPtrs hp,
                                                                 const uint16_t *__restrict__ q,
                                                                 int64_t rows, int Hq, int Hkv,
                                                                 uint32_t *__restrict__ out) {
  constexpr int D = kHeadDim, NH = kHidden, W = BITS / 32;
  constexpr int N1 = MLP ? NH : BITS;          // first product's columns
  constexpr int NT1 = N1 / 16, NT2 = MLP ? BITS / 16 : 0;   // 16-column tiles
  static_assert(NT1 <= 16 && NT2 <= 16, "one tile per wavefront");
  // The weights are copied to LDS with contiguous loads (16 lanes per 256-byte row
  // segment): reading the matrix-core fragments straight from memory (16 rows x 64 bytes
  // per load instruction) takes several times longer through one CU.  Rows are padded by
  // 16 bytes so that the fragment reads from LDS spread over the banks.
  constexpr int P1 = D + 8, P2 = NH + 8;
  __shared__ __attribute__((aligned(16))) uint16_t w1s[N1 * P1];
  __shared__ __attribute__((aligned(16))) uint16_t w2s[MLP ? BITS * P2 : 8];
  // The group means as three bf16 parts (x = p0 + p1 + p2 exactly), split once per
  // element by the thread that sums it and read by every wavefront as its A fragments
  // (splitting in each wavefront repeated the same work sixteen times).  Rows padded by
  // 16 bytes.
  constexpr int PX = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t xb[3][kQTile][PX];
  __shared__ __attribute__((aligned(16))) uint16_t hs[MLP ? kQTile : 1][MLP ? P2 : 8];
  __shared__ uint32_t words[kQTile][W];
  const int64_t r0 = (int64_t)blockIdx.x * kQTile;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool has1 = wave < NT1, has2 = MLP && wave < NT2;
  // Group means: thread t -> row t/64, dims 2*(t%64), +1.  The query rows are requested
  // before the weights, so that the two round trips to memory overlap; all G <= 8 loads
  // are in flight before any is summed.
  const int rr = t >> 6, e0 = 2 * (t & 63);
  const int G = Hq / Hkv;
  uint32_t qv[kMaxGroup];
  {
    const int64_t r = r0 + rr;
    const int64_t b = r / Hkv, hg = r - b * Hkv;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j)
      qv[j] = (r < rows && j < G)
                  ? *reinterpret_cast<const uint32_t *>(q + (size_t)((b * Hq + hg * G + j) * D + e0))
                  : 0u;
  }
  // The MLP's biases for this lane's columns, requested with the rest and without a
  // branch (the compiler waits for a load at the end of the branch that holds it, which
  // would put two round trips before the weights are requested): a missing bias reads a
  // weight instead and is replaced by zero.  col < 256 = kHidden; the second product's
  // columns are below BITS where they are used.
  float bias1 = 0.f, bias2 = 0.f;
  if constexpr (MLP) {
    const int col = 16 * wave + n;
    const float v1 = elem<true>(hp.b1 ? hp.b1 : hp.W1, (size_t)col);
    const float v2 = elem<true>(hp.b2 ? hp.b2 : hp.W2, (size_t)(col & (BITS - 1)));
    bias1 = (has1 && hp.b1) ? v1 : 0.f;
    bias2 = (has2 && hp.b2) ? v2 : 0.f;
  }
  {
    constexpr int C1 = N1 * D / 8, C2 = MLP ? BITS * NH / 8 : 0;   // 16-byte vectors
    constexpr int L1 = (C1 + 1023) / 1024, L2 = (C2 + 1023) / 1024;
    const uint4 *g1 = static_cast<const uint4 *>(MLP ? hp.W1 : hp.R);
    uint4 v1[L1];
#pragma unroll
    for (int i = 0; i < L1; ++i) {
      const int c = t + 1024 * i;
      v1[i] = c < C1 ? g1[c] : make_uint4(0, 0, 0, 0);
    }
    uint4 v2[L2 > 0 ? L2 : 1];
    if constexpr (MLP) {
      const uint4 *g2 = static_cast<const uint4 *>(hp.W2);
#pragma unroll
      for (int i = 0; i < L2; ++i) {
        const int c = t + 1024 * i;
        v2[i] = c < C2 ? g2[c] : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < L1; ++i) {
      const int c = t + 1024 * i;
      if (c < C1) *reinterpret_cast<uint4 *>(&w1s[(c / (D / 8)) * P1 + 8 * (c % (D / 8))]) = v1[i];
    }
    if constexpr (MLP) {
#pragma unroll
      for (int i = 0; i < L2; ++i) {
        const int c = t + 1024 * i;
        if (c < C2) *reinterpret_cast<uint4 *>(&w2s[(c / (NH / 8)) * P2 + 8 * (c % (NH / 8))]) = v2[i];
      }
    }
  }
  if (t < kQTile * W) words[t / W][t % W] = 0u;
  {
    float acc0 = 0.f, acc1 = 0.f;
    if (r0 + rr < rows) {
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) {
        acc0 += __uint_as_float(qv[j] << 16);
        acc1 += __uint_as_float(qv[j] & 0xFFFF0000u);
      }
      acc0 = acc0 / (float)G;
      acc1 = acc1 / (float)G;
    }
    float x0 = acc0, x1 = acc1;
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const uint32_t b0 = bf16_bits(x0), b1 = bf16_bits(x1);
      *reinterpret_cast<uint32_t *>(&xb[part][rr][e0]) = b0 | (b1 << 16);
      x0 -= __uint_as_float(b0 << 16);                 // exact
      x1 -= __uint_as_float(b1 << 16);
    }
  }
  __syncthreads();
  f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
  if (has1) {
    // A fragments of x: three bf16 parts per k-step.
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int col = 16 * wave + n;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 p0 = *reinterpret_cast<const bf16x8 *>(&xb[0][n][32 * ks + 8 * g]);
      const bf16x8 p1 = *reinterpret_cast<const bf16x8 *>(&xb[1][n][32 * ks + 8 * g]);
      const bf16x8 p2 = *reinterpret_cast<const bf16x8 *>(&xb[2][n][32 * ks + 8 * g]);
      const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(&w1s[col * P1 + 32 * ks + 8 * g]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p0, bw, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, bw, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p2, bw, acc, 0, 0, 0);
    }
    if constexpr (MLP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) hs[4 * g + j][col] = (uint16_t)bf16_bits(gelu(acc[j] + bias1));
    } else {
      y = acc;
    }
  }
  if constexpr (MLP) {
    __syncthreads();
    if (has2) {
      const int col = 16 * wave + n;
#pragma unroll
      for (int ks = 0; ks < NH / 32; ++ks) {
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&hs[n][32 * ks + 8 * g]);
        const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(&w2s[col * P2 + 32 * ks + 8 * g]);
        y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw, y, 0, 0, 0);
      }
    }
  }
  // Sign bits: wavefront w covers bits 16w .. 16w+15; the ballot of register j holds, in
  // lanes 16g .. 16g+15, those bits of row 4g + j.
  constexpr int NT = MLP ? NT2 : NT1;
  if (wave < NT) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t m = __ballot(y[j] + bias2 > 0.f);
      if (lane < 4) {
        const int row = 4 * lane + j;
        const uint32_t bits16 = (uint32_t)(m >> (16 * lane)) & 0xFFFFu;
        atomicOr(&words[row][wave >> 1], bits16 << (16 * (wave & 1)));
      }
    }
  }
  __syncthreads();
  if (t < kQTile * W) {
    const int rr = t / W, wd = t - rr * W;
    if (r0 + rr < rows) out[(r0 + rr) * W + wd] = words[rr][wd];
  }
}

// ------------------------------------------------------------------ sign codes
// SIGN hash (Self-Indexing KVCache: Abstract, sign-based 1-bit keys): bit j = [x_j > 0],
// no projection.  Keys: 16 lanes per key, lane l turns elements 8l .. 8l+7 into byte l
// of the 16-byte code (bits 8l .. 8l+7, least significant first), so a wavefront reads
// 4 whole rows and writes 4 whole codes.  Bound by HBM bandwidth.
template <bool BF16>
__global__ __launch_bounds__(256) void encode_keys_sign_kernel(const void *__restrict__ k,
                                                               int64_t nt, int64_t cap,
                                                               int64_t t0, int64_t total,
                                                               uint8_t *__restrict__ codes) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t key = gid >> 4;
  const int l = (int)(gid & 15);
  if (key >= total) return;
  const int64_t bh = key / nt;
  const int64_t row = bh * cap + t0 + (key - bh * nt);
  float x[8];
  if constexpr (BF16) {
    const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(k) + row * kHeadDim + 8 * l);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(k) + row * kHeadDim + 8 * l);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  uint32_t byte = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) byte |= (x[e] > 0.f ? 1u : 0u) << e;
  codes[row * 16 + l] = (uint8_t)byte;
}

// Queries: one workgroup of 128 threads per (b, KV head); thread j takes element j of
// the group-mean query (fp32, as the other query encoders), and each wavefront's ballot
// is 64 bits of the code.
template <bool BF16>
__global__ __launch_bounds__(128) void encode_query_sign_kernel(const void *__restrict__ q,
                                                                int Hq, int Hkv,
                                                                uint32_t *__restrict__ out) {
  const int64_t r = blockIdx.x;
  const int j = threadIdx.x;
  const int64_t b = r / Hkv, hg = r - b * Hkv;
  const int G = Hq / Hkv;
  float acc = 0.f;
  for (int g = 0; g < G; ++g) acc += elem<BF16>(q, (size_t)((b * Hq + hg * G + g) * kHeadDim + j));
  acc = acc / (float)G;
  const uint64_t m = __ballot(acc > 0.f);
  if ((j & 63) == 0) {
    out[r * 4 + 2 * (j >> 6)] = (uint32_t)m;
    out[r * 4 + 2 * (j >> 6) + 1] = (uint32_t)(m >> 32);
  }
}

// ------------------------------------------------------------------ MFMA kernel
template <bool MLP, int BITS, bool BIAS = false> struct EncLayout {
  static constexpr int JT = BITS / 32;                // 32-bit output tiles
  static constexpr int F1 = MLP ? 8 * 8 : JT * 8;     // first-GEMM fragments
  static constexpr int F2 = MLP ? JT * 16 : 0;        // second-GEMM fragments
  // LDS fragment order: per hidden (or bit) tile, its 8 first-GEMM k-steps, then (MLP)
  // its 2 * JT second-GEMM fragments, so that one tile's reads share a base address
  // and take constant offsets within the 16-bit offset field.
  static constexpr int FB = MLP ? 8 + 2 * JT : 8;
  static constexpr int NB1 = MLP ? kHidden : 0;       // b1 floats
  static constexpr int NB2 = MLP ? BITS : 0;          // b2 floats
  // Wavefronts per workgroup.  The MLP weights fill most of LDS, so one workgroup holds
  // a CU.  Without biases, 12 wavefronts (3 per SIMD, at most 168 registers each) run
  // the pipelined stages; with biases, 8 (2 per SIMD) run one hidden tile at a time.
  // The LSH projection is small; several workgroups share a CU.
  static constexpr int WAVES = MLP ? (BIAS ? 8 : 12) : 4;
  static constexpr int PER_CU = MLP ? 1 : 4;
};

// Vector instructions scheduled after each matrix-core product in the MLP's pipelined
// stages (a stage holds 16 products and about 150 vector instructions).
constexpr int kGeluGroup = 9;

typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;   // an LDS-resident vector

// Bit position, inside its 32-bit tile, of accumulator register r of lane group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

// One tile = 32 tokens per wavefront.  Lane (i, g) (i = lane % 32, g = lane / 32) holds
// token i of the tile: the B operand reads its elements 64 g + 8 ks .. + 7 for k-step
// ks, and accumulator register r holds output row acc_row(r, g) of token i.
// BIAS: the MLP has b1 or b2 (a null bias reads as zero).
template <bool MLP, int BITS, bool BIAS>
__global__ __launch_bounds__((EncLayout<MLP, BITS, BIAS>::WAVES * 64)) void encode_keys_mfma_kernel(
    HashPtrs hp, const uint16_t *__restrict__ K, int64_t nt, int64_t cap, int64_t t0,
    int64_t total_rows, int64_t n_tiles, uint32_t *__restrict__ codes) {
  using L = EncLayout<MLP, BITS, BIAS>;
  constexpr int JT = L::JT;
  constexpr int W = BITS / 32;
  constexpr int NWG = L::WAVES * 64;
  __shared__ u32x4 frag[L::F1 + L::F2][64];
  __shared__ float bias[BIAS ? L::NB1 + L::NB2 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int lg = lane >> 5;

  // Stage the weights in fragment order.
  const uint16_t *A1 = static_cast<const uint16_t *>(MLP ? hp.W1 : hp.R);
  for (int f = tid; f < L::F1 * 64; f += NWG) {
    const int fi = f >> 6, fl = f & 63, i = fl & 31, g = fl >> 5;
    const int tile = fi >> 3, ks = fi & 7;      // (hidden or bit tile, k-step)
    const uint16_t *src = A1 + (size_t)(32 * tile + i) * kHeadDim + 64 * g + 8 * ks;
    frag[tile * L::FB + ks][fl] = *reinterpret_cast<const u32x4 *>(src);
  }
  static_assert(MLP || !BIAS, "LSH has no bias");
  if constexpr (MLP) {
    const uint16_t *A2 = static_cast<const uint16_t *>(hp.W2);
    for (int f = tid; f < L::F2 * 64; f += NWG) {
      const int fi = f >> 6, fl = f & 63, i = fl & 31, g = fl >> 5;
      const int ks2 = fi / JT, jt = fi - ks2 * JT, ht = ks2 >> 1, half = ks2 & 1;
      const uint16_t *row = A2 + (size_t)(32 * jt + i) * kHidden + 32 * ht + 16 * half + 4 * g;
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(row);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 8);
      frag[ht * L::FB + 8 + half * JT + jt][fl] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    if constexpr (BIAS) {
      for (int j = tid; j < L::NB1 + L::NB2; j += NWG) {
        const void *bp = j < L::NB1 ? hp.b1 : hp.b2;
        const int jj = j < L::NB1 ? j : j - L::NB1;
        bias[j] = bp ? elem<true>(bp, jj) : 0.f;
      }
    }
  }
  __syncthreads();

  // Lane li's row of the current tile, its position in the cache (head bh, token t0 +
  // off) and its cache row mem.  Tiles advance by a fixed stride of rows, so the
  // division by nt happens once; each step adds the stride's quotient and remainder.
  const int64_t tstride = (int64_t)gridDim.x * L::WAVES;
  const int64_t step = tstride * 32;
  const int64_t q = step / nt, rem = step - q * nt;
  const int64_t dmem = q * cap + rem;
  int64_t tile = (int64_t)blockIdx.x * L::WAVES + wave;
  int64_t row = tile * 32 + li;
  int64_t off = row % nt;
  int64_t mem = (row / nt) * cap + t0 + off;
  // Rows past the end read row 0 instead (a token column only feeds its own outputs,
  // and those are not stored), so every load is unconditional.
  auto load = [&](bf16x8 (&x)[8]) {
    const uint16_t *src = K + (size_t)(row < total_rows ? mem : 0) * kHeadDim + 64 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      x[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src + 8 * ks));
  };
  // The LSH projection is bound by the key reads: each wavefront requests its next
  // tile's keys before working on the current one.  (The MLP's registers are taken by
  // its pipelined stages, and its products hide the reads anyway.)
  constexpr bool PREFETCH = !MLP;
  bf16x8 xn[8];
  if (PREFETCH && tile < n_tiles) load(xn);
  for (; tile < n_tiles; tile += tstride) {
    const bool ok = row < total_rows;
    bf16x8 xf[8];
    if constexpr (PREFETCH) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) xf[ks] = xn[ks];
    } else {
      load(xf);
    }
    const int64_t mem_st = mem;
    row += step;
    off += rem;
    mem += dmem;
    if (off >= nt) {
      off -= nt;
      mem += cap - nt;
    }
    if (PREFETCH && tile + tstride < n_tiles) load(xn);

    f32x16 yacc[JT];        // the first product into each starts from a zero accumulator

    if constexpr (MLP) {
      // H^T tile ht (hidden units 32 ht .. 32 ht + 31) of the first GEMM.
      // Hidden tile ht's fragments are read through a base pointer the compiler cannot
      // re-derive, so every read is that base plus a constant offset (left to itself,
      // it shares one running base between tiles and needs an add per read for the
      // offsets that fall outside the unsigned offset field).
      auto block = [&](int ht) {
        lds_u32x4 *b = (lds_u32x4 *)(&frag[ht * L::FB][lane]);
        asm volatile("" : "+v"(b));
        return b;
      };
      auto gemm1 = [&](int ht) {
        lds_u32x4 *b = block(ht);
        f32x16 h = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          h = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[64 * ks]), xf[ks], h,
                                                      0, 0, 0);
        return h;
      };
      // Bias, GELU and bf16 rounding of H^T tile ht: the B operand of its two k-steps of
      // the second GEMM.  Register r of lane group g is hidden unit 32 ht + acc_row(r, g);
      // k-step half h of the second GEMM takes r = 8h .. 8h+7.
      struct Hid {
        bf16x8 h[2];
      };
      auto gelu_pack = [&](int ht, const f32x16 &hacc) {
        Hid out;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            float a0 = hacc[r], a1 = hacc[r + 1];
            if constexpr (BIAS) {
              a0 += bias[32 * ht + acc_row(r, lg)];
              a1 += bias[32 * ht + acc_row(r + 1, lg)];
            }
            const bf16x2 pr = {(__bf16)gelu(a0), (__bf16)gelu(a1)};
            w[e] = __builtin_bit_cast(uint32_t, pr);
          }
          out.h[half] = __builtin_bit_cast(bf16x8, w);
        }
        return out;
      };
      // Hidden tile ht's share of the second GEMM (the first share starts from zero).
      auto gemm2 = [&](int ht, const Hid &hb, bool first) {
        lds_u32x4 *b = block(ht);
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int j = 0; j < JT; ++j)
            yacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, b[64 * (8 + half * JT + j)]), hb.h[half],
                first && half == 0 ? f32x16{} : yacc[j], 0, 0, 0);
      };
      if constexpr (!BIAS) {
        // Software pipeline over the eight hidden tiles: while the vector ALU computes
        // tile ht's GELU, the matrix cores run the second GEMM of tile ht-1 and the first
        // GEMM of tile ht+1 (neither depends on that GELU).  Each such stage is one
        // scheduling region whose 16 products are interleaved with the GELU's
        // instructions, so that one wavefront keeps both units busy; the other
        // wavefronts of the SIMD fill the gaps.
        auto interleave = [] {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one matrix-core product
            __builtin_amdgcn_sched_group_barrier(0x002, kGeluGroup, 0);   // vector ALU
          }
        };
        f32x16 ha = gemm1(0);
        f32x16 hb = gemm1(1);
        Hid pa = gelu_pack(0, ha);
        gemm2(0, pa, true);
        ha = gemm1(2);
        Hid pb = gelu_pack(1, hb);
        interleave();
#pragma unroll 1
        for (int ht = 2; ht < 6; ht += 2) {
          gemm2(ht - 1, pb, false);
          hb = gemm1(ht + 1);
          pa = gelu_pack(ht, ha);
          interleave();
          gemm2(ht, pa, false);
          ha = gemm1(ht + 2);
          pb = gelu_pack(ht + 1, hb);
          interleave();
        }
        gemm2(5, pb, false);
        hb = gemm1(7);
        pa = gelu_pack(6, ha);
        interleave();
        gemm2(6, pa, false);
        pb = gelu_pack(7, hb);
        gemm2(7, pb, false);
      } else {
        // With biases: one hidden tile at a time (the bias reads need the registers).
#pragma unroll
        for (int j = 0; j < JT; ++j) yacc[j] = f32x16{};
#pragma unroll 1
        for (int ht = 0; ht < 8; ++ht) gemm2(ht, gelu_pack(ht, gemm1(ht)), false);
      }
    } else {
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          yacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, frag[j * 8 + ks][lane]),
                                                            xf[ks], ks == 0 ? f32x16{} : yacc[j], 0, 0, 0);
    }

    // Sign bits.  Lanes i and i+32 hold complementary halves of each word of token i;
    // OR them, then lane group g stores words g*JT/2 .. of token i.
    uint32_t words[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      // acc_row(r, lg) = acc_row(r, 0) + 4 lg: constant shifts per register, then one
      // shift by the lane group.
      uint32_t w = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float y = yacc[j][r];
        if constexpr (BIAS) y += bias[L::NB1 + 32 * j + acc_row(r, lg)];
        w |= (y > 0.f ? 1u : 0u) << acc_row(r, 0);
      }
      w <<= 4 * lg;
      words[j] = w | __shfl_xor(w, 32);
    }
    if (ok) {
      uint32_t *dst = codes + (size_t)mem_st * W + (W / 2) * lg;
      if constexpr (W == 4)
        *reinterpret_cast<u32x2 *>(dst) = lg ? u32x2{words[2], words[3]} : u32x2{words[0], words[1]};
      else
        *dst = lg ? words[1] : words[0];
    }
  }
}

template <bool MLP, int BITS, bool BIAS>
hipError_t mfma_launch(const HashPtrs &hp, const void *k, int64_t nt, int64_t cap, int64_t t0,
                       int64_t total, uint32_t *codes, hipStream_t st) {
  using L = EncLayout<MLP, BITS, BIAS>;
  const int64_t n_tiles = (total + 31) / 32;
  int64_t grid = (n_tiles + L::WAVES - 1) / L::WAVES;
  if (grid > 256 * L::PER_CU) grid = 256 * L::PER_CU;
  hipLaunchKernelGGL((encode_keys_mfma_kernel<MLP, BITS, BIAS>), dim3((unsigned)grid),
                     dim3(L::WAVES * 64), 0, st, hp, static_cast<const uint16_t *>(k), nt, cap,
                     t0, total, n_tiles, codes);
  return hipGetLastError();
}

template <bool BF16, bool MLP, int BITS>
hipError_t valu_launch(const HashPtrs &hp, const void *x, int64_t rows, int64_t nt, int64_t cap,
                       int64_t t0, uint32_t *out, hipStream_t st) {
  hipLaunchKernelGGL((encode_valu_kernel<BF16, MLP, BITS>), dim3((unsigned)rows), dim3(256), 0,
                     st, hp, x, nt, cap, t0, out);
  return hipGetLastError();
}

template <bool BF16>
hipError_t valu_dispatch(const hk_hash &h, const void *x, int64_t rows, int64_t nt, int64_t cap,
                         int64_t t0, uint32_t *out, hipStream_t st) {
  const HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const bool mlp = h.kind == HK_HASH_MLP;
  if (mlp && h.bits == 128) return valu_launch<BF16, true, 128>(hp, x, rows, nt, cap, t0, out, st);
  if (mlp) return valu_launch<BF16, true, 64>(hp, x, rows, nt, cap, t0, out, st);
  if (h.bits == 128) return valu_launch<BF16, false, 128>(hp, x, rows, nt, cap, t0, out, st);
  return valu_launch<BF16, false, 64>(hp, x, rows, nt, cap, t0, out, st);
}

}  // namespace

hipError_t launch_encode_keys(const hk_hash &h, const void *k, int B, int Hkv, int64_t cap,
                              int64_t t0, int64_t t1, uint32_t *codes, hipStream_t st) {
  const int64_t nt = t1 - t0;
  const int64_t total = (int64_t)B * Hkv * nt;
  if (total == 0) return hipSuccess;
  if (h.kind == HK_HASH_SIGN) {
    const dim3 grid((unsigned)((total * 16 + 255) / 256));
    uint8_t *cb = reinterpret_cast<uint8_t *>(codes);
    if (h.dtype == HK_BF16)
      hipLaunchKernelGGL(encode_keys_sign_kernel<true>, grid, dim3(256), 0, st, k, nt, cap, t0, total, cb);
    else
      hipLaunchKernelGGL(encode_keys_sign_kernel<false>, grid, dim3(256), 0, st, k, nt, cap, t0, total, cb);
    return hipGetLastError();
  }
  if (h.dtype == HK_F32) return valu_dispatch<false>(h, k, total, nt, cap, t0, codes, st);
  const HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const bool mlp = h.kind == HK_HASH_MLP;
  const bool bias = h.b1 != nullptr || h.b2 != nullptr;
  if (mlp && h.bits == 128)
    return bias ? mfma_launch<true, 128, true>(hp, k, nt, cap, t0, total, codes, st)
                : mfma_launch<true, 128, false>(hp, k, nt, cap, t0, total, codes, st);
  if (mlp)
    return bias ? mfma_launch<true, 64, true>(hp, k, nt, cap, t0, total, codes, st)
                : mfma_launch<true, 64, false>(hp, k, nt, cap, t0, total, codes, st);
  if (h.bits == 128) return mfma_launch<false, 128, false>(hp, k, nt, cap, t0, total, codes, st);
  return mfma_launch<false, 64, false>(hp, k, nt, cap, t0, total, codes, st);
}

hipError_t launch_encode_query(const hk_hash &h, const void *q, int B, int Hq, int Hkv,
                               uint32_t *qcodes, hipStream_t st) {
  const int64_t rows = (int64_t)B * Hkv;
  if (rows == 0) return hipSuccess;
  if (h.kind == HK_HASH_SIGN) {
    if (h.dtype == HK_BF16)
      hipLaunchKernelGGL(encode_query_sign_kernel<true>, dim3((unsigned)rows), dim3(128), 0, st, q, Hq, Hkv, qcodes);
    else
      hipLaunchKernelGGL(encode_query_sign_kernel<false>, dim3((unsigned)rows), dim3(128), 0, st, q, Hq, Hkv, qcodes);
    return hipGetLastError();
  }
  const HashPtrs hp{h.R, h.W1, h.b1, h.W2, h.b2};
  const bool mlp = h.kind == HK_HASH_MLP, bf = h.dtype == HK_BF16;
  if (bf) {
    const dim3 g16((unsigned)((rows + kQTile - 1) / kQTile));
    const uint16_t *qb = static_cast<const uint16_t *>(q);
    if (mlp && h.bits == 128)
      hipLaunchKernelGGL((encode_query_mfma_kernel<true, 128>), g16, dim3(1024), 0, st, hp, qb, rows, Hq, Hkv, qcodes);
    else if (mlp)
      hipLaunchKernelGGL((encode_query_mfma_kernel<true, 64>), g16, dim3(1024), 0, st, hp, qb, rows, Hq, Hkv, qcodes);
    else if (h.bits == 128)
      hipLaunchKernelGGL((encode_query_mfma_kernel<false, 128>), g16, dim3(1024), 0, st, hp, qb, rows, Hq, Hkv, qcodes);
    else
      hipLaunchKernelGGL((encode_query_mfma_kernel<false, 64>), g16, dim3(1024), 0, st, hp, qb, rows, Hq, Hkv, qcodes);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + kQRows - 1) / kQRows));
#define HK_Q(BFV, MLPV, BITSV)                                                                \
  hipLaunchKernelGGL((encode_query_kernel<BFV, MLPV, BITSV>), grid, dim3(256), 0, st, hp, q, \
                     rows, Hq, Hkv, qcodes)
  if (mlp) { if (h.bits == 128) HK_Q(false, true, 128); else HK_Q(false, true, 64); }
  else { if (h.bits == 128) HK_Q(false, false, 128); else HK_Q(false, false, 64); }
#undef HK_Q
  return hipGetLastError();
}

}  // namespace hk
