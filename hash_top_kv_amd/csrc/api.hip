// The C ABI of libhk: host-side argument checks, workspace sizing and dispatch.
// Every entry point validates on the host before enqueueing anything, launches only on
// the caller's stream, allocates nothing and keeps no state between calls.
#include <mutex>

#include "hk_internal.h"

using namespace hk;

namespace {

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

inline hk_status from_hip(hipError_t e) { return e == hipSuccess ? HK_OK : HK_ERR_HIP; }

// The kernels read and write these tensors as 16-byte (8-byte for 64-bit codes) vectors.
inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline uintptr_t code_align(int bits) { return bits == 64 ? 8 : 16; }

hk_status check_hash(const hk_hash *h) {
  if (!h) return HK_ERR_INVALID_ARGUMENT;
  if (h->dtype != HK_F32 && h->dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (h->d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (h->bits != 64 && h->bits != 128) return HK_ERR_UNSUPPORTED;
  if (h->kind == HK_HASH_LSH) {
    if (!h->R) return HK_ERR_INVALID_ARGUMENT;
    if (!aligned(h->R, 16)) return HK_ERR_UNSUPPORTED;
  } else if (h->kind == HK_HASH_MLP) {
    if (h->hidden != kHidden) return HK_ERR_UNSUPPORTED;
    if (!h->W1 || !h->W2) return HK_ERR_INVALID_ARGUMENT;
    if (!aligned(h->W1, 16) || !aligned(h->W2, 16)) return HK_ERR_UNSUPPORTED;
  } else if (h->kind == HK_HASH_SIGN) {
    if (h->bits != kHeadDim) return HK_ERR_UNSUPPORTED;
  } else {
    return HK_ERR_UNSUPPORTED;
  }
  return HK_OK;
}

hk_status check_retrieve(int bits, int B, int Hkv, int64_t cap, int64_t n_ctx, int n_sink,
                         int n_local, int k) {
  if (bits != 64 && bits != 128) return HK_ERR_UNSUPPORTED;
  if (B < 0 || Hkv < 0 || cap < 0 || n_ctx < 0 || n_sink < 0 || n_local < 0 || k < 0)
    return HK_ERR_INVALID_ARGUMENT;
  if (n_ctx > cap) return HK_ERR_INVALID_ARGUMENT;
  if (n_ctx > INT32_MAX) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv > 65535) return HK_ERR_UNSUPPORTED;
  return HK_OK;
}

// Workspace of hk_retrieve_attend_noalloc: a file-scope array that each GPU holds for the
// life of the process.  Host code never names it directly: its device address on each
// device comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the first call made
// with that device current, then kept).
hk_status static_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HK_OK;
}

}  // namespace

extern "C" {

const char *hk_strerror(hk_status s) {
  switch (s) {
    case HK_OK: return "success";
    case HK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HK_ERR_UNSUPPORTED: return "unsupported shape, dtype or code width";
    case HK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HK_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

hk_status hk_encode_keys(const hk_hash *h, const void *k, int B, int Hkv, int64_t cap,
                         int64_t t0, int64_t t1, uint32_t *codes, void *stream) {
  hk_status s = check_hash(h);
  if (s != HK_OK) return s;
  if (B < 0 || Hkv < 0 || cap < 0 || t0 < 0 || t1 < t0 || t1 > cap) return HK_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hkv * (t1 - t0) == 0) return HK_OK;
  if (!k || !codes) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(k, 16) || !aligned(codes, code_align(h->bits))) return HK_ERR_UNSUPPORTED;
  return from_hip(launch_encode_keys(*h, k, B, Hkv, cap, t0, t1, codes, as_stream(stream)));
}

hk_status hk_encode_query(const hk_hash *h, const void *q, int B, int Hq, int Hkv,
                          uint32_t *qcodes, void *stream) {
  hk_status s = check_hash(h);
  if (s != HK_OK) return s;
  if (B < 0 || Hq < 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq < Hkv) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv == 0) return HK_OK;
  if (!q || !qcodes) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16)) return HK_ERR_UNSUPPORTED;
  return from_hip(launch_encode_query(*h, q, B, Hq, Hkv, qcodes, as_stream(stream)));
}

size_t hk_retrieve_topk_workspace(int bits, int B, int Hkv, int64_t n_ctx, int n_sink,
                                  int n_local, int k) {
  if (check_retrieve(bits, B, Hkv, n_ctx, n_ctx, n_sink, n_local, k) != HK_OK) return 0;
  return plan_retrieve(bits, B, Hkv, n_ctx, n_sink, n_local, k).total;
}

hk_status hk_hamming_scan(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                          int Hkv, int64_t cap, int64_t n_ctx, int n_sink, int n_local,
                          int k, void *ws, size_t ws_bytes, void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  const RetrievePlan p = plan_retrieve(bits, B, Hkv, n_ctx, n_sink, n_local, k);
  if (p.BH == 0 || p.S == 0) return HK_OK;
  if (!codes || !qcodes || !ws) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_hamming_scan(p, codes, qcodes, cap, ws, as_stream(stream)));
}

hk_status hk_hamming_scan_query(const hk_hash *h, const void *q, int B, int Hq, int Hkv,
                                const uint32_t *codes, int64_t cap, int64_t n_ctx, int n_sink,
                                int n_local, int k, uint32_t *qcodes, void *ws, size_t ws_bytes,
                                void *stream) {
  hk_status s = check_hash(h);
  if (s != HK_OK) return s;
  if (B < 0 || Hq < 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq < Hkv) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  s = check_retrieve(h->bits, B, Hkv, cap, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  if ((int64_t)B * Hkv == 0) return HK_OK;
  if (!q || !qcodes) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16)) return HK_ERR_UNSUPPORTED;
  const RetrievePlan p = plan_retrieve(h->bits, B, Hkv, n_ctx, n_sink, n_local, k);
  if (p.S > 0) {
    if (!codes || !ws) return HK_ERR_INVALID_ARGUMENT;
    if (!aligned(codes, code_align(h->bits))) return HK_ERR_UNSUPPORTED;
    if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  }
  hipStream_t st = as_stream(stream);
  if (scan_hashes_query(p, *h))
    return from_hip(launch_hamming_scan_query(p, *h, q, Hq, Hkv, codes, cap, qcodes, ws, st));
  hipError_t e = launch_encode_query(*h, q, B, Hq, Hkv, qcodes, st);
  if (e != hipSuccess || p.S == 0) return from_hip(e);
  return from_hip(launch_hamming_scan(p, codes, qcodes, cap, ws, st));
}

hk_status hk_topk_select(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                         int k, int32_t *idx, int32_t *count, void *ws, size_t ws_bytes,
                         void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, n_ctx, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  const RetrievePlan p = plan_retrieve(bits, B, Hkv, n_ctx, n_sink, n_local, k);
  if (p.BH == 0) return HK_OK;
  if (!count || !ws || (p.keff > 0 && !idx)) return HK_ERR_INVALID_ARGUMENT;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_topk_select(p, k, idx, count, ws, as_stream(stream)));
}

hk_status hk_retrieve_topk(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                           int Hkv, int64_t cap, int64_t n_ctx, int n_sink, int n_local,
                           int k, int32_t *idx, int32_t *count, void *ws, size_t ws_bytes,
                           void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  const RetrievePlan p = plan_retrieve(bits, B, Hkv, n_ctx, n_sink, n_local, k);
  if (p.BH == 0) return HK_OK;
  if (!count || !ws || (p.keff > 0 && !idx)) return HK_ERR_INVALID_ARGUMENT;
  if (p.S > 0 && (!codes || !qcodes)) return HK_ERR_INVALID_ARGUMENT;
  if (p.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = launch_hamming_scan(p, codes, qcodes, cap, ws, as_stream(stream));
  if (e != hipSuccess) return HK_ERR_HIP;
  return from_hip(launch_topk_select(p, k, idx, count, ws, as_stream(stream)));
}

size_t hk_retrieve_attend_workspace(int bits, int B, int Hq, int Hkv, int64_t n_ctx,
                                    int n_sink, int n_local, int topk) {
  if (check_retrieve(bits, B, Hkv, n_ctx, n_ctx, n_sink, n_local, topk) != HK_OK) return 0;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0 || Hq / Hkv > kMaxGroup) return 0;
  return plan_fused(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk).total;
}

hk_status hk_retrieve_attend(const uint32_t *codes, const uint32_t *qcodes, int bits,
                             const void *q, const void *kc, const void *vc, int dtype, int B,
                             int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx, int n_sink,
                             int n_local, int topk, float scale, int32_t *idx, int32_t *count,
                             float *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, topk);
  if (s != HK_OK) return s;
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  const FusedPlan p = plan_fused(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk);
  if (!q || !count || !o || !lse || !ws) return HK_ERR_INVALID_ARGUMENT;
  if (p.parts > 0 && (!kc || !vc)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && (!codes || !qcodes)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.keff > 0 && !idx) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16)) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = as_stream(stream);
  hipError_t e = launch_hamming_scan(p.r, codes, qcodes, cap, ws, st);
  if (e == hipSuccess)
    e = launch_fused_attend(p, q, kc, vc, dtype, B, Hq, Hkv, cap, scale, topk, idx, count, o, lse,
                            ws, st);
  return from_hip(e);
}

hk_status hk_decode_step(const hk_hash *h, const void *q, const uint32_t *codes,
                         const void *kc, const void *vc, int B, int Hq, int Hkv, int d,
                         int64_t cap, int64_t n_ctx, int n_sink, int n_local, int topk,
                         float scale, uint32_t *qcodes, int32_t *idx, int32_t *count, float *o,
                         float *lse, void *ws, size_t ws_bytes, void *stream) {
  hk_status s = check_hash(h);
  if (s != HK_OK) return s;
  const int bits = h->bits, dtype = h->dtype;
  s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, topk);
  if (s != HK_OK) return s;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  const FusedPlan p = plan_fused(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk);
  if (!q || !qcodes || !count || !o || !lse || !ws) return HK_ERR_INVALID_ARGUMENT;
  if (p.parts > 0 && (!kc || !vc)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && !codes) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.keff > 0 && !idx) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16)) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = as_stream(stream);
  if (tiny_step_fits(B, Hq, Hkv, p.r.C, p.r.keff, p.n_win))
    return from_hip(launch_tiny_step(*h, p.r, q, codes, kc, vc, B, Hq, Hkv, cap, topk, scale,
                                     p.win_sinks, p.win_local0, p.n_win, qcodes, idx, count, o,
                                     lse, st));
  hipError_t e;
  if (scan_hashes_query(p.r, *h)) {
    e = launch_hamming_scan_query(p.r, *h, q, Hq, Hkv, codes, cap, qcodes, ws, st);
  } else {
    e = launch_encode_query(*h, q, B, Hq, Hkv, qcodes, st);
    if (e == hipSuccess) e = launch_hamming_scan(p.r, codes, qcodes, cap, ws, st);
  }
  if (e == hipSuccess)
    e = launch_fused_attend(p, q, kc, vc, dtype, B, Hq, Hkv, cap, scale, topk, idx, count, o, lse,
                            ws, st);
  return from_hip(e);
}

hk_status hk_retrieve_attend_noalloc(const uint32_t *codes, const uint32_t *qcodes, int bits,
                                     const void *q, const void *kc, const void *vc, int dtype,
                                     int B, int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx,
                                     int n_sink, int n_local, int topk, float scale,
                                     int32_t *idx, int32_t *count, float *o, float *lse,
                                     void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, topk);
  if (s != HK_OK) return s;
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  const FusedPlan p = plan_fused(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk);
  if (p.total > kStaticScratchBytes) return HK_ERR_WORKSPACE_TOO_SMALL;
  void *ws = nullptr;
  s = static_scratch(&ws);
  if (s != HK_OK) return s;
  return hk_retrieve_attend(codes, qcodes, bits, q, kc, vc, dtype, B, Hq, Hkv, d, cap, n_ctx,
                            n_sink, n_local, topk, scale, idx, count, o, lse, ws, p.total,
                            stream);
}

hk_status hk_select_attend(int bits, const void *q, const void *kc, const void *vc, int dtype,
                           int B, int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx,
                           int n_sink, int n_local, int topk, float scale, int32_t *idx,
                           int32_t *count, float *o, float *lse, void *ws, size_t ws_bytes,
                           void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, topk);
  if (s != HK_OK) return s;
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  const FusedPlan p = plan_fused(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk);
  if (!q || !count || !o || !lse || !ws) return HK_ERR_INVALID_ARGUMENT;
  if (p.parts > 0 && (!kc || !vc)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.keff > 0 && !idx) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16)) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = as_stream(stream);
  return from_hip(launch_fused_attend(p, q, kc, vc, dtype, B, Hq, Hkv, cap, scale, topk, idx,
                                      count, o, lse, ws, st));
}

hk_status hk_window_indices(int64_t n_ctx, int n_sink, int n_local, int32_t *idx,
                            int32_t *n_out, void *stream) {
  if (n_ctx < 0 || n_sink < 0 || n_local < 0 || !n_out) return HK_ERR_INVALID_ARGUMENT;
  if (n_ctx > INT32_MAX) return HK_ERR_UNSUPPORTED;
  const int64_t sinks = n_sink < n_ctx ? n_sink : n_ctx;
  const int64_t local0 = (n_ctx - n_local) > n_sink ? (n_ctx - n_local) : n_sink;
  const int64_t n = sinks + (n_ctx > local0 ? n_ctx - local0 : 0);
  *n_out = (int32_t)n;
  if (n == 0 || !idx) return HK_OK;   // idx == NULL: size query only
  return from_hip(launch_window_indices(n_ctx, n_sink, n_local, idx, as_stream(stream)));
}

size_t hk_sparse_decode_workspace(int B, int Hq, int Hkv, int d, int max_count) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || max_count < 0 || d != kHeadDim) return 0;
  return plan_decode(B, Hq, Hkv, max_count).total;
}

hk_status hk_sparse_decode(const void *q, const void *k, const void *v, int dtype, int B,
                           int Hq, int Hkv, int d, int64_t cap, const int32_t *idx,
                           int64_t idx_stride, const int32_t *count, int max_count,
                           float scale, float *o, float *lse, void *ws, size_t ws_bytes,
                           void *stream) {
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq < Hkv || cap < 0 || max_count < 0 ||
      idx_stride < 0)
    return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv > 65535) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  if (!q || !o || !lse) return HK_ERR_INVALID_ARGUMENT;
  if (max_count > 0 && (!k || !v || !idx)) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return HK_ERR_UNSUPPORTED;
  const DecodePlan p = plan_decode(B, Hq, Hkv, max_count);
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  if (p.total > 0 && !ws) return HK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_sparse_decode(p, q, k, v, dtype, B, Hq, Hkv, cap, idx, idx_stride,
                                       count, max_count, scale, o, lse, ws,
                                       as_stream(stream)));
}

hk_status hk_lse_merge(const float *o_parts, const float *lse_parts, int P, int64_t rows,
                       int d, float *o, float *lse, void *stream) {
  if (P < 1 || d < 1 || rows < 0) return HK_ERR_INVALID_ARGUMENT;
  if (rows == 0) return HK_OK;
  if (!o_parts || !lse_parts || !o || !lse) return HK_ERR_INVALID_ARGUMENT;
  if (rows > INT32_MAX) return HK_ERR_UNSUPPORTED;
  return from_hip(launch_lse_merge(o_parts, lse_parts, P, rows, d, o, lse, as_stream(stream)));
}

size_t hk_evict_workspace(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local) {
  if (check_retrieve(bits, B, Hkv, n_ctx, n_ctx, n_sink, n_local, 0) != HK_OK) return 0;
  return plan_evict(bits, B, Hkv, n_ctx, n_sink, n_local).total;
}

hk_status hk_evict_select(const uint32_t *codes, const uint32_t *qcodes, int bits, int B, int Hkv,
                          int64_t cap, int64_t n_ctx, int n_sink, int n_local, int32_t *victim,
                          void *ws, size_t ws_bytes, void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, n_ctx, n_sink, n_local, 0);
  if (s != HK_OK) return s;
  const EvictPlan p = plan_evict(bits, B, Hkv, n_ctx, n_sink, n_local);
  if (p.BH == 0) return HK_OK;
  if (!victim || !ws || (p.S > 0 && (!codes || !qcodes))) return HK_ERR_INVALID_ARGUMENT;
  if (p.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_evict_select(p, codes, qcodes, cap, victim, ws, as_stream(stream)));
}

hk_status hk_evict_replace(const void *k_new, const void *v_new, const uint32_t *code_new,
                           int dtype, int bits, int B, int Hkv, int d, int64_t cap,
                           const int32_t *victim, void *kc, void *vc, uint32_t *codes,
                           void *stream) {
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (bits != 64 && bits != 128) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (B < 0 || Hkv < 0 || cap < 0) return HK_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hkv == 0) return HK_OK;
  if ((int64_t)B * Hkv > 65535) return HK_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !code_new || !victim || !kc || !vc || !codes)
    return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kc, 16) || !aligned(vc, 16))
    return HK_ERR_UNSUPPORTED;
  return from_hip(launch_evict_replace(k_new, v_new, code_new, dtype == HK_BF16 ? 2 : 4, bits / 32,
                                       B * Hkv, cap, victim, kc, vc, codes, as_stream(stream)));
}

size_t hk_exact_topk_workspace(int B, int Hkv, int64_t n_ctx, int n_sink, int n_local, int k) {
  if (check_retrieve(128, B, Hkv, n_ctx, n_ctx, n_sink, n_local, k) != HK_OK) return 0;
  return plan_exact(B, Hkv, n_ctx, n_sink, n_local, k).total;
}

hk_status hk_exact_topk(const void *q, const void *kc, int dtype, int B, int Hq, int Hkv, int d,
                        int64_t cap, int64_t n_ctx, int n_sink, int n_local, int k, int32_t *idx,
                        int32_t *count, void *ws, size_t ws_bytes, void *stream) {
  hk_status s = check_retrieve(128, B, Hkv, cap, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hq < 0 || (Hkv > 0 && Hq % Hkv != 0) || (Hkv == 0 && Hq != 0)) return HK_ERR_INVALID_ARGUMENT;
  if (Hkv > 0 && Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  const ExactPlan p = plan_exact(B, Hkv, n_ctx, n_sink, n_local, k);
  if (p.BH == 0) return HK_OK;
  if (!count || !ws || (p.keff > 0 && (!idx || !q || !kc))) return HK_ERR_INVALID_ARGUMENT;
  if (p.keff > 0 && !aligned(kc, 16)) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_exact_topk(p, q, kc, dtype, Hq, Hkv, cap, k, idx, count, ws,
                                    as_stream(stream)));
}

hk_status hk_topk_intersect(const int32_t *a, const int32_t *count_a, int64_t stride_a,
                            const int32_t *b, const int32_t *count_b, int64_t stride_b,
                            int n_lists, int32_t *inter, void *stream) {
  if (n_lists < 0 || stride_a < 0 || stride_b < 0) return HK_ERR_INVALID_ARGUMENT;
  if (n_lists == 0) return HK_OK;
  if (n_lists > INT32_MAX / 2) return HK_ERR_UNSUPPORTED;
  if (!a || !count_a || !b || !count_b || !inter) return HK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_intersect(a, count_a, stride_a, b, count_b, stride_b, n_lists, inter,
                                   as_stream(stream)));
}

hk_status hk_retrieve_topk_qheads(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                                  int Hq, int Hkv, int64_t cap, int64_t n_ctx, int n_sink,
                                  int n_local, int k, int32_t *idx, int32_t *count, void *ws,
                                  size_t ws_bytes, void *stream) {
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  hk_status s = check_retrieve(bits, B, Hq, cap, n_ctx, n_sink, n_local, k);
  if (s != HK_OK) return s;
  const RetrievePlan p = plan_retrieve(bits, B, Hq, n_ctx, n_sink, n_local, k);
  if (p.BH == 0) return HK_OK;
  if (!count || !ws || (p.keff > 0 && !idx) || (p.S > 0 && (!codes || !qcodes)))
    return HK_ERR_INVALID_ARGUMENT;
  if (p.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = as_stream(stream);
  hipError_t e = launch_hamming_scan_qheads(p, Hq / Hkv, codes, qcodes, cap, ws, st);
  if (e != hipSuccess) return HK_ERR_HIP;
  return from_hip(launch_topk_select(p, k, idx, count, ws, st));
}

hk_status hk_sparse_decode_qheads(const void *q, const void *k, const void *v, int dtype, int B,
                                  int Hq, int Hkv, int d, int64_t cap, const int32_t *idx,
                                  int64_t idx_stride, const int32_t *count, int max_count,
                                  float scale, float *o, float *lse, void *ws, size_t ws_bytes,
                                  void *stream) {
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq < Hkv || cap < 0 || max_count < 0 ||
      idx_stride < 0)
    return HK_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * Hq > 65535) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  if (!q || !o || !lse) return HK_ERR_INVALID_ARGUMENT;
  if (max_count > 0 && (!k || !v || !idx)) return HK_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return HK_ERR_UNSUPPORTED;
  const DecodePlan p = plan_decode(B, Hq, Hq, max_count);
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  if (p.total > 0 && !ws) return HK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_sparse_decode(p, q, k, v, dtype, B, Hq, Hq, cap, idx, idx_stride, count,
                                       max_count, scale, o, lse, ws, as_stream(stream),
                                       Hq / Hkv));
}

hk_status hk_retrieve_attend_varlen(const uint32_t *codes, const uint32_t *qcodes, int bits,
                                    const void *q, const void *kc, const void *vc, int dtype,
                                    int B, int Hq, int Hkv, int d, int64_t cap,
                                    const int32_t *ctx_len, int64_t max_ctx, int n_sink,
                                    int n_local, int topk, float scale, int32_t *idx,
                                    int32_t *count, float *o, float *lse, void *ws,
                                    size_t ws_bytes, void *stream) {
  hk_status s = check_retrieve(bits, B, Hkv, cap, max_ctx, n_sink, n_local, topk);
  if (s != HK_OK) return s;
  if (dtype != HK_F32 && dtype != HK_BF16) return HK_ERR_UNSUPPORTED;
  if (d != kHeadDim) return HK_ERR_UNSUPPORTED;
  if (Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0) return HK_ERR_INVALID_ARGUMENT;
  if (Hq / Hkv > kMaxGroup) return HK_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq == 0) return HK_OK;
  if (!ctx_len) return HK_ERR_INVALID_ARGUMENT;
  const FusedPlan p = plan_fused(bits, B, Hq, Hkv, max_ctx, n_sink, n_local, topk);
  if (!q || !count || !o || !lse || !ws) return HK_ERR_INVALID_ARGUMENT;
  if (p.parts > 0 && (!kc || !vc)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && (!codes || !qcodes)) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.keff > 0 && !idx) return HK_ERR_INVALID_ARGUMENT;
  if (p.r.S > 0 && !aligned(codes, code_align(bits))) return HK_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16)) return HK_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return HK_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = as_stream(stream);
  hipError_t e = launch_hamming_scan(p.r, codes, qcodes, cap, ws, st, ctx_len, Hkv, n_local,
                                     max_ctx);
  if (e == hipSuccess)
    e = launch_fused_attend(p, q, kc, vc, dtype, B, Hq, Hkv, cap, scale, topk, idx, count, o, lse,
                            ws, st, ctx_len);
  return from_hip(e);
}

}  // extern "C"
