/*
 * hk.h -- C ABI of the binary-hash KV-cache retrieval decode path for MI355X (gfx950).
 *
 * One decode step of binary-hash retrieval attention:
 *   1. keys and the current query are hashed to packed sign-bit codes, by a Gaussian
 *      random projection (HashEvict: Abstract, "binarized Gaussian projections") or by
 *      the sign of a two-layer MLP (Spotlight Attention: Approach);
 *   2. the cached key codes are compared with the query code by Hamming distance
 *      (HashEvict: Abstract; Spotlight Attention: Key results, "bitwise hashing
 *      retrieval");
 *   3. the top-k tokens per head are kept (Spotlight Attention: summary, top-2%);
 *   4. exact softmax attention runs over those tokens only, and over a static
 *      sink + local window (RetrievalAttention, elamur summary: Summary);
 *   5. the partial results are combined by exact log-sum-exp rescaling
 *      (RetrievalAttention, atlas summary: Approach).
 *
 * Conventions shared by every call:
 *  - Pointers named as device pointers are caller-owned device memory; the library
 *    allocates no device memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call only
 *    enqueues kernels on it and returns; nothing synchronises and nothing reads device
 *    memory from the host.  Device faults surface at the caller's next synchronisation.
 *  - Arguments are checked on the host before anything is enqueued.  A bad argument
 *    returns HK_ERR_INVALID_ARGUMENT or HK_ERR_UNSUPPORTED and enqueues nothing.  A
 *    failed launch returns HK_ERR_HIP.
 *  - Head dimension d is 128.  Code widths are 64 or 128 bits, stored as bits/32
 *    uint32 words per token: bit j is bit (j mod 32) of word j/32 (least significant
 *    first), words in increasing order.  A bit is 1 iff its pre-sign value is > 0.
 *  - GQA: query head h belongs to KV head h / G with G = Hq / Hkv (contiguous groups).
 *  - Token indices are int32; contexts are limited to 2^31 - 1 tokens.
 *  - Alignment: hash weights (R, W1, W2), keys, queries, K/V caches and key codes are
 *    read or written as 16-byte vectors (8-byte for 64-bit codes); a pointer that is not
 *    aligned to that returns HK_ERR_UNSUPPORTED.  (Allocations from hipMalloc and
 *    PyTorch are 256-byte aligned; row strides are multiples of 16 bytes by the shapes.)
 */
#ifndef HK_H
#define HK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hk_status {
  HK_OK = 0,
  HK_ERR_INVALID_ARGUMENT = 1,
  HK_ERR_UNSUPPORTED = 2,
  HK_ERR_WORKSPACE_TOO_SMALL = 3,
  HK_ERR_HIP = 4
} hk_status;

typedef enum hk_dtype { HK_F32 = 0, HK_BF16 = 1 } hk_dtype;

typedef enum hk_hash_kind { HK_HASH_LSH = 0, HK_HASH_MLP = 1, HK_HASH_SIGN = 2 } hk_hash_kind;

/* Hash parameters: a host struct that points at caller-owned device tensors.
 * LSH  (HashEvict: Abstract): y = R x, R [bits][d] row-major, row j gives bit j.
 * MLP  (Spotlight Attention: Approach): y = W2 rho(GELU(W1 x + b1)) + b2 with
 *      W1 [hidden][d], W2 [bits][hidden] ([out][in], row-major), optional biases
 *      b1 [hidden] and b2 [bits] (NULL = zero), GELU in its exact erf form, and rho the
 *      rounding of the hidden activation to bf16 (nearest-even) when dtype is HK_BF16.
 * SIGN (Self-Indexing KVCache: Abstract, "sign-based 1-bit" keys): y = x, the identity
 *      projection; bits = d = 128 and no weight tensors (R, W1, W2, b1, b2 are ignored).
 * All tensors have element type `dtype`, which is also the element type of the keys and
 * queries the hash encodes.  d must be 128, bits 64 or 128 (128 for SIGN), hidden 256
 * (MLP) or 0. */
typedef struct hk_hash {
  int32_t kind;    /* hk_hash_kind */
  int32_t dtype;   /* hk_dtype */
  int32_t d;
  int32_t bits;
  int32_t hidden;
  const void *R;
  const void *W1;
  const void *b1;
  const void *W2;
  const void *b2;
} hk_hash;

/* Static string describing a status; never NULL. */
const char *hk_strerror(hk_status s);

/* Encode cached keys into codes (prefill: t0 = 0, t1 = n; append: t1 = t0 + 1).
 * Spotlight Attention (Approach) hashes keys with the sign of an MLP; HashEvict
 * (Abstract) with a binarized Gaussian projection kept in a GPU-resident structure.
 *   k      device [B][Hkv][cap][d], element type h->dtype.
 *   codes  device [B][Hkv][cap][bits/32] uint32; tokens t0 <= t < t1 of every (b, head)
 *          are written, nothing else.
 * Errors: t0 < 0, t1 < t0, t1 > cap, negative B/Hkv, NULL pointers -> INVALID_ARGUMENT;
 * unsupported hash shape -> UNSUPPORTED.  t0 == t1 or B*Hkv == 0 enqueues nothing. */
hk_status hk_encode_keys(const hk_hash *h, const void *k, int B, int Hkv, int64_t cap,
                         int64_t t0, int64_t t1, uint32_t *codes, void *stream);

/* Encode the query of one decode step, one code per KV head: the code of the mean of
 * the G query vectors of the head's group (the mean ranks keys by the group's summed
 * logit), computed in fp32 without rounding the mean.
 *   q       device [B][Hq][d], element type h->dtype.
 *   qcodes  device [B][Hkv][bits/32] uint32 (written).
 * Errors: Hq % Hkv != 0, NULL pointers -> INVALID_ARGUMENT; G = Hq / Hkv > 8 ->
 * UNSUPPORTED. */
hk_status hk_encode_query(const hk_hash *h, const void *q, int B, int Hq, int Hkv,
                          uint32_t *qcodes, void *stream);

/* Workspace bytes needed by hk_retrieve_topk / hk_hamming_scan / hk_topk_select. */
size_t hk_retrieve_topk_workspace(int bits, int B, int Hkv, int64_t n_ctx, int n_sink,
                                  int n_local, int k);

/* Per-head top-k retrieval by Hamming distance (HashEvict: Abstract; Spotlight
 * Attention: Key results).  Candidates of every (b, head) are tokens
 * n_sink <= t < n_ctx - n_local (sink and local tokens are attended separately);
 * k_eff = min(k, max(0, n_ctx - n_sink - n_local)) of them are selected by
 * (distance ascending, token index ascending), a unique set.
 *   codes   device [B][Hkv][cap][bits/32]; qcodes device [B][Hkv][bits/32].
 *   idx     device [B][Hkv][k] int32: the first k_eff entries of each row are the
 *           selected tokens in ascending order; later entries are left untouched.
 *   count   device [B][Hkv] int32, set to k_eff.
 *   ws      device workspace of at least hk_retrieve_topk_workspace(...) bytes, 256-byte
 *           aligned; its contents on entry do not matter.
 * Errors: bits not 64/128 -> UNSUPPORTED; n_ctx > cap, negative sizes, NULL pointers ->
 * INVALID_ARGUMENT; small ws -> WORKSPACE_TOO_SMALL. */
hk_status hk_retrieve_topk(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                           int Hkv, int64_t cap, int64_t n_ctx, int n_sink, int n_local,
                           int k, int32_t *idx, int32_t *count, void *ws, size_t ws_bytes,
                           void *stream);

/* The two halves of hk_retrieve_topk, for callers that time or overlap them
 * separately; called in this order with the same arguments and workspace they produce
 * exactly what hk_retrieve_topk produces.  hk_hamming_scan reads every candidate code
 * once and leaves per-token distances and per-chunk distance histograms in ws;
 * hk_topk_select derives the distance threshold and the tie quota from them and writes
 * idx and count. */
hk_status hk_hamming_scan(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                          int Hkv, int64_t cap, int64_t n_ctx, int n_sink, int n_local,
                          int k, void *ws, size_t ws_bytes, void *stream);
/* hk_encode_query followed by hk_hamming_scan in one call: the query code of every
 * (b, KV head) -- the code of the group mean of its G query rows, as hk_encode_query
 * defines it -- and the scan of the cached codes against it.  For a small scan (at most
 * 512 scan workgroups, see hk_retrieve_topk_workspace's plan) every scan workgroup
 * computes its head's code itself in fp32 from q and the hash weights, which saves the
 * encoder's kernel and its dependent round trip in a latency-bound step; larger scans
 * run the two kernels.  fp32 and sign hashes give hk_encode_query's codes bit for bit;
 * bf16 LSH and MLP hashes computed inside the scan use the fp32 arithmetic of the fp32
 * encoder instead of the matrix cores, so a code bit can differ from hk_encode_query's
 * only where the pre-sign value is within fp32 rounding of zero.
 *   h, q, B, Hq, Hkv  as hk_encode_query; codes, cap, n_ctx, n_sink, n_local, k, ws,
 *           ws_bytes as hk_hamming_scan (bits = h->bits).
 *   qcodes  device [B][Hkv][bits/32] uint32 (written): the codes the scan used.
 * A following hk_topk_select or hk_select_attend continues from ws as after
 * hk_hamming_scan.  Errors: those of hk_encode_query and hk_hamming_scan. */
hk_status hk_hamming_scan_query(const hk_hash *h, const void *q, int B, int Hq, int Hkv,
                                const uint32_t *codes, int64_t cap, int64_t n_ctx, int n_sink,
                                int n_local, int k, uint32_t *qcodes, void *ws, size_t ws_bytes,
                                void *stream);
hk_status hk_topk_select(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local,
                         int k, int32_t *idx, int32_t *count, void *ws, size_t ws_bytes,
                         void *stream);

/* Workspace bytes needed by hk_retrieve_attend. */
size_t hk_retrieve_attend_workspace(int bits, int B, int Hq, int Hkv, int64_t n_ctx,
                                    int n_sink, int n_local, int topk);

/* One decode step after the query hash, fused: Hamming top-k retrieval as
 * hk_retrieve_topk (same idx and count), then exact attention of every query head over
 * its KV head's selected tokens together with the static sink + local window
 * [0, min(n_sink, n_ctx)) U [max(n_sink, n_ctx - n_local), n_ctx), i.e. the log-sum-exp
 * merge of the two partial attentions (RetrievalAttention, atlas summary: Approach;
 * Spotlight Attention: summary).  Equal, up to floating-point rounding, to
 * hk_retrieve_topk + hk_sparse_decode over idx + hk_sparse_decode over the window +
 * hk_lse_merge, in fewer kernels: each chunk's workgroup attends directly over the
 * tokens it selects.
 *   codes, qcodes, bits, cap, n_ctx, n_sink, n_local, topk, idx, count: as in
 *               hk_retrieve_topk (idx may be NULL when no token can be selected).
 *   q, kc, vc, dtype, d, scale: as q, k, v, dtype, d, scale of hk_sparse_decode.
 *   o, lse      device float [B][Hq][d] and [B][Hq] (written): the merged attention; an
 *               empty selection and window give o = 0, lse = -inf.
 *   ws          hk_retrieve_attend_workspace(...) bytes, 256-byte aligned, contents on
 *               entry irrelevant.
 * Errors: as hk_retrieve_topk and hk_sparse_decode. */
hk_status hk_retrieve_attend(const uint32_t *codes, const uint32_t *qcodes, int bits,
                             const void *q, const void *kc, const void *vc, int dtype, int B,
                             int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx, int n_sink,
                             int n_local, int topk, float scale, int32_t *idx, int32_t *count,
                             float *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/* hk_retrieve_attend without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
 * The workspace is a 64 MiB array that the library holds on each GPU it runs on until the
 * process ends (enough for 16 sequences x 128K tokens x 8 KV heads); the call allocates
 * nothing and frees nothing.  Arguments, results and errors are those of
 * hk_retrieve_attend; a problem whose workspace, hk_retrieve_attend_workspace(...), exceeds
 * 64 MiB returns HK_ERR_WORKSPACE_TOO_SMALL and enqueues nothing.  All calls on one GPU
 * share the array: calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give undefined results.  The array's contents on
 * entry do not matter. */
hk_status hk_retrieve_attend_noalloc(const uint32_t *codes, const uint32_t *qcodes, int bits,
                                     const void *q, const void *kc, const void *vc, int dtype,
                                     int B, int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx,
                                     int n_sink, int n_local, int topk, float scale,
                                     int32_t *idx, int32_t *count, float *o, float *lse,
                                     void *stream);

/* The part of hk_retrieve_attend that follows the Hamming scan: called after
 * hk_hamming_scan(codes, qcodes, bits, B, Hkv, cap, n_ctx, n_sink, n_local, topk, ws, ...)
 * on the same stream and workspace (of hk_retrieve_attend_workspace(...) bytes), it
 * produces exactly what hk_retrieve_attend produces.  For callers that time or overlap
 * the scan separately. */
hk_status hk_select_attend(int bits, const void *q, const void *kc, const void *vc, int dtype,
                           int B, int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx,
                           int n_sink, int n_local, int topk, float scale, int32_t *idx,
                           int32_t *count, float *o, float *lse, void *ws, size_t ws_bytes,
                           void *stream);

/* Write the static window [0, min(s, n)) U [max(s, n - w), n) in ascending order
 * (tokens kept by fixed patterns: RetrievalAttention, elamur summary: Summary).
 *   idx    device int32 array of at least *n_out entries (written), or NULL to
 *          only query the size (nothing is enqueued then).
 *   n_out  host int32: receives the window size, computed on the host.
 * Errors: negative sizes, NULL n_out -> INVALID_ARGUMENT. */
hk_status hk_window_indices(int64_t n_ctx, int n_sink, int n_local, int32_t *idx,
                            int32_t *n_out, void *stream);

/* Workspace bytes needed by hk_sparse_decode. */
size_t hk_sparse_decode_workspace(int B, int Hq, int Hkv, int d, int max_count);

/* Exact softmax attention of every query head over its KV head's token list
 * ("partial attention" over retrieved tokens: RetrievalAttention, elamur summary:
 * Summary; Spotlight Attention: summary).  For query head h of batch b with KV head
 * g = h / G: l_j = scale * q . K[b][g][j] over j in the list, o = sum softmax(l)_j V_j,
 * lse = ln sum exp(l_j).  The K/V rows of a list are read once and shared by the G query
 * heads of the group; accumulation is fp32.
 *   q, k, v     device; q [B][Hq][d], k and v [B][Hkv][cap][d], element type dtype.
 *   idx         device int32; list of (b, g) starts at idx + (b*Hkv + g) * idx_stride
 *               (idx_stride 0 = one list shared by all heads); entries must be in
 *               [0, cap).
 *   count       device int32 [B][Hkv], entries clamped to [0, max_count]; NULL = every
 *               list has max_count entries.
 *   max_count   host upper bound of the list lengths (sizes the launch).
 *   o, lse      device float [B][Hq][d] and [B][Hq] (written).  An empty list gives
 *               o = 0 and lse = -inf.
 *   ws          device workspace of hk_sparse_decode_workspace(...) bytes (split-K
 *               partials), 256-byte aligned.
 * Errors: d != 128 or G > 8 -> UNSUPPORTED; Hq % Hkv != 0, NULL pointers, negative
 * sizes -> INVALID_ARGUMENT; small ws -> WORKSPACE_TOO_SMALL. */
hk_status hk_sparse_decode(const void *q, const void *k, const void *v, int dtype, int B,
                           int Hq, int Hkv, int d, int64_t cap, const int32_t *idx,
                           int64_t idx_stride, const int32_t *count, int max_count,
                           float scale, float *o, float *lse, void *ws, size_t ws_bytes,
                           void *stream);

/* Exact log-sum-exp merge of P partial attentions of disjoint token sets
 * (RetrievalAttention, atlas summary: Approach):  m = max_p lse_p,
 * o = sum_p e^(lse_p - m) o_p / sum_p e^(lse_p - m),  lse = m + ln sum_p e^(lse_p - m).
 * Parts with lse = -inf are ignored; if all are, o = 0 and lse = -inf.
 *   o_parts [P][rows][d], lse_parts [P][rows] device float; o [rows][d], lse [rows]
 *   device float (written; may not alias the parts).
 * Errors: P < 1, d < 1, rows < 0, NULL pointers -> INVALID_ARGUMENT. */
hk_status hk_lse_merge(const float *o_parts, const float *lse_parts, int P, int64_t rows,
                       int d, float *o, float *lse, void *stream);

/* Workspace bytes needed by hk_evict_select (8 bytes per chunk of 2048 candidates). */
size_t hk_evict_workspace(int bits, int B, int Hkv, int64_t n_ctx, int n_sink, int n_local);

/* HashEvict's victim of one decode step (HashEvict: Abstract): per (b, head), the
 * candidate n_sink <= t < n_ctx - n_local whose key code is farthest from the query code
 * in Hamming distance -- the token least similar to the current query, expected to get
 * the lowest attention score -- with ties going to the lowest token index.
 *   codes, qcodes, bits, cap, n_ctx, n_sink, n_local: as in hk_retrieve_topk.
 *   victim  device int32 [B][Hkv] (written): the victim's token index, or -1 when the
 *           head has no candidate.
 *   ws      device workspace of hk_evict_workspace(...) bytes, 256-byte aligned.
 * Errors: as hk_retrieve_topk. */
hk_status hk_evict_select(const uint32_t *codes, const uint32_t *qcodes, int bits, int B, int Hkv,
                          int64_t cap, int64_t n_ctx, int n_sink, int n_local, int32_t *victim,
                          void *ws, size_t ws_bytes, void *stream);

/* The current token takes the victim's slot (HashEvict: Abstract): for every (b, head)
 * with 0 <= victim < cap, K[b][head][victim] = k_new[b][head], V[...] = v_new[b][head]
 * and codes[b][head][victim] = code_new[b][head]; heads with any other victim are left
 * unchanged.  code_new is the new key's code, e.g. from hk_encode_query with Hq = Hkv
 * (G = 1, the code of the key itself).
 *   k_new, v_new  device [B][Hkv][d], element type dtype.
 *   code_new      device uint32 [B][Hkv][bits/32].
 *   victim        device int32 [B][Hkv], e.g. from hk_evict_select.
 *   kc, vc        device [B][Hkv][cap][d]; codes device uint32 [B][Hkv][cap][bits/32].
 * Errors: d != 128, bits not 64/128 -> UNSUPPORTED; negative sizes, NULL pointers ->
 * INVALID_ARGUMENT. */
hk_status hk_evict_replace(const void *k_new, const void *v_new, const uint32_t *code_new,
                           int dtype, int bits, int B, int Hkv, int d, int64_t cap,
                           const int32_t *victim, void *kc, void *vc, uint32_t *codes,
                           void *stream);

/* Workspace bytes needed by hk_exact_topk (about 4 bytes per candidate). */
size_t hk_exact_topk_workspace(int B, int Hkv, int64_t n_ctx, int n_sink, int n_local, int k);

/* Exact top-k by attention logit: the "oracle top-k" that Spotlight Attention measures
 * its hash retrieval against (Key results) and the exact Flat search of
 * RetrievalAttention (atlas summary: Results).  Per (b, KV head g), the candidates
 * n_sink <= t < n_ctx - n_local are ranked by the group's summed logit
 * sum_{h in group g} q_h . K[b][g][t] (computed in fp32), largest first, ties to the
 * lower token; k_eff = min(k, number of candidates) are selected.
 *   q, kc, dtype, B, Hq, Hkv, d, cap: as hk_sparse_decode (q, k).
 *   idx, count, ws: as hk_retrieve_topk (ascending token order; ws of
 *                   hk_exact_topk_workspace(...) bytes).
 * Errors: as hk_retrieve_topk and hk_sparse_decode. */
hk_status hk_exact_topk(const void *q, const void *kc, int dtype, int B, int Hq, int Hkv, int d,
                        int64_t cap, int64_t n_ctx, int n_sink, int n_local, int k, int32_t *idx,
                        int32_t *count, void *ws, size_t ws_bytes, void *stream);

/* Sizes of the intersections of n_lists pairs of ascending token lists: list l of a is
 * a + l*stride_a with count_a[l] entries (clamped to [0, stride_a]), likewise for b;
 * inter[l] = |A_l n B_l|.  With |A_l u B_l| = count_a[l] + count_b[l] - inter[l] this
 * gives the retrieval IoU of Spotlight Attention (Key results).
 *   a, count_a, b, count_b  device int32; inter device int32 [n_lists] (written).
 * Errors: negative sizes, NULL pointers -> INVALID_ARGUMENT. */
hk_status hk_topk_intersect(const int32_t *a, const int32_t *count_a, int64_t stride_a,
                            const int32_t *b, const int32_t *count_b, int64_t stride_b,
                            int n_lists, int32_t *inter, void *stream);

/* Per-query-head retrieval, the GQA choice of RetrievalAttention (elamur summary:
 * Summary -- an index per query head): one top-k set per query head instead of one per
 * KV head.  Query head h (of KV head h / G, G = Hq / Hkv) compares its own code
 * qcodes[b][h] with the codes of its KV head; selection as hk_retrieve_topk.  Each
 * cached code is read once for the whole group.
 *   codes   device [B][Hkv][cap][bits/32]; qcodes device [B][Hq][bits/32], e.g. from
 *           hk_encode_query with Hkv = Hq (each head's own query).
 *   idx     device int32 [B][Hq][k]; count device int32 [B][Hq].
 *   ws      hk_retrieve_topk_workspace(bits, B, Hq, ...) bytes (the workspace of Hq heads).
 * Errors: as hk_retrieve_topk; Hq % Hkv != 0 -> INVALID_ARGUMENT; G > 8 -> UNSUPPORTED. */
hk_status hk_retrieve_topk_qheads(const uint32_t *codes, const uint32_t *qcodes, int bits, int B,
                                  int Hq, int Hkv, int64_t cap, int64_t n_ctx, int n_sink,
                                  int n_local, int k, int32_t *idx, int32_t *count, void *ws,
                                  size_t ws_bytes, void *stream);

/* Attention of every query head over its own token list (per-query-head selection):
 * as hk_sparse_decode, except that the list of query head h of batch b starts at
 * idx + (b*Hq + h) * idx_stride with count[b][h] entries, and is scored against the K/V
 * rows of KV head h / G.  ws: hk_sparse_decode_workspace(B, Hq, Hq, d, max_count) bytes.
 * Errors: as hk_sparse_decode. */
hk_status hk_sparse_decode_qheads(const void *q, const void *k, const void *v, int dtype, int B,
                                  int Hq, int Hkv, int d, int64_t cap, const int32_t *idx,
                                  int64_t idx_stride, const int32_t *count, int max_count,
                                  float scale, float *o, float *lse, void *ws, size_t ws_bytes,
                                  void *stream);

/* The whole decode step of one layer from the query: hk_encode_query, then
 * hk_retrieve_attend (Spotlight Attention: Approach; RetrievalAttention, atlas summary:
 * Approach), with the query hash computed inside the scan where the scan is small
 * (hk_hamming_scan_query).  Heads with one query head each (Hq == Hkv), at most 4096
 * candidates and at most 1024 selected + window rows (and at most 256 heads) run the
 * whole step in one workgroup per head: the query hash, the scan, the selection and
 * one attention pass over the selected and window tokens together, with no partials
 * and no merge.  Everything else runs the kernels of hk_hamming_scan_query and
 * hk_select_attend.
 *   h, q         as hk_encode_query; q, kc and vc have element type h->dtype.
 *   codes, kc, vc, B, Hq, Hkv, d, cap, n_ctx, n_sink, n_local, topk, scale, idx, count,
 *   o, lse, ws, ws_bytes  as hk_retrieve_attend (ws of hk_retrieve_attend_workspace(
 *                h->bits, ...) bytes).
 *   qcodes       device [B][Hkv][bits/32] uint32 (written): the query codes used, as
 *                hk_hamming_scan_query reports them.
 * idx and count are those of hk_retrieve_topk for these query codes; o and lse agree
 * with hk_retrieve_attend's to rounding (the single pass sums the two parts in another
 * order than the merge).  Errors: those of hk_encode_query and hk_retrieve_attend. */
hk_status hk_decode_step(const hk_hash *h, const void *q, const uint32_t *codes,
                         const void *kc, const void *vc, int B, int Hq, int Hkv, int d,
                         int64_t cap, int64_t n_ctx, int n_sink, int n_local, int topk,
                         float scale, uint32_t *qcodes, int32_t *idx, int32_t *count, float *o,
                         float *lse, void *ws, size_t ws_bytes, void *stream);

/* hk_retrieve_attend for a batch of sequences of their own lengths: sequence b holds
 * ctx_len[b] cached tokens (clamped to [0, max_ctx]); its candidates, budget
 * k_eff = min(topk, candidates), window and count follow its own length, exactly as a
 * call of hk_retrieve_attend with n_ctx = ctx_len[b] on that sequence alone.
 *   ctx_len  device int32 [B].
 *   max_ctx  host: an upper bound of the lengths (<= cap), which sizes the launch and the
 *            workspace: hk_retrieve_attend_workspace(bits, B, Hq, Hkv, max_ctx, ...).
 * Other arguments and errors as hk_retrieve_attend; ctx_len NULL -> INVALID_ARGUMENT. */
hk_status hk_retrieve_attend_varlen(const uint32_t *codes, const uint32_t *qcodes, int bits,
                                    const void *q, const void *kc, const void *vc, int dtype,
                                    int B, int Hq, int Hkv, int d, int64_t cap,
                                    const int32_t *ctx_len, int64_t max_ctx, int n_sink,
                                    int n_local, int topk, float scale, int32_t *idx,
                                    int32_t *count, float *o, float *lse, void *ws,
                                    size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HK_H */
