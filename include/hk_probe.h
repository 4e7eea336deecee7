/*
 * hk_probe.h -- measurement aids beside the decode path of hk.h, in a library of their own
 * (libhk_probe.so).  They are not steps of the method: a plain streaming read and a plain
 * random-row gather, whose measured rates are set beside the kernels' bandwidth figures
 * and the spec peak.  Conventions (device pointers, stream, host-side checks, status
 * codes) are those of hk.h.
 */
#ifndef HK_PROBE_H
#define HK_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "hk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* A plain streaming read of `bytes` (a multiple of 16) from device memory src (16-byte
 * aligned) with 16-byte non-temporal loads, one pass of 32 KB per workgroup (the Hamming
 * scan's access pattern): the rate that the kernels' bandwidth figures are compared with
 * beside the spec peak.
 *   sink  device uint32 array of hk_read_probe_sink_words(bytes) entries (written: the
 *         XOR of the words each workgroup read, so the loads are kept).
 * Errors: bytes not a multiple of 16, or NULL src / sink with bytes > 0 ->
 * INVALID_ARGUMENT; src not 16-byte aligned -> UNSUPPORTED; bytes = 0 enqueues nothing. */
size_t hk_read_probe_sink_words(size_t bytes);
hk_status hk_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* A plain gather of K/V rows in the access pattern of the attention (the rows a
 * partial-attention step reads; RetrievalAttention, elamur summary: Summary), so that the
 * attention kernels' gather rates can be set against the rate of a pure read of the same
 * rows.  For each of the n_idx entries of idx, reads the
 * 256-byte row idx[i] of k and of v ([table_rows][256 bytes], 16-byte aligned; a bf16
 * d = 128 K/V cache viewed as one table); entries outside [0, table_rows) read row 0.
 * Workgroup b takes entries [b*rows_per_block, (b+1)*rows_per_block).
 *   sink  device uint32 array of hk_gather_probe_sink_words(n_idx, rows_per_block)
 *         entries (written: the XOR of the words each workgroup read).
 * Errors: n_idx < 0, rows_per_block not a multiple of 16 in [16, 4096], or NULL k / v /
 * idx / sink or table_rows < 1 with n_idx > 0 -> INVALID_ARGUMENT; k or v not 16-byte
 * aligned -> UNSUPPORTED; n_idx = 0 enqueues nothing.  The sink size is 0 for invalid
 * arguments. */
size_t hk_gather_probe_sink_words(int64_t n_idx, int rows_per_block);
hk_status hk_gather_probe(const void *k, const void *v, int64_t table_rows, const int32_t *idx,
                          int64_t n_idx, int rows_per_block, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HK_PROBE_H */
