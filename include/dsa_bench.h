/*
 * dsa_bench.h - measurement kernels exported by libdsa.so beside the DSA
 * path.  They compute nothing of the method: they read memory the way the
 * path's kernels do, so a benchmark can set the path's achieved bandwidth
 * against what this GPU's HBM delivers for the same access pattern.
 *
 * Conventions as dsa.h: device pointers owned by the caller, asynchronous
 * on `stream` (hipStream_t as void*), a dsa_status return, message through
 * dsa_last_error().
 */
#ifndef DSA_BENCH_H
#define DSA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes from `src` once (16-byte nontemporal loads, each
 * 64-lane load a contiguous 1 KB run, 2048 work-groups striding over the
 * buffer) and folds them into one word written to *sink (so the reads are
 * not optimised away).  src and bytes must be 16-byte multiples/aligned;
 * sink is a device word.  Errors: INVALID_ARG. */
int dsa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Reads the indexer-key stream of a decode batch the way the scan does and
 * nothing else: for each request, the first ceil(seqlens_k[b] / 64) pages
 * named by its page-table row, each 8 KB page as eight contiguous 1 KB
 * loads, 128-page ranges per 4-wave work-group, two pages in flight per
 * wave.  k8_cache: uint8 [num_pages, 64, 128]; page_table int32 [B,
 * max_pages_per_req]; seqlens_k int32 [B] (device); max_seqlen_k bounds
 * them.  Page ids outside [0, num_pages) read nothing.  The fold of what it
 * read goes to *sink.  Errors: INVALID_ARG. */
int dsa_bench_key_stream_read(const uint8_t* k8_cache, int32_t num_pages, const int32_t* page_table,
                              int32_t batch, int32_t max_pages_per_req, const int32_t* seqlens_k,
                              int32_t max_seqlen_k, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_BENCH_H */
