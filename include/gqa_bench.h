/*
 * gqa_bench.h — measurement aid exported by libgqa_decode.so.  Not part of
 * the decode path: it gives the practical HBM read rate of the machine, the
 * second denominator (beside the 8 TB/s peak) that the attention kernels'
 * effective bandwidth is reported against.
 */
#ifndef GQA_BENCH_H
#define GQA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at device pointer `src` (16-byte aligned,
 * bytes a multiple of 16) by `workgroups` workgroups of 256 threads, each
 * reading a grid-stride share in 16-byte non-temporal loads.  Workgroup w
 * writes the XOR of all 32-bit words it read to sink[w] (device memory of
 * `workgroups` uint32 words, owned by the caller), so the XOR of
 * sink[0 .. workgroups) equals the XOR of every word of the buffer.
 * Enqueued on `stream`; never synchronises, allocates nothing.
 * Errors: GQA_ERR_NULL (src or sink NULL), GQA_ERR_SHAPE (misaligned src,
 * bytes not a multiple of 16, workgroups < 1); > 0: hipError_t of the
 * launch. */
int gqa_bench_stream_read(const void *src, size_t bytes, uint32_t *sink, int workgroups,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_BENCH_H */
