/*
 * pa_bench.h — measurement helpers for libpa (not part of the attention
 * method).  They give the bandwidth ceilings the attention kernels are judged
 * against on this machine.
 *
 * Same conventions as pa.h: device pointers, caller-owned memory, work
 * enqueued on `stream` (a hipStream_t, NULL = default), no allocation, no
 * synchronisation, synchronous status codes (pa_status_t).
 */
#ifndef PA_BENCH_H_
#define PA_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read: every byte of src[0, bytes) is read once with 16-byte
 * vector loads (bytes must be a multiple of 16, src 16-byte aligned); one
 * 32-bit XOR of all data is OR-ed into *sink so the reads cannot be elided.
 */
pa_status_t pa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Paged read: the K and V rows of every sequence's first seq_lens[s] tokens,
 * for every KV head, read through block_tables exactly as the decode kernel
 * reads them (head_dim 128, 16-bit elements, block_size % 16 == 0, parts of
 * at most 768 tokens per wave) with no arithmetic on them.  Bytes read =
 * sum(seq_lens rounded up to 16) * 2 * num_kv_heads * 256.  *sink as above.
 */
pa_status_t pa_bench_paged_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H_ */
