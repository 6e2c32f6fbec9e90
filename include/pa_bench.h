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

/*
 * Per-kernel timing.  Between pa_bench_timing_begin() and
 * pa_bench_timing_end(), every kernel the library launches (from any entry
 * point, on any stream) is bracketed by two hipEvents recorded on the stream
 * it is launched on.  pa_bench_timing_end() waits for those events and
 * returns, per kernel name, the number of launches and their summed
 * duration in milliseconds (entries sorted by descending total; at most
 * max_entries are written, *n_entries receives the number written).  Events
 * come from a pool owned by the library; not thread-safe.  Timing adds a few
 * microseconds per launch: use it to split time among kernels, not for the
 * headline clock.
 */
typedef struct {
  char name[64];
  int32_t launches;
  double total_ms;
} pa_kernel_time_t;

pa_status_t pa_bench_timing_begin(void);
pa_status_t pa_bench_timing_end(pa_kernel_time_t* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* PA_BENCH_H_ */
