/*
 * pa.h — ragged paged attention for continuous batching, MI355X (gfx950).
 *
 * One step of continuous batching flattens the step's new tokens of S
 * sequences into one [T] batch, writes their K/V into a paged cache through
 * slot_mapping, then attends each new query row to its own sequence's cached
 * K/V through that sequence's block table, causally.  Prefill chunks and
 * decode tokens share the batch.
 *
 * Pages cited below:
 *   [FS] "vLLM Continuous Batching：从 Forward Shape 理解两个核心参数"
 *   [VP] "vLLM 原理"
 *   [CB] "LLM 推理引擎 Continuous Batching 与 PagedAttention：从 vLLM 原理到生产级部署实战"
 *   [BN] "vLLM 学习笔记（2）：从单请求到批处理"
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to caller-owned, contiguous,
 *     row-major memory.  The library never allocates or frees device memory
 *     and never waits for the device on the host (unless the plan trace of
 *     pa_set_trace is on); all work is enqueued on
 *     `stream` (a hipStream_t; NULL = default stream) and is complete when
 *     that stream is.  The caller owns the KV cache (the engine allocates
 *     one pool and hands out per-layer views, [VP] §3.6).
 *   - One exception, in pa_attention and pa_write_kv_attention only: on a
 *     large mixed batch (prefill rows, head_dim 128, a block size that is a
 *     multiple of 16, at least 64 sequences and at most 64 new tokens per
 *     sequence on average) the prefill kernel (and the two-tile decode
 *     launch after it) runs on a side stream beside the one-tile decode
 *     launch, which stays on `stream`.  That stream
 *     (non-blocking, default priority) and its two events are created by
 *     the library on the first such call on a device and kept until the
 *     process ends; the fork from and join back into `stream` are event
 *     records and waits made under a process-wide lock, so the call still
 *     completes with `stream`.  pa_attention_noalloc never uses it.
 *   - Host-checkable problems (null pointers, bad sizes, unsupported shapes,
 *     a too-small workspace, a failed launch) are returned synchronously as
 *     pa_status_t and nothing is enqueued.
 *   - Data-dependent problems found on the device are OR-ed into *d_err (an
 *     int32 in device memory, may be NULL) as PA_DERR_* bits; the caller reads
 *     it whenever it likes.  Outputs of rows touched by such a problem are
 *     unspecified, but no access ever leaves the buffers described here.
 *   - int32 is used for every index, as the pages' metadata is int32.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,   /* IEEE float32 */
  PA_BF16 = 1,  /* bfloat16 */
  PA_F16 = 2    /* IEEE float16 */
} pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,        /* a size argument is negative, zero where it must not be, or overflows int32 indexing */
  PA_ERR_DTYPE = 3,        /* unknown dtype */
  PA_ERR_UNSUPPORTED = 4,  /* well formed but not implemented (e.g. head_dim > 256) */
  PA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than pa_attention_workspace_size() */
  PA_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed */
  PA_ERR_VALUE = 7         /* a non-size argument is invalid (a non-finite softmax scale) */
} pa_status_t;

/* Device-side data-error bits (OR-ed into *d_err). */
enum {
  PA_DERR_QLEN_GT_SEQLEN = 1,  /* query_len < 0, seq_len < 0 or query_len > seq_len */
  PA_DERR_TOKEN_SUM = 2,       /* sum(query_lens) != num_tokens, or query_start_loc inconsistent */
  PA_DERR_BLOCK_OOB = 4,       /* a block-table entry a sequence needs is < 0 or >= num_blocks,
                                  or the table is too narrow for seq_len */
  PA_DERR_SLOT_OOB = 8,        /* a slot_mapping entry >= num_blocks * block_size */
  PA_DERR_OVERFLOW = 16,       /* a prefix sum exceeds INT32_MAX */
  PA_DERR_HINT = 32,           /* pa_attention: a query_len exceeds the max_query_len hint */
  PA_DERR_DUP_SLOT = 64        /* pa_write_kv with validation on: two rows share a slot */
};

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status_t s);

/* Description of the HIP error behind the most recent PA_ERR_HIP returned
 * to this thread ("" if none).  Static storage, valid until the next call. */
const char* pa_last_hip_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t pa_version(void);

/*
 * Kernel selection for pa_attention, process-wide (not thread-safe against
 * concurrent pa_attention calls; meant for tests and tuning):
 *   PA_POLICY_AUTO (default)  fast paths where supported, generic elsewhere
 *   PA_POLICY_GENERIC         always the generic fp32 kernel
 *   PA_POLICY_FAST            fast paths only; PA_ERR_UNSUPPORTED otherwise
 * Returns the previous policy, or -1 for an unknown value (unchanged).
 */
enum { PA_POLICY_AUTO = 0, PA_POLICY_GENERIC = 1, PA_POLICY_FAST = 2 };
int32_t pa_set_kernel_policy(int32_t policy);

/*
 * Input validation, process-wide (same thread-safety as the kernel policy):
 * 1 = on, 0 = off (the default, or on when the environment variable
 * PA_VALIDATE is set to anything but "" or "0" when the library is loaded).
 * With it on, pa_write_kv with a non-NULL d_err
 * also checks that no two rows of the call share an in-range slot and flags
 * PA_DERR_DUP_SLOT if they do ([VP] §2.1: copy-on-write keeps writers apart,
 * so a repeated slot is invalid input).  The check is one extra launch of
 * O(num_tokens^2) compares: a debugging aid.  Returns the previous setting,
 * or -1 for a value other than 0 or 1 (unchanged).
 */
int32_t pa_set_validation(int32_t on);

/*
 * Plan trace, process-wide (same thread-safety as the kernel policy): 1 = on,
 * 0 = off (the default, or on when the environment variable PA_TRACE is set
 * to anything but "" or "0" when the library is loaded).  With it on, every
 * pa_attention or pa_write_kv_attention call that launched its kernels then
 * waits for its stream, copies its work plan from the workspace to the host
 * and prints it to stderr, each line starting with "[pa_trace]": the path
 * taken, the work split (query heads per KV head, decode parts, rows per
 * decode item, whether prefill rows and shared prefixes are planned, whether
 * the decode launches ran beside the prefill kernel, where the KV write of
 * pa_write_kv_attention ran, workspace bytes),
 * the prefill list (prefill query tiles and shared-prefix parts), every
 * shared-prefix group (its members, prefix tokens and parts), the first
 * entries of each decode list, and d_err.  The wait makes it a debugging aid:
 * not for timing or graph capture.  pa_attention_noalloc never traces.
 * Returns the previous setting, or -1 for a value other than 0 or 1
 * (unchanged).
 */
int32_t pa_set_trace(int32_t on);

/*
 * pa_build_metadata — flat-batch metadata of one step.
 *
 * [FS] §2.1 (query_start_loc is a prefix sum with the total appended; each
 * new token's position; seq_lens after the step), [BN] (lengths 3,5,2 give
 * [0,3,8,10]), [VP] §3.7 (cu_seqlens_q / cu_seqlens_k), [FS] §2.3 第一步 and
 * 第二步 (slot = physical block * block_size + offset, found through the
 * sequence's block table at logical block pos / block_size).
 *
 * Inputs:
 *   query_lens [S]   new tokens of each sequence this step (>= 0)
 *   seq_lens   [S]   KV length of each sequence after this step, new tokens
 *                    included (query_len <= seq_len)
 *   num_seqs S >= 0, num_tokens T >= 0 (must equal sum(query_lens))
 *   block_tables [S, max_blocks_per_seq], -1 padded; may be NULL, then
 *                    slot_mapping is not written and the table is not checked
 *   block_size >= 1, num_blocks >= 1 (only read when block_tables != NULL)
 * Outputs:
 *   query_start_loc [S+1]  0, running sum of query_lens, total last
 *   seq_start_loc   [S+1]  same over seq_lens
 *   positions       [T]    row i of sequence s: seq_lens[s] - query_lens[s] + i
 *   token_to_seq    [T]    s
 *   slot_mapping    [T]    (nullable) physical slot of each new token, -1 when
 *                          its block-table entry is invalid (PA_DERR_BLOCK_OOB)
 *   stats           [6]    (nullable) num_decodes (query_len == 1),
 *                          num_prefills (query_len > 1), num_decode_tokens,
 *                          num_prefill_tokens, max_query_len, max_seq_len
 * Device checks: PA_DERR_QLEN_GT_SEQLEN, PA_DERR_TOKEN_SUM, PA_DERR_OVERFLOW,
 * and (with a table) PA_DERR_BLOCK_OOB for every entry in each sequence's
 * used range [0, ceil(seq_len / block_size)).
 */
pa_status_t pa_build_metadata(const int32_t* query_lens, const int32_t* seq_lens, int32_t num_seqs,
                              int32_t num_tokens, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                              int32_t* query_start_loc, int32_t* seq_start_loc, int32_t* positions,
                              int32_t* token_to_seq, int32_t* slot_mapping, int32_t* stats,
                              int32_t* d_err, void* stream);

/*
 * pa_write_kv — scatter this step's new K/V rows into the paged cache.
 *
 * [FS] §2.3 第一步 (slot_mapping says where each new token's K/V goes;
 * written before attention), [VP] §3.7 (store_kvcache(k, v, k_cache,
 * v_cache, slot_mapping) runs first in Attention.forward).
 *
 *   k, v        [T, num_kv_heads, head_dim]  new rows, `dtype`
 *   slot_mapping [T]  slot of row t; negative = skip the row
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim], `dtype`;
 *               slot s is block s / block_size, offset s % block_size
 * A pure copy: stored bits are moved unchanged; the caches are never read.
 * Slots >= num_blocks * block_size are skipped and flag PA_DERR_SLOT_OOB.
 * Two rows with the same non-negative slot are invalid input (the copy-on-
 * write rule of [VP] §2.1 keeps writers apart); which row wins is unspecified,
 * and with validation on (pa_set_validation) the call flags PA_DERR_DUP_SLOT.
 */
pa_status_t pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                        int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                        int32_t num_blocks, int32_t block_size, pa_dtype_t dtype, int32_t* d_err,
                        void* stream);

/*
 * pa_copy_blocks — copy whole KV blocks by (source, destination) pairs.
 *
 * The device half of copy-on-write ([VP] §2.1: before a block shared by
 * several sequences (ref_count > 1) is written, the writer gets a fresh block
 * holding a copy, and its table is repointed) and of swapping ([CB] §4.4:
 * blocks move to CPU memory under memory pressure and back later).
 *
 *   src_k, src_v  [src_num_blocks, block_size, Hkv, D] source pool (K and V)
 *   dst_k, dst_v  [dst_num_blocks, block_size, Hkv, D] destination pool; may
 *                 be the same pool as the source (copy-on-write)
 *   pairs         [num_pairs, 2] int32 (source block, destination block),
 *                 device-accessible memory
 *   block_bytes   bytes of one block of one of K/V (block_size*Hkv*D*esize),
 *                 a multiple of 16
 * Any pool may live in device memory or in pinned host memory the device can
 * access (for swap-out / swap-in).  A pure copy of bits.  Pairs with a block
 * id out of range are skipped and flag PA_DERR_BLOCK_OOB.  A destination
 * written twice, or a block that is both a destination and a source of the
 * same call, is invalid input (order unspecified).
 */
pa_status_t pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                           int32_t src_num_blocks, int32_t dst_num_blocks, const int32_t* pairs,
                           int32_t num_pairs, int64_t block_bytes, int32_t* d_err, void* stream);

/*
 * Bytes of device workspace pa_attention needs for these sizes and hints
 * (split-K partial results, shared-prefix partial results and the call's
 * work plan).  Depends only on its arguments; pass the same max_query_len and
 * max_seq_len as to pa_attention.  0 when such a call needs none.
 */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                   int32_t max_seq_len);

/*
 * pa_attention — ragged causal paged attention over the cache.
 *
 * [FS] §2.3 and §2.3补充 第二步: each sequence s takes its rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 of the flat batch and reads its
 * own K/V through block_tables[s]; row i sits at position
 * p = seq_lens[s] - query_len + i and sees positions 0..p of its own
 * sequence only.  [VP] §1.1: a decode row is the last row of softmax(QK^T)V.
 * For query head h the KV head is h / (num_q_heads / num_kv_heads).
 *
 *   out[t, h, :] = sum_{j<=p} e^{x_j - max x} V[j, g, :] / sum_{j<=p} e^{x_j - max x},
 *   x_j = scale * <q[t, h, :], K[j, g, :]>.
 *
 *   q    [T, num_q_heads, head_dim], `dtype`
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim], `dtype`
 *        (already holding this step's rows: write first, then attend)
 *   block_tables [S, max_blocks_per_seq], -1 padded; only the first
 *        ceil(seq_len / block_size) entries of a row are read
 *   query_start_loc [S+1], seq_lens [S]
 *   max_query_len, max_seq_len: host-side size hints used to shape the
 *        launch (like max_seqlen_q / max_seqlen_k in [VP] §3.7); >= 1 when
 *        T > 0.  Results do not depend on them being tight.  max_query_len
 *        must bound every query_len: a longer one flags PA_DERR_HINT and
 *        that sequence's rows are unspecified (computed or zero).  A
 *        sequence longer than max_seq_len is computed correctly (its split
 *        parts just get longer).
 *   scale  softmax scale (1/sqrt(head_dim) in the usual model); any finite
 *        value.  A non-finite scale returns PA_ERR_VALUE.  The MFMA paths
 *        take scale > 0; a call with scale <= 0 runs on the generic kernel
 *        (PA_POLICY_FAST: PA_ERR_UNSUPPORTED).
 *   out  [T, num_q_heads, head_dim], `dtype`
 *   workspace: device memory of at least pa_attention_workspace_size() bytes;
 *        contents on entry are irrelevant, on exit unspecified.
 * Arithmetic is fp32 (inputs widened, products and sums in fp32), output
 * rounded to `dtype` (nearest-even).  Supported: num_q_heads % num_kv_heads
 * == 0, 1 <= head_dim <= 256, block_size >= 1.  bf16/fp16 with head_dim 64,
 * 128 or 256, a block_size that is a multiple of 16 or divides 16,
 * num_q_heads / num_kv_heads <= 16, scale > 0 and q, the caches, out and
 * workspace 16-byte aligned take the MFMA fast paths; everything else takes
 * a generic fp32 kernel.
 * The caches are never written.  Rows of sequences whose metadata is invalid
 * are written as zeros and flag PA_DERR_*.
 */
pa_status_t pa_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* query_start_loc,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_query_len, int32_t max_seq_len, float scale, pa_dtype_t dtype,
                         void* out, void* workspace, size_t workspace_bytes, int32_t* d_err,
                         void* stream);

/*
 * pa_write_kv_attention — pa_write_kv followed by pa_attention, in one call.
 *
 * [VP] §3.7: the attention layer's forward stores the step's new K/V into
 * the cache and then attends, as one operation; [FS] §2.3 第一步/第二步: the
 * write goes first.  This call does exactly that: its results (the caches
 * and out) are those of pa_write_kv(k, v, slot_mapping, num_tokens,
 * num_kv_heads, head_dim, k_cache, v_cache, num_blocks, block_size, dtype,
 * d_err, stream) followed by pa_attention(...) with the same arguments, bit
 * for bit.  The difference is only in scheduling: the attention call's
 * planning launch reads lengths and block tables, not the cache, so when the
 * call has one (prefill rows, or contexts long enough for shared prefixes)
 * the write runs in that launch as workgroups of its own, beside the
 * planning workgroup, and every kernel that reads the cache follows it on
 * `stream`.  Otherwise (no planning launch; k, v, the caches or the row size
 * not 16-byte aligned; validation on) the write is a launch of its own
 * before everything else on `stream`.
 *   k, v  [num_tokens, num_kv_heads, head_dim], `dtype`: the new rows
 *   slot_mapping [num_tokens]: as for pa_write_kv (from pa_build_metadata)
 *   every other argument: as for pa_attention (k_cache / v_cache are
 *        written, so they are not const here)
 * Errors: pa_write_kv's checks, then pa_attention's; nothing is enqueued
 * unless both pass.  With pa_set_validation on, the duplicate-slot check of
 * pa_write_kv runs too.
 */
pa_status_t pa_write_kv_attention(const void* k, const void* v, const int32_t* slot_mapping, const void* q,
                                  void* k_cache, void* v_cache, const int32_t* block_tables,
                                  const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_seq_len,
                                  float scale, pa_dtype_t dtype, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t* d_err, void* stream);

/*
 * pa_attention_noalloc — pa_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, meaning and results as pa_attention, without the
 * workspace: the library uses a static device array of
 * PA_NOALLOC_SCRATCH_BYTES instead (one per device, held from the library's
 * first use of that device until the process ends).  The call allocates and
 * frees nothing; its first call on a device looks the array's address up.
 *   - A call whose pa_attention_workspace_size() exceeds
 *     PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on one device shares that device's array, and nothing in it
 *     needs to start at any value.  Calls that overlap on one device (on
 *     different streams, or from several threads, without ordering between
 *     them) race on it: the caller must order them.
 *   - Every launch stays on `stream` (pa_attention may put a large mixed
 *     batch's prefill kernel on the library's side stream).
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status_t pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_query_len, int32_t max_seq_len, float scale,
                                 pa_dtype_t dtype, void* out, int32_t* d_err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
